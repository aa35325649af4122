// S1 -- latent cache write (vLLM learning book ch. 07 §2.2 steps 2-3 and §2.3; mini-infer 17
// 版本 1 kv_a split and 坑 3): per new token, the row [RMSNorm(c_kv) * gamma | RoPE(k_pe, pos)]
// is scattered to slot slot_mapping[j] of the paged cache [n_blocks, 16, 1, 576].
//
// One wavefront per token: lane l owns latent channels 8l..8l+7 and (for l < 32) RoPE pair l.
// The row is evaluated in fp64 and rounded once to the storage dtype, so in fp32 storage the
// result is the correctly rounded value of the exact expression.  The traffic is one row in and
// one row out per token (about 2.3 KB in bf16); the kernel is latency-bound at decode sizes.
#include "cache_write_impl.h"

namespace mla {

template <typename T>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  cache_write_token<T>(a, blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

__global__ __launch_bounds__(256) void cache_write_fp8_kernel(CacheWriteArgs a) {
  cache_write_fp8_token<uint16_t>(a, blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

hipError_t launch_cache_write_fp8(const CacheWriteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  launch(cache_write_fp8_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cache_write(bool bf16, const CacheWriteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int grid = (a.T + 3) / 4;
  if (bf16)
    launch(cache_write_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, a);
  else
    launch(cache_write_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
