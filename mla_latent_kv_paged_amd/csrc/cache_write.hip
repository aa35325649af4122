// S1 -- latent cache write (vLLM learning book ch. 07 §2.2 steps 2-3 and §2.3; mini-infer 17
// 版本 1 kv_a split and 坑 3): per new token, the row [RMSNorm(c_kv) * gamma | RoPE(k_pe, pos)]
// is scattered to slot slot_mapping[j] of the paged cache [n_blocks, 16, 1, 576].
//
// One wavefront per token: lane l owns latent channels 8l..8l+7 and (for l < 32) RoPE pair l.
// The row is evaluated in fp64 and rounded once to the storage dtype, so in fp32 storage the
// result is the correctly rounded value of the exact expression.  The traffic is one row in and
// one row out per token (about 2.3 KB in bf16); the kernel is latency-bound at decode sizes.
#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ double load_f64(const uint16_t* p, int64_t i) { return double(bf16_to_f32(p[i])); }
__device__ __forceinline__ double load_f64(const float* p, int64_t i) { return double(p[i]); }
__device__ __forceinline__ void store_round(uint16_t* p, int64_t i, double v) { p[i] = f64_to_bf16(v); }
__device__ __forceinline__ void store_round(float* p, int64_t i, double v) { p[i] = float(v); }

template <typename T>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= a.T) return;
  // every load of the token is issued before any of them is inspected (one memory round trip)
  const T* c = static_cast<const T*>(a.c_kv) + int64_t(j) * a.c_stride;
  const T* k = static_cast<const T*>(a.k_pe) + int64_t(j) * a.k_stride;
  const int slot = a.slots[j];
  const int pos = a.positions[j];
  double x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = load_f64(c, lane * 8 + e);
  const double kx0 = load_f64(k, 2 * (lane & (NPAIR - 1)));
  const double kx1 = load_f64(k, 2 * (lane & (NPAIR - 1)) + 1);
  double gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] = a.gamma[lane * 8 + e];
  if (slot < 0 || int64_t(slot) >= a.num_slots) return;  // padding or out-of-pool slot: skipped
  T* dst = static_cast<T*>(a.cache) + int64_t(slot) * ROW;
  const bool pos_ok = pos >= 0 && pos <= a.max_position;
  const double2 cs = a.rope[int64_t(pos_ok ? pos : 0) * NPAIR + (lane & (NPAIR - 1))];

  // RMSNorm over the 512 latent channels (fp64): x / sqrt(mean(x^2) + eps) * gamma
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double denom = sqrt(ss / double(DC) + a.eps);
  const double nan = __builtin_nan("");
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double y = x[e] / denom * gm[e];
    store_round(dst, lane * 8 + e, pos_ok ? y : nan);
  }

  // RoPE on k_pe: pair i = (x[2i], x[2i+1]) rotated by pos * theta^(-2i/64)
  if (lane < NPAIR) {
    const double x0 = kx0, x1 = kx1;
    double y0 = nan, y1 = nan;
    if (pos_ok) {
      y0 = x0 * cs.x - x1 * cs.y;
      y1 = x0 * cs.y + x1 * cs.x;
    }
    store_round(dst, DC + 2 * lane, y0);
    store_round(dst, DC + 2 * lane + 1, y1);
  }
}

hipError_t launch_cache_write(bool bf16, const CacheWriteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int grid = (a.T + 3) / 4;
  if (bf16)
    cache_write_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else
    cache_write_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
