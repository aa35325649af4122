// Measurement kernels: the practical ceilings the decode kernel's latent-cache stream is judged
// against (not part of the compute path).
//
//  stream_read_kernel   a plain read of `bytes` contiguous bytes into registers, each workgroup a
//                       contiguous range read 32 KiB at a time (global_load_dwordx4 with the non-temporal
//                       hint, eight loads per lane in flight), one word per thread written so that the
//                       loads are kept: the device's streaming-read rate.
//  gather_dma_kernel    the 16-row bf16 decode kernel's data movement and nothing else: the same work
//                       units (sequence, split), the same XCD-contiguous unit order, two waves per
//                       workgroup striding over the split's blocks, each with a ring of three 18 KiB
//                       LDS stages fed by global_load_lds_dwordx4 (non-temporal) two blocks ahead, the same zero-block
//                       substitution for tokens past the context.  A block is "consumed" by one LDS read
//                       once it has landed.  No MFMA, no softmax, no partial store.
//  mfma_loop_kernel     the matrix cores' issue rate for one instruction shape: every wave runs
//                       independent chains of v_mfma_f32_16x16x32_bf16 (eight) or v_mfma_f32_32x32x16_bf16
//                       (four) on register operands, four waves per SIMD.  Its counters (MFMA busy cycles
//                       per active GPU cycle) define a fully issued matrix pipe for that shape, against
//                       which a kernel's counters are read.
#include "mla_internal.h"

namespace mla {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* src, int64_t n16, uint32_t* sink) {
  // workgroup g reads the contiguous range [g n16 / grid, (g+1) n16 / grid) of 16-byte granules, 32 KiB
  // per step (eight coalesced 4 KiB loads, all in flight)
  const int64_t lo = n16 * blockIdx.x / gridDim.x, hi = n16 * (blockIdx.x + 1) / gridDim.x;
  u32x4_t x = {0u, 0u, 0u, 0u};
  int64_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(src + i + k * 256);
#pragma unroll
    for (int k = 0; k < 8; ++k) x ^= v[k];
  }
  for (; i < hi; i += 256) x ^= __builtin_nontemporal_load(src + i);
  sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

namespace {
constexpr int kBlockBytes = BLK * ROW * 2;  // one paged block of bf16 rows
constexpr int kNS = 3;                      // ring stages per wave
constexpr int kChunks = kBlockBytes / 1024;

__device__ __forceinline__ void wait_blocks_g(int n) {
  if (n <= 0)
    wait_vmcnt<0>();
  else if (n == 1)
    wait_vmcnt<kChunks>();
  else
    wait_vmcnt<2 * kChunks>();
}
}  // namespace

__global__ __launch_bounds__(128) void gather_dma_kernel(DecodeArgs a, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char ring_mem[2 * kNS * kBlockBytes];
  const int per_xcd = (a.units + 7) >> 3;
  const int u = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (u >= a.units) return;
  const int j = (u / a.n_rt) % a.n_split;
  const int b = u / (a.n_rt * a.n_split);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 7, lgr = lane >> 3;
  const int kb0 = j * a.split_blocks;
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);
  lds_char_t* const ring = (lds_char_t*)ring_mem + w * (kNS * kBlockBytes);

  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;
  const int in_row = min(a.split_blocks, a.bt_stride - kb0) - w;
  const int nid = in_row > 0 ? (in_row + 1) / 2 : 0;
  const int phys_lo = lane < nid ? bt[kb0 + w + 2 * lane] : 0;
  const int phys_hi = lane + 64 < nid ? bt[kb0 + w + 2 * (lane + 64)] : 0;
  asm volatile("" ::"v"(phys_lo), "v"(phys_hi));
  auto phys_of = [&](int i) {
    return i < 64 ? __builtin_amdgcn_readlane(phys_lo, i & 63) : __builtin_amdgcn_readlane(phys_hi, i & 63);
  };
  const int nblk = (ctx + BLK - 1) / BLK;
  int kb1 = kb0 + a.split_blocks;
  if (kb1 > nblk) kb1 = nblk;
  const int span = kb1 - kb0 - w;
  const int nwb = span > 0 ? (span + 1) / 2 : 0;
  auto issue = [&](int i) {
    const int kb = kb0 + w + 2 * i;
    const int phys = phys_of(i);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(ring + (i % kNS) * kBlockBytes)));
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int trow = 8 * tg + lrow;
      const bool ok = unsigned(phys) < unsigned(a.num_blocks) && kb * BLK + trow < ctx;
      const char* src =
          (ok ? cache + (int64_t(phys) * BLK + trow) * (ROW * 2) : zero + trow * (ROW * 2)) + 16 * lgr;
#pragma unroll
      for (int gq = 0; gq < 9; ++gq) dma16_nt(src + 128 * gq, dst + 1024 * (9 * tg + gq));
    }
  };
  const int pre = nwb < kNS - 1 ? nwb : kNS - 1;
  for (int i = 0; i < pre; ++i) issue(i);
  uint32_t x = 0;
  for (int i = 0; i < nwb; ++i) {
    if (i + kNS - 1 < nwb) issue(i + kNS - 1);
    const int ahead = nwb - 1 - i < kNS - 1 ? nwb - 1 - i : kNS - 1;
    wait_blocks_g(ahead);
    asm volatile("" ::: "memory");
    x ^= *(const __attribute__((address_space(3))) uint32_t*)(ring + (i % kNS) * kBlockBytes + 16 * lane);
    asm volatile("" ::: "memory");
  }
  wait_vmcnt<0>();
  sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = x;
}

// SHAPE 0: eight chains of v_mfma_f32_16x16x32_bf16; SHAPE 1: four chains of v_mfma_f32_32x32x16_bf16
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, uint32_t* sink) {
  // bf16 operands 1.0 and 2^-10: the sums stay small and finite for any iteration count used here
  u32x4_t a = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4_t b = {0x3a803a80u, 0x3a803a80u, 0x3a803a80u, 0x3a803a80u};
  asm volatile("" : "+v"(a), "+v"(b));
  float x = 0.f;
  if constexpr (SHAPE == 0) {
    f32x4_t acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma32v(a, b, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) x += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {
    f32x16_t acc[kMfmaChains / 2];
#pragma unroll
    for (int c = 0; c < kMfmaChains / 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kMfmaChains / 2; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                         acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kMfmaChains / 2; ++c) x += acc[c][0] + acc[c][15];
  }
  sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = __float_as_uint(x);
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t s) {
  launch(stream_read_kernel, dim3(grid), dim3(256), 0, s, static_cast<const u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_gather_dma(const DecodeArgs& a, uint32_t* sink, hipStream_t s) {
  const int grid = ((a.units + 7) >> 3) << 3;
  launch(gather_dma_kernel, dim3(grid), dim3(128), 0, s, a, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int shape, int iters, uint32_t* sink, int grid, hipStream_t s) {
  if (shape == 0)
    launch(mfma_loop_kernel<0>, dim3(grid), dim3(256), 0, s, iters, sink);
  else
    launch(mfma_loop_kernel<1>, dim3(grid), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace mla
