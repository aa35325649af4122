// The projections around the attention in one layer's decode step from hidden states
// (mla_layer_decode_step; vLLM learning book ch. 07 §2.2 wrapper forward and the DeepseekV3DecoderLayer
// listing; mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收", 版本 1: q_proj, kv_a_proj_with_mqa
// split at kv_lora_rank, o_proj):
//   x        = input_layernorm(hidden) = hidden / sqrt(mean(hidden^2) + eps) * gamma_in   (optional)
//   [q | c_kv | k_pe] = x [q_proj; kv_a_proj]^T        (H*192 + 576 outputs per token)
//   out      = attn [o_proj]^T (+ hidden, the residual)  (D outputs per token)
// Both are skinny GEMMs Y[M, N] = X[M, K] W[N, K]^T with M = the step's new tokens (1 to a few
// hundred) and the weights streamed once: bound by HBM on the weight bytes, not by the MFMAs.
//
// Above 16 tokens, proj_gemm_kernel splits K into chunks of 512 over workgroups, so that the X rows (the tokens, read by
// every output tile) come from L2 only once per (output tile of 64, chunk): each workgroup stages its X
// chunk in LDS and streams 64 W rows of the chunk, v_mfma_f32_16x16x32_bf16 with the outputs on M and
// the tokens on N.  Its fp32 partial tile goes to a workspace, and proj_reduce_kernel (the next launch)
// adds the chunks in chunk order and applies the epilogue: deterministic, and ordered by the kernel
// boundary (a reduction inside the GEMM by the last workgroup to arrive needed device-scope fences,
// each an L2 write-back and invalidate on this multi-XCD part, and took three times as long).  The
// input norm's gamma is folded into the weight rows when the layer is attached (layer_pack_kernel), and
// its 1/rms per token comes from the sums of squares of the same X chunks, so that x is never written
// out.
#include "mla_internal.h"

namespace mla {

namespace {
constexpr int kProjWaves = 8;  // proj_gemm_small_kernel: waves per workgroup, each owning K / 8
constexpr int kProjSteps = 4;  // proj_gemm_small_kernel: K steps of 32 per register batch
}  // namespace

// dst[r, k] = src[r, k] * gamma[k] rounded to bf16 (round to nearest even), or a plain copy without
// gamma: the weight rows of one projection as the layer step reads them
__global__ __launch_bounds__(256) void layer_pack_kernel(const uint16_t* src, const uint16_t* gamma, uint16_t* dst,
                                                         int64_t n, int K) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    const uint16_t v = src[i];
    dst[i] = gamma ? f32_to_bf16(bf16_to_f32(v) * bf16_to_f32(gamma[i % K])) : v;
  }
}

hipError_t launch_layer_pack(const void* src, const void* gamma, void* dst, int64_t rows, int K, hipStream_t s) {
  const int64_t n = rows * K;
  const int64_t grid = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  launch(layer_pack_kernel, dim3(int(grid)), dim3(256), 0, s, static_cast<const uint16_t*>(src),
         static_cast<const uint16_t*>(gamma), static_cast<uint16_t*>(dst), n, K);
  return hipGetLastError();
}

// Workgroup (n tile of 64 outputs, K chunk kc of 512, m tile of 16 MT tokens), four waves.  The X chunk
// [16 MT tokens x 512] moves into LDS once by DMA (one 1 KiB row per instruction; rows padded by 16 bytes
// so that the 16 rows an MFMA operand reads fall in distinct banks); wave w streams its own 16 W rows
// (16 loads of 16 bytes per lane, all in flight) and multiplies them against every token tile.  The
// partial tile goes to the workspace, and the workgroups of n tile 0 also write the chunk's per-token
// sums of squares; proj_reduce_kernel adds the chunks in chunk order.
template <int MT>
__global__ __launch_bounds__(256) void proj_gemm_kernel(ProjArgs a) {
  constexpr int kRowBytes = kProjChunk * 2 + 16;  // LDS row of the X chunk, padded
  __shared__ __attribute__((aligned(16))) char xs[16 * MT * kRowBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int ntile = int(blockIdx.x), kc = int(blockIdx.y), mtile = int(blockIdx.z);
  const int n0 = ntile * 64, k0 = kc * kProjChunk, m0 = mtile * 16 * MT;
  const int ks = a.K / kProjChunk;

  // X chunk -> LDS: wave w moves rows w, w + 4, ... (rows past M repeat row M - 1)
  {
    const uint32_t base = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t((lds_char_t*)xs)));
#pragma unroll
    for (int i = 0; i < 4 * MT; ++i) {
      const int r = 4 * i + w;
      if (r < 16 * MT) {
        const int m = m0 + r < a.M ? m0 + r : a.M - 1;
        dma16(a.X + int64_t(m) * a.x_stride + k0 + 8 * lane, base + uint32_t(r * kRowBytes));
      }
    }
  }
  // W rows n0 + 16 w + r16, K block g of each of the 16 steps of the chunk
  const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.W + int64_t(n0 + 16 * w + r16) * a.K + k0 + 8 * g);
  u32x4_t wr[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) wr[s] = wp[4 * s];
  // every load of this wave has landed (the W loads are needed right away; waiting for the X rows alone
  // would rely on the compiler keeping the W loads after the wait)
  wait_vmcnt<0>();
  lds_barrier();

  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4_t b = *(const lds_u32x4_t*)((lds_char_t*)xs + (16 * t + r16) * kRowBytes + 64 * s + 16 * g);
      acc[t] = mfma32v(wr[s], b, acc[t]);
    }

  // partial tile [64 tokens x 64 outputs] of this chunk: token m0 + 16 t + r16, outputs 16 w + 4 g .. + 3
  float* part = a.part + ((int64_t(mtile) * gridDim.x + ntile) * ks + kc) * (64 * 64);
#pragma unroll
  for (int t = 0; t < MT; ++t)
    *reinterpret_cast<f32x4_t*>(part + (16 * t + r16) * 64 + 16 * w + 4 * g) = acc[t];
  // sums of squares of the chunk's X rows (the input norm), by n tile 0: four threads per row, 128
  // values each
  if (a.norm && ntile == 0 && int(threadIdx.x) < 64 * MT) {
    const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const u32x4_t v = *(const lds_u32x4_t*)((lds_char_t*)xs + r * kRowBytes + 256 * q + 16 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xffff0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (q == 0) a.ss_part[(int64_t(mtile) * ks + kc) * 64 + r] = ss;
  }
}

// Up to 16 tokens (one column tile): workgroup = 16 outputs, its 8 waves splitting K eight ways, each
// wave issuing all the loads of its K range before the first MFMA (two register batches of 4 K steps,
// the second in flight while the first multiplies); the 8 partial tiles are summed through LDS in wave
// order, and the epilogue is applied in the same launch.  With so few tokens the X rows are a few KB and
// re-reading them per output tile costs nothing, while one launch fewer does.
__global__ __launch_bounds__(kProjWaves * 64) void proj_gemm_small_kernel(ProjArgs a) {
  constexpr int MT = 1;
  __shared__ f32x4_t red[kProjWaves][MT][64];
  __shared__ float ssr[kProjWaves][MT][16];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = int(blockIdx.x) * 16;
  const int m0 = int(blockIdx.y) * 16 * MT;
  const int kw = a.K / kProjWaves;  // a multiple of 32 * kProjSteps (the host checks K)
  const int kbeg = w * kw;

  // A operand: W row n0 + r16, K block g of each step; B operand of column tile t: X row
  // m0 + 16 t + r16 (rows past M read row M - 1 and are not stored), K block g
  const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.W + int64_t(n0 + r16) * a.K + kbeg + 8 * g);
  const u32x4_t* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + 16 * t + r16;
    xp[t] = reinterpret_cast<const u32x4_t*>(a.X + int64_t(m < a.M ? m : a.M - 1) * a.x_stride + kbeg + 8 * g);
  }
  f32x4_t acc[MT];
  float ss[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    ss[t] = 0.f;
  }

  u32x4_t a0[kProjSteps], b0[kProjSteps][MT], a1[kProjSteps], b1[kProjSteps][MT];
  // a batch: kProjSteps K steps of 32 from K offset kb of this wave's range (granules of 8 values)
  auto load = [&](u32x4_t (&av)[kProjSteps], u32x4_t (&bv)[kProjSteps][MT], int kb) {
#pragma unroll
    for (int s = 0; s < kProjSteps; ++s) {
      av[s] = wp[(kb + 32 * s) / 8];
#pragma unroll
      for (int t = 0; t < MT; ++t) bv[s][t] = xp[t][(kb + 32 * s) / 8];
    }
  };
  auto compute = [&](const u32x4_t (&av)[kProjSteps], const u32x4_t (&bv)[kProjSteps][MT]) {
#pragma unroll
    for (int s = 0; s < kProjSteps; ++s)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        acc[t] = mfma32v(av[s], bv[s][t], acc[t]);
        if (a.norm) {
          const u32x4_t v = bv[s][t];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xffff0000u);
            ss[t] = fmaf(lo, lo, ss[t]);
            ss[t] = fmaf(hi, hi, ss[t]);
          }
        }
      }
  };
  constexpr int kBatch = 32 * kProjSteps;
  load(a0, b0, 0);
  for (int kb = 0; kb < kw; kb += 2 * kBatch) {
    const bool second = kb + kBatch < kw;
    if (second) load(a1, b1, kb + kBatch);
    compute(a0, b0);
    if (kb + 2 * kBatch < kw) load(a0, b0, kb + 2 * kBatch);
    if (second) compute(a1, b1);
  }

  // the eight waves' partial tiles (and sums of squares) summed in wave order
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    red[w][t][lane] = acc[t];
    if (a.norm) {
      float v = ss[t];
      v = xor32_add(xor16_add(v));
      if (g == 0) ssr[w][t][r16] = v;
    }
  }
  __syncthreads();
  if (w >= MT) return;
  const int t = w;  // wave t finishes column tile t
  const int m = m0 + 16 * t + r16;
  if (m >= a.M) return;
  f32x4_t v = red[0][t][lane];
#pragma unroll
  for (int ww = 1; ww < kProjWaves; ++ww) v += red[ww][t][lane];
  if (a.norm) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kProjWaves; ++ww) s += ssr[ww][t][r16];
    v *= 1.f / sqrtf(s / float(a.K) + a.eps);
  }
  // lane holds outputs n0 + 4g .. +3 of token m
  const int n = n0 + 4 * g;
  if (a.mode == 0) {
    if (n < a.n_split)  // query values, bf16, [M, n_split]
      *reinterpret_cast<uint2*>(a.y0 + int64_t(m) * a.n_split + n) =
          make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
    else  // [c_kv | k_pe] rows, fp32, [M, N - n_split]
      *reinterpret_cast<f32x4_t*>(a.y1 + int64_t(m) * (a.N - a.n_split) + (n - a.n_split)) = v;
  } else {
    const int64_t o = int64_t(m) * a.N + n;
    if (a.R) {
      const uint2 r = *reinterpret_cast<const uint2*>(a.R + o);
      v[0] += bf16_to_f32(uint16_t(r.x & 0xffffu));
      v[1] += bf16_to_f32(uint16_t(r.x >> 16));
      v[2] += bf16_to_f32(uint16_t(r.y & 0xffffu));
      v[3] += bf16_to_f32(uint16_t(r.y >> 16));
    }
    *reinterpret_cast<uint2*>(a.out + o) = make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
  }
}

// Y[m, n .. n+3] = sum over the K chunks, in chunk order, of the partial tiles (times 1/rms of X row m
// with the input norm), then the epilogue: one thread per four outputs of one token.
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // [M, N / 4]
  const int nq = a.N / 4;
  if (i >= int64_t(a.M) * nq) return;
  const int m = int(i / nq), n = int(i % nq) * 4;
  const int ks = a.K / kProjChunk;
  const int mtile = m / 64, r = m % 64;
  const int ntiles = a.N / 64;
  const float* p = a.part + (int64_t(mtile) * ntiles + n / 64) * ks * (64 * 64) + r * 64 + n % 64;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
  for (int c = 1; c < ks; ++c) v += *reinterpret_cast<const f32x4_t*>(p + int64_t(c) * (64 * 64));
  if (a.norm) {
    const float* sp = a.ss_part + int64_t(mtile) * ks * 64 + r;
    float s2 = sp[0];
    for (int c = 1; c < ks; ++c) s2 += sp[c * 64];
    v *= 1.f / sqrtf(s2 / float(a.K) + a.eps);
  }
  if (a.mode == 0) {
    if (n < a.n_split)  // query values, bf16, [M, n_split]
      *reinterpret_cast<uint2*>(a.y0 + int64_t(m) * a.n_split + n) =
          make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
    else  // [c_kv | k_pe] rows, fp32, [M, N - n_split]
      *reinterpret_cast<f32x4_t*>(a.y1 + int64_t(m) * (a.N - a.n_split) + (n - a.n_split)) = v;
  } else {
    const int64_t o = int64_t(m) * a.N + n;
    if (a.R) {
      const uint2 rr = *reinterpret_cast<const uint2*>(a.R + o);
      v[0] += __uint_as_float(rr.x << 16);
      v[1] += __uint_as_float(rr.x & 0xffff0000u);
      v[2] += __uint_as_float(rr.y << 16);
      v[3] += __uint_as_float(rr.y & 0xffff0000u);
    }
    *reinterpret_cast<uint2*>(a.out + o) = make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
  }
}

hipError_t launch_proj_gemm(const ProjArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.N % 64 != 0 || a.K % kProjChunk != 0) return hipErrorInvalidValue;
  if (a.M <= 16) {
    if (a.K % (kProjWaves * 32 * kProjSteps) != 0) return hipErrorInvalidValue;
    launch(proj_gemm_small_kernel, dim3(a.N / 16), dim3(kProjWaves * 64), 0, s, a);
    return hipGetLastError();
  }
  launch(proj_gemm_kernel<4>, dim3(a.N / 64, a.K / kProjChunk, (a.M + 63) / 64), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = int64_t(a.M) * (a.N / 4);
  launch(proj_reduce_kernel, dim3(int((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
