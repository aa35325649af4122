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
// proj_gemm_kernel: a workgroup owns 16 outputs n (one MFMA row tile) and 16 MT tokens m (MT column
// tiles of v_mfma_f32_16x16x32_bf16); its 8 waves split K eight ways, each wave issuing all the loads
// of its K range before the first MFMA (two register batches of 4 K steps, the second in flight while
// the first multiplies), then the 8 partial tiles are summed through LDS in a fixed order
// (deterministic, no atomics).  Both operands come straight from global memory: the W rows once, the
// X rows (a few hundred KB) out of the L2.  The input norm's gamma is folded into the weight rows
// when the layer is attached (layer_pack_kernel), and its 1/rms per token comes from the sum of
// squares of the same X values the MFMAs read, so that x is never written out.
#include "mla_internal.h"

namespace mla {

namespace {
constexpr int kProjWaves = 8;  // waves per workgroup, each owning K / 8
constexpr int kProjSteps = 4;  // K steps of 32 per register batch
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
  layer_pack_kernel<<<int(grid), 256, 0, s>>>(static_cast<const uint16_t*>(src), static_cast<const uint16_t*>(gamma),
                                              static_cast<uint16_t*>(dst), n, K);
  return hipGetLastError();
}

template <int MT>
__global__ __launch_bounds__(kProjWaves * 64) void proj_gemm_kernel(ProjArgs a) {
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
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
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

hipError_t launch_proj_gemm(const ProjArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.N % 16 != 0 || a.K % (kProjWaves * 32 * kProjSteps) != 0) return hipErrorInvalidValue;
  if (a.M <= 16) {
    proj_gemm_kernel<1><<<dim3(a.N / 16, 1), kProjWaves * 64, 0, s>>>(a);
  } else {
    proj_gemm_kernel<4><<<dim3(a.N / 16, (a.M + 63) / 64), kProjWaves * 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
