// S6/S7 -- split-KV combine and the W_uv output projection (mini-infer 17 "MLA Attention：从 KV
// Cache 压缩到矩阵吸收", 版本 3: the value up-projection is applied after attention).
// Split j of row (n, h) left (m_j, l_j, acc_j[512]) with m_j in log2 units; the exact softmax
// result is the log-sum-exp merge
//   o_lat = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j,   M = max_j m_j,
// and then out[n, h, :] = o_lat . W_uv[h]^T.  Splits are merged in index order: deterministic.
//
// One workgroup per (head, 16 query rows): merged o_lat rows are staged in LDS (32 KB) and the
// 512 x 128 W_uv[h] slab is streamed once per workgroup; fp32 accumulation, one rounding.
#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ float ldw(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ldw(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void sto(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void sto(float* p, int64_t i, float v) { p[i] = v; }

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
  __shared__ float olat[16][DC];

  for (int r = 0; r < 16; ++r) {
    const int row = r0 + r;
    if (row >= a.n_q) break;
    const int b = row / a.q_len;
    const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
    const int nblk = (ctx + BLK - 1) / BLK;
    int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
    if (ns > a.n_split) ns = a.n_split;
    const int64_t base = (int64_t(row) * a.H + h) * a.n_split;
    float M = -INFINITY;
    for (int j = 0; j < ns; ++j) M = fmaxf(M, a.part_ml[base + j].x);
    float den = 0.f, num0 = 0.f, num1 = 0.f;
    for (int j = 0; j < ns; ++j) {
      const float2 ml = a.part_ml[base + j];
      if (ml.x == -INFINITY) continue;
      const float wgt = exp2f(ml.x - M);
      den = fmaf(wgt, ml.y, den);
      const float* acc = a.part_acc + (base + j) * DC;
      num0 = fmaf(wgt, acc[tid], num0);
      num1 = fmaf(wgt, acc[tid + 256], num1);
    }
    olat[r][tid] = num0 / den;
    olat[r][tid + 256] = num1 / den;
  }
  __syncthreads();

  const T* wuv = static_cast<const T*>(a.W_uvT) + int64_t(h) * DC * DV;
  const int v = tid & (DV - 1);
  const int rh = (tid >> 7) * 8;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int c = 0; c < DC; ++c) {
    const float w = ldw(wuv, int64_t(c) * DV + v);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fmaf(olat[rh + i][c], w, o[i]);
  }
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + rh + i;
    if (row < a.n_q) sto(out, (int64_t(row) * a.H + h) * DV + v, o[i]);
  }
}

hipError_t launch_combine(bool bf16, const CombineArgs& a, hipStream_t s) {
  dim3 grid(a.H, (a.n_q + 15) / 16);
  if (bf16)
    combine_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else
    combine_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
