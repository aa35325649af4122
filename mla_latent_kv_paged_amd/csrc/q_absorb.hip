// S2 -- query side of the absorbed decode (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收",
// 版本 3 and 设计取舍; vLLM learning book ch. 07 §2.4 Decoupled RoPE):
//   q_lat[n,h,:] = q_nope[n,h,:] . W_uk[h]            (W_uk folded into the query, DC values)
//   q_pe'[n,h,:] = RoPE(q_pe[n,h,:], p_n),  p_n = ctx_b - q_len + i  for row n = b*q_len + i
// Both are scaled by softmax_scale*log2(e) so that the decode kernel works in log2 units, and
// stored as one [q_lat | q_pe'] row of 576 values per (n, h) in the storage dtype.
//
// One workgroup per (head, 16 query rows): W_uk[h] (128 x 512) is streamed once per workgroup
// with each thread owning two latent columns; fp32 accumulation.
#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }

template <typename T>
__global__ __launch_bounds__(256) void q_absorb_kernel(QAbsorbArgs a) {
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
  const T* q = static_cast<const T*>(a.q);
  const T* wuk = static_cast<const T*>(a.W_uk) + int64_t(h) * DN * DC;
  T* qcat = static_cast<T*>(a.qcat);

  __shared__ float qn[16][DN];
  __shared__ float qp[16][DR];
  for (int idx = tid; idx < 16 * QW; idx += 256) {
    const int r = idx / QW, d = idx % QW;
    const int row = r0 + r;
    const float v = row < a.n_q ? ld(q, (int64_t(row) * a.H + h) * QW + d) : 0.f;
    if (d < DN)
      qn[r][d] = v;
    else
      qp[r][d - DN] = v;
  }
  __syncthreads();

  float acc0[16], acc1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  for (int n = 0; n < DN; ++n) {
    const float w0 = ld(wuk, int64_t(n) * DC + tid);
    const float w1 = ld(wuk, int64_t(n) * DC + tid + 256);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[r] = fmaf(qn[r][n], w0, acc0[r]);
      acc1[r] = fmaf(qn[r][n], w1, acc1[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + r;
    if (row < a.n_q) {
      T* o = qcat + (int64_t(row) * a.H + h) * ROW;
      st(o, tid, acc0[r] * a.qscale);
      st(o, tid + 256, acc1[r] * a.qscale);
    }
  }

  // RoPE on q_pe at the query position, evaluated in fp64 then scaled and rounded once.
  for (int idx = tid; idx < 16 * NPAIR; idx += 256) {
    const int r = idx / NPAIR, i = idx % NPAIR;
    const int row = r0 + r;
    if (row >= a.n_q) continue;
    const int b = row / a.q_len, iq = row % a.q_len;
    const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
    const int pos = ctx - a.q_len + iq;
    float y0 = __builtin_nanf(""), y1 = __builtin_nanf("");
    if (pos >= 0 && pos <= a.max_position) {
      const double2 cs = a.rope[int64_t(pos) * NPAIR + i];
      const double x0 = qp[r][2 * i], x1 = qp[r][2 * i + 1];
      y0 = float((x0 * cs.x - x1 * cs.y) * double(a.qscale));
      y1 = float((x0 * cs.y + x1 * cs.x) * double(a.qscale));
    }
    T* o = qcat + (int64_t(row) * a.H + h) * ROW + DC;
    st(o, 2 * i, y0);
    st(o, 2 * i + 1, y1);
  }
}

hipError_t launch_q_absorb(bool bf16, const QAbsorbArgs& a, hipStream_t s) {
  dim3 grid(a.H, (a.n_q + 15) / 16);
  if (bf16)
    q_absorb_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else
    q_absorb_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
