// S2 -- query side of the absorbed decode (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收",
// 版本 3 and 设计取舍; vLLM learning book ch. 07 §2.4 Decoupled RoPE):
//   q_lat[n,h,:] = q_nope[n,h,:] . W_uk[h]            (W_uk folded into the query, DC values)
//   q_pe'[n,h,:] = RoPE(q_pe[n,h,:], p_n),  p_n = ctx_b - q_len + i  for row n = b*q_len + i
// Both are scaled by softmax_scale*log2(e) so that the decode kernel works in log2 units, and
// stored as one [q_lat | q_pe'] row of 576 values per (n, h) in the storage dtype.
//
// bf16 storage: a batched MFMA GEMM per head, computed transposed so that each lane stores four
// consecutive channels: q_lat^T[c, n] = sum_k W_uk^T[c, k] q_nope^T[k, n], K = 128 (4 steps of
// v_mfma_f32_16x16x32_bf16).  A workgroup owns 64 channels x 64 query rows of one head (each wave
// 16 channels); operands are read straight from global memory (16 B per lane per step).
// fp32 storage: one workgroup per (head, 16 query rows) on the vector ALUs, W_uk[h] streamed once
// per workgroup, each thread owning two latent columns.  Both accumulate in fp32.
#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }

// RoPE of q_pe for one (row, head, pair), fp64 then scaled and rounded once.
__device__ __forceinline__ void rope_q_pair(const QAbsorbArgs& a, int row, int h, int i, float x0f, float x1f,
                                            float* y0, float* y1) {
  const int b = row / a.q_len, iq = row % a.q_len;
  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int pos = ctx - a.q_len + iq;
  *y0 = __builtin_nanf("");
  *y1 = __builtin_nanf("");
  if (pos >= 0 && pos <= a.max_position) {
    const double2 cs = a.rope[int64_t(pos) * NPAIR + i];
    const double x0 = x0f, x1 = x1f;
    *y0 = float((x0 * cs.x - x1 * cs.y) * double(a.qscale));
    *y1 = float((x0 * cs.y + x1 * cs.x) * double(a.qscale));
  }
}

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
    float y0, y1;
    rope_q_pair(a, row, h, i, qp[r][2 * i], qp[r][2 * i + 1], &y0, &y1);
    T* o = qcat + (int64_t(row) * a.H + h) * ROW + DC;
    st(o, 2 * i, y0);
    st(o, 2 * i + 1, y1);
  }
}

__global__ __launch_bounds__(256) void q_absorb_bf16_kernel(QAbsorbArgs a) {
  const int h = blockIdx.x;
  const int c_blk = blockIdx.y;  // 64 channels
  const int n_blk = blockIdx.z;  // 64 query rows
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  uint16_t* qcat = static_cast<uint16_t*>(a.qcat);
  const int c0 = c_blk * 64 + w * 16;
  // A = W_uk^T rows c0..c0+15 (granule 4*ks + g of the 128-wide row)
  const uint4* wrow = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.W_ukT) +
                                                     (int64_t(h) * DC + c0 + r16) * DN);
  uint4 af[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) af[ks] = wrow[4 * ks + g];
  // all B-operand loads are issued up front and unconditionally (rows past n_q read row 0 and
  // are not stored), so that the 16 loads of a lane are in flight together
  uint4 bq[4][4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int n = n_blk * 64 + tt * 16 + r16;
    const uint4* qrow = reinterpret_cast<const uint4*>(q + (int64_t(n < a.n_q ? n : 0) * a.H + h) * QW);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bq[tt][ks] = qrow[4 * ks + g];
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma32(af[ks], bq[tt][ks], acc);
    // lane holds query row n (column), channels c0 + 4g .. +3 (rows)
    const int n = n_blk * 64 + tt * 16 + r16;
    if (n < a.n_q) {
      *reinterpret_cast<uint2*>(qcat + (int64_t(n) * a.H + h) * ROW + c0 + 4 * g) =
          make_uint2(cvt_pk_bf16(acc[0] * a.qscale, acc[1] * a.qscale), cvt_pk_bf16(acc[2] * a.qscale, acc[3] * a.qscale));
    }
  }
  // RoPE part: the 8 channel-block workgroups of this (head, 64 rows) each take 8 rows x 32 pairs,
  // one pair per thread, so that the two dependent loads (context length, rotation table) are paid
  // once per thread.
  {
    const int r = c_blk * 8 + (threadIdx.x >> 5), i = threadIdx.x & 31;
    const int n = n_blk * 64 + r;
    if (n < a.n_q) {
      const uint16_t* src = q + (int64_t(n) * a.H + h) * QW + DN;
      float y0, y1;
      rope_q_pair(a, n, h, i, bf16_to_f32(src[2 * i]), bf16_to_f32(src[2 * i + 1]), &y0, &y1);
      uint16_t* o = qcat + (int64_t(n) * a.H + h) * ROW + DC;
      *reinterpret_cast<uint32_t*>(o + 2 * i) = cvt_pk_bf16(y0, y1);
    }
  }
}

hipError_t launch_q_absorb(bool bf16, const QAbsorbArgs& a, hipStream_t s) {
  if (bf16) {
    dim3 grid(a.H, DC / 64, (a.n_q + 63) / 64);
    q_absorb_bf16_kernel<<<grid, 256, 0, s>>>(a);
  } else {
    dim3 grid(a.H, (a.n_q + 15) / 16);
    q_absorb_kernel<float><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
