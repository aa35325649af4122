// S3-S6 in fp32 storage -- split-KV paged decode on the vector ALUs (no MFMA: the fp32 mode is
// the precision reference of the library, not its throughput path).
//   s_t = [q_lat | q_pe'] . [c_t | k_pe_t]          (query pre-scaled by scale*log2(e))
//   causal visibility t <= p (mini-infer 17 踩坑记录 坑 2), online softmax in log2 units,
//   acc = sum_t 2^(s_t - m) c_t, written as one (m, l, acc[512]) partial per split.
// Paged addressing: token t of sequence b lives in block block_table[b][t/16], slot t%16
// (bxzpzcl.cn hybrid KV-cache page §2.1; vLLM learning book ch. 07 §2.3 cache shape).
//
// Workgroup = one (split, sequence, query row, head) with 256 threads: for each 16-token block,
// 16 threads per token form the 576-wide dot product, then every thread updates two of the 512
// accumulator columns.  A block_table entry outside the pool reads as zeros.
#include "mla_internal.h"

namespace mla {

__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeArgs a) {
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int rr = blockIdx.z;  // iq * H + h
  const int iq = rr / a.H, h = rr % a.H;
  const int tid = threadIdx.x;
  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int nblk = (ctx + BLK - 1) / BLK;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  if (j >= ns || j >= a.n_split) return;
  const int L = ctx - a.q_len + iq + 1;  // tokens visible to this query
  const int kb0 = j * a.split_blocks;
  int kb1 = kb0 + a.split_blocks;
  const int lblk = (L + BLK - 1) / BLK;
  if (kb1 > lblk) kb1 = lblk;
  const int row = b * a.q_len + iq;

  __shared__ float q[ROW];
  __shared__ float sc[BLK];
  const float* qsrc = static_cast<const float*>(a.qcat) + (int64_t(row) * a.H + h) * ROW;
  for (int d = tid; d < ROW; d += 256) q[d] = qsrc[d];
  __syncthreads();

  const float* cache = static_cast<const float*>(a.cache);
  const int t = tid >> 4, u = tid & 15;
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int kb = kb0; kb < kb1; ++kb) {
    const int phys = a.block_table[int64_t(b) * a.bt_stride + kb];
    const bool blk_ok = phys >= 0 && phys < a.num_blocks;
    const float* blk = cache + int64_t(blk_ok ? phys : 0) * BLK * ROW;
    const int tok = kb * BLK + t;
    float part = 0.f;
    if (blk_ok && tok < L) {
      for (int d = u; d < ROW; d += 16) part = fmaf(q[d], blk[t * ROW + d], part);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) part += __shfl_xor(part, off, 16);
    if (u == 0) sc[t] = tok < L ? part : -INFINITY;
    __syncthreads();
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < BLK; ++i) mb = fmaxf(mb, sc[i]);
    const float mn = fmaxf(m, mb);
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - mn);
    float p[BLK];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      p[i] = sc[i] == -INFINITY ? 0.f : exp2f(sc[i] - mn);
      ps += p[i];
    }
    l = l * alpha + ps;
    acc0 *= alpha;
    acc1 *= alpha;
    if (blk_ok) {
#pragma unroll
      for (int i = 0; i < BLK; ++i) {
        if (kb * BLK + i < L) {
          acc0 = fmaf(p[i], blk[i * ROW + tid], acc0);
          acc1 = fmaf(p[i], blk[i * ROW + tid + 256], acc1);
        }
      }
    }
    m = mn;
    __syncthreads();
  }
  const int64_t pidx = (int64_t(row) * a.H + h) * a.n_split + j;
  if (tid == 0) a.part_ml[pidx] = make_float2(m, l);
  a.part_acc[pidx * DC + tid] = acc0;
  a.part_acc[pidx * DC + tid + 256] = acc1;
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.batch, a.q_len * a.H);
  launch(decode_f32_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
