// S3-S6 in bf16 storage -- split-KV paged MLA decode on the CDNA4 matrix cores.
//
// What is computed (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收", 版本 3 and 设计取舍;
// 踩坑记录 坑 2 causal mask; vLLM learning book ch. 07 §2.3 paged cache shape; bxzpzcl.cn
// hybrid KV-cache page §2.1 block table): for one sequence b, one split of its context and one
// tile of 16 query rows r (16 heads of one query token),
//   s[r,t]  = [q_lat | q_pe'][r] . [c_t | k_pe_t]    (query pre-scaled by scale*log2 e)
//   masked for t > p (causal) and t >= ctx
//   m, l, acc[r, 0:512] = online-softmax state of sum_t 2^(s[r,t]-m) c_t
// and one (m, l, acc) partial per (row, split) is written for the combine pass.
//
// How (gfx950 specifics):
//  * A paged block is 16 tokens x 576 bf16 = 18,432 contiguous bytes.  Each lane of a wave loads
//    the 16-byte granules (token t = lane%16, granule 4s + lane/16), s = 0..17, straight into
//    registers: that is the A-operand layout of v_mfma_f32_16x16x32_bf16 with tokens on M, so the
//    scores S^T = C . Q^T come out of 18 MFMAs with no LDS traffic for C.  The K order inside an
//    MFMA is free as long as both operands use it; Q uses the same granule order.
//  * The query tile (16 rows x 576) sits in LDS, shared by the workgroup's waves (B operand).
//  * Score layout: lane l holds row r = l%16 and tokens 4(l/16)..+3, so the row max needs two
//    cross-lane steps and the softmax state stays per lane.
//  * P.C needs C transposed (the contraction runs over tokens).  The c_kv part of the block is
//    written to a per-wave LDS tile and read back with ds_read_b64_tr_b16, which yields the
//    A operand of v_mfma_f32_16x16x16_bf16 (512 channels on M in 32 tiles, tokens on K); P^T is
//    the B operand and is exactly the score registers converted to bf16.  The accumulator lands
//    with row r = lane%16 again, so the online-softmax rescale is lane-local.
//  * The waves of a workgroup stride over the split's blocks independently (no barrier in the
//    loop); at the end their states are merged in LDS in a fixed tree order (deterministic).
//  * Lanes whose token is past the visible range load nothing and hold zeros, and their scores
//    are selected to -inf, so stale or NaN slots never reach the arithmetic.
#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// swizzle of the per-wave C tile (16 rows of 64 granules): keeps both the granule writes
// (16 rows, same granule) and the transposed reads (8 rows x 2 granules per half-wave) spread
// over distinct bank groups.
__device__ __forceinline__ int ct_swz(int t) { return ((t & 7) << 1) | (t >> 3); }

template <int NW>
__global__ __launch_bounds__(NW * 64) void decode_bf16_kernel(DecodeArgs a) {
  __shared__ uint4 q_lds[16 * 72];
  __shared__ uint4 c_lds[NW * 16 * 64];
  __shared__ float m_lds[NW][16];
  __shared__ float l_lds[NW][16];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;

  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int rt = blockIdx.z;
  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int nblk = (ctx + BLK - 1) / BLK;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  if (j >= ns || j >= a.n_split) return;
  const int tiles_per_q = a.H >> 4;
  const int iq = rt / tiles_per_q;
  const int h0 = (rt % tiles_per_q) << 4;
  const int L = ctx - a.q_len + iq + 1;
  const int kb0 = j * a.split_blocks;
  int kb1 = kb0 + a.split_blocks;
  const int lblk = (L + BLK - 1) / BLK;
  if (kb1 > lblk) kb1 = lblk;
  const int row = b * a.q_len + iq;

  // query tile -> LDS, granule (r, c) at r*72 + (c ^ (r & 7))
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.qcat) +
                                                       (int64_t(row) * a.H + h0) * ROW);
    for (int idx = threadIdx.x; idx < 16 * 72; idx += NW * 64) {
      const int r = idx / 72, c = idx - r * 72;
      q_lds[r * 72 + (c ^ (r & 7))] = qsrc[idx];
    }
  }
  __syncthreads();

  f32x4_t acc[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) acc[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  uint4* cbuf = c_lds + w * 16 * 64;
  const char* cache = static_cast<const char*>(a.cache);
  const int wr_swz = ct_swz(r16);
  const int tr_t = 4 * g + (r16 >> 2);
  const int tr_swz = ct_swz(tr_t);
  const int tr_cofs = (r16 & 3) >> 1;
  const int tr_half = r16 & 1;
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;

  for (int kb = kb0 + w; kb < kb1; kb += NW) {
    const int phys = bt[kb];
    const bool blk_ok = unsigned(phys) < unsigned(a.num_blocks);
    const int tok = kb * BLK + r16;
    const bool ld_ok = blk_ok && tok < L;
    const uint4* src = reinterpret_cast<const uint4*>(cache + (int64_t(blk_ok ? phys : 0) * BLK + r16) * (ROW * 2));
    uint4 creg[18];
#pragma unroll
    for (int s = 0; s < 18; ++s) creg[s] = ld_ok ? src[4 * s + g] : make_uint4(0u, 0u, 0u, 0u);
    // c_kv part of the block -> per-wave LDS tile (row = token) for the transposed P.C operand
#pragma unroll
    for (int s = 0; s < 16; ++s) cbuf[r16 * 64 + ((4 * s + g) ^ wr_swz)] = creg[s];

    // scores: S^T[t][r] = sum_k C[t][k] * Q[r][k]
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      const int c = 4 * s + g;
      const uint4 qv = q_lds[r16 * 72 + (c ^ (r16 & 7))];
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(creg[s]), as_bf16x8(qv), sc, 0, 0, 0);
    }

    // mask + online softmax (row r16; this lane holds tokens 4g..4g+3 of the block)
    float sv[4];
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (kb * BLK + 4 * g + i < L) ? sc[i] : -INFINITY;
      mb = fmaxf(mb, sv[i]);
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mn = fmaxf(m, mb);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2f(sv[i] - mn);
    lsum = lsum * alpha + (p[0] + p[1]) + (p[2] + p[3]);
    m = mn;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) acc[jj] *= alpha;
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));

    // transposed reads of the c_kv tile written above
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const uint16_t* ap = reinterpret_cast<const uint16_t*>(cbuf + tr_t * 64 + ((2 * jj + tr_cofs) ^ tr_swz)) + tr_half * 4;
      const s16x4_t av = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(ap));
      acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb, acc[jj], 0, 0, 0);
    }
    asm volatile("" ::: "memory");
  }

  // merge the waves' states: row max, rescale, fixed-order tree sum through LDS
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (g == 0) {
    m_lds[w][r16] = m;
    l_lds[w][r16] = lsum;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, m_lds[ww][r16]);
  float Ltot = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float mw = m_lds[ww][r16];
    if (mw != -INFINITY) Ltot += exp2f(mw - M) * l_lds[ww][r16];
  }
  const float sw = (m == -INFINITY) ? 0.f : exp2f(m - M);
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) acc[jj] *= sw;

  float* slots = reinterpret_cast<float*>(c_lds);  // NW/2 slots of 16 x 512 floats
#pragma unroll
  for (int stride = NW / 2; stride >= 1; stride >>= 1) {
    if (w >= stride && w < 2 * stride) {
      float* sl = slots + (w - stride) * (16 * DC);
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) *reinterpret_cast<f32x4_t*>(sl + r16 * DC + 16 * jj + 4 * g) = acc[jj];
    }
    __syncthreads();
    if (w < stride) {
      const float* sl = slots + w * (16 * DC);
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) acc[jj] += *reinterpret_cast<const f32x4_t*>(sl + r16 * DC + 16 * jj + 4 * g);
    }
    __syncthreads();
  }

  if (w == 0) {
    const int64_t pidx = (int64_t(row) * a.H + h0 + r16) * a.n_split + j;
    float* dst = a.part_acc + pidx * DC;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) *reinterpret_cast<f32x4_t*>(dst + 16 * jj + 4 * g) = acc[jj];
    if (g == 0) a.part_ml[pidx] = make_float2(M, Ltot);
  }
}

hipError_t launch_decode(bool bf16, const DecodeArgs& a, int waves, hipStream_t s) {
  if (!bf16) return launch_decode_f32(a, s);
  dim3 grid(a.n_split, a.batch, (a.H / 16) * a.q_len);
  switch (waves) {
    case 4:
      decode_bf16_kernel<4><<<grid, 256, 0, s>>>(a);
      break;
    case 8:
      decode_bf16_kernel<8><<<grid, 512, 0, s>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
