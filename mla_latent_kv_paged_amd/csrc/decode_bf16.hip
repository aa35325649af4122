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

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// swizzle of the per-wave C tile (16 rows of 64 granules): keeps both the granule writes
// (16 rows, same granule) and the transposed reads (8 rows x 2 granules per half-wave) spread
// over distinct bank groups.
__device__ __forceinline__ int ct_swz(int t) { return ((t & 7) << 1) | (t >> 3); }

// Issue the loads of one paged block (16 tokens x 576 bf16) into registers: lane (t = lane%16,
// g = lane/16) takes granules 4s + g of token t's row, s = 0..17.  The loads are unconditional
// (no divergent branch, so the compiler can keep several blocks in flight): a lane whose token is
// not visible, whose block id is outside the pool, or whose wave has no block left (!have)
// reads the zero block instead.
__device__ __forceinline__ void load_block(uint4 (&buf)[18], const char* cache, const char* zero, int phys,
                                           bool have, int kb, int L, int num_blocks, int r16, int g) {
  const bool ld_ok = have && unsigned(phys) < unsigned(num_blocks) && (kb * BLK + r16) < L;
  const char* rowp = ld_ok ? cache + (int64_t(phys) * BLK + r16) * (ROW * 2) : zero + r16 * (ROW * 2);
  const uint4* src = reinterpret_cast<const uint4*>(rowp);
#pragma unroll
  for (int s = 0; s < 18; ++s) buf[s] = src[4 * s + g];
}

// Running-max slack of the online softmax (log2 units): the max used for the exponentials is
// only moved when a block's max exceeds it by more than this, so P <= 2^8 and the accumulator
// rescale (a multiply of all 128 accumulator registers) is skipped for most blocks.  The result
// is the same softmax; only the common factor carried in (acc, l) differs.
constexpr float kMaxSlack = 8.f;

template <int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void decode_bf16_kernel(DecodeArgs a) {
  __shared__ uint4 c_lds[NW * 16 * 64];
  __shared__ float m_lds[NW][16];
  __shared__ float l_lds[NW][16];

  // Work unit u = (sequence b, split j, row tile rt), rt fastest.  Workgroup i is dispatched to
  // XCD i % 8; each XCD gets a contiguous range of units so that the row tiles and neighbouring
  // splits of a sequence share one L2.
  const int per_xcd = (a.units + 7) >> 3;
  const int u = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (u >= a.units) return;
  const int rt = u % a.n_rt;
  const int j = (u / a.n_rt) % a.n_split;
  const int b = u / (a.n_rt * a.n_split);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r16 = lane & 15;
  const int g = lane >> 4;

  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int nblk = (ctx + BLK - 1) / BLK;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  if (j >= ns) return;
  const int tiles_per_q = a.H >> 4;
  const int iq = rt / tiles_per_q;
  const int h0 = (rt % tiles_per_q) << 4;
  const int L = ctx - a.q_len + iq + 1;
  const int kb0 = j * a.split_blocks;
  int kb1 = kb0 + a.split_blocks;
  const int lblk = (L + BLK - 1) / BLK;
  if (kb1 > lblk) kb1 = lblk;
  const int row = b * a.q_len + iq;

  // query tile in registers, in the B-operand layout of the score MFMA: lane (r, g) holds
  // granules 4e + g of query row r (head h0 + r), e = 0..17
  uint4 qreg[18];
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.qcat) +
                                                       (int64_t(row) * a.H + h0 + r16) * ROW);
#pragma unroll
    for (int e = 0; e < 18; ++e) qreg[e] = qsrc[4 * e + g];
  }

  f32x4_t acc[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) acc[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  uint4* cbuf = c_lds + w * 16 * 64;
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);
  // LDS addresses.  The swizzle only touches the low 4 bits of a granule index, so granule
  // 16*q + x of a row maps to 16*q + (x ^ swz): a few per-lane base pointers plus immediate
  // offsets cover every access.
  const int wr_swz = ct_swz(r16);
  uint4* wr_base[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) wr_base[e2] = cbuf + r16 * 64 + ((4 * e2 + g) ^ wr_swz);
  const int tr_t = 4 * g + (r16 >> 2);
  const int tr_swz = ct_swz(tr_t);
  const int tr_cofs = (r16 & 3) >> 1;
  const int tr_half = r16 & 1;
  const uint16_t* tr_base[8];
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8)
    tr_base[r8] = reinterpret_cast<const uint16_t*>(cbuf + tr_t * 64 + ((2 * r8 + tr_cofs) ^ tr_swz)) + tr_half * 4;
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;

  // this wave's blocks: kb0 + w + NW*i, i < nwb (nwb <= 128).  Lane l holds the physical ids of
  // the wave's blocks l and 64 + l, so each lookup is a register read (v_readlane), not a memory
  // round trip in front of the next loads.
  const int span = kb1 - kb0 - w;
  const int nwb = span > 0 ? (span + NW - 1) / NW : 0;
  const int phys_lo = lane < nwb ? bt[kb0 + w + NW * lane] : 0;
  const int phys_hi = lane + 64 < nwb ? bt[kb0 + w + NW * (lane + 64)] : 0;
  auto phys_of = [&](int i) {
    return i < 64 ? __builtin_amdgcn_readlane(phys_lo, i & 63) : __builtin_amdgcn_readlane(phys_hi, i & 63);
  };

  // NBUF (2 or 3) named register buffers processed in turn with no conditional in the loop body,
  // so that the loads of the others stay in flight while one is consumed.  A short tail is padded
  // with missing blocks (zero data, every token masked).
  uint4 bufA[18], bufB[18], bufC[18];
  load_block(bufA, cache, zero, phys_of(0), 0 < nwb, kb0 + w, L, a.num_blocks, r16, g);
  load_block(bufB, cache, zero, phys_of(1), 1 < nwb, kb0 + w + NW, L, a.num_blocks,
             r16, g);
  if (NBUF == 3)
    load_block(bufC, cache, zero, phys_of(2), 2 < nwb, kb0 + w + 2 * NW, L,
               a.num_blocks, r16, g);

  // One block: c_kv -> LDS tile, scores, refill of the buffer with block i + 2, online softmax,
  // P.C on the matrix cores.
  auto process = [&](uint4 (&buf)[18], int i) {
    const int kb = kb0 + w + NW * i;
    const bool have = i < nwb;
#pragma unroll
    for (int e = 0; e < 16; ++e) wr_base[e & 3][16 * (e >> 2)] = buf[e];

    // scores: S^T[t][r] = sum_k C[t][k] * Q[r][k], two independent MFMA chains
    f32x4_t sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 18; e += 2) {
      sc0 = mfma32(buf[e], qreg[e], sc0);
      sc1 = mfma32(buf[e + 1], qreg[e + 1], sc1);
    }
    const f32x4_t sc = sc0 + sc1;
    const int inext = i + NBUF;
    load_block(buf, cache, zero, phys_of(inext & 127), inext < nwb, kb0 + w + NW * inext,
               L, a.num_blocks, r16, g);

    // mask + online softmax (row r16; this lane holds tokens 4g..4g+3 of the block)
    float sv[4];
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sv[t] = (have && kb * BLK + 4 * g + t < L) ? sc[t] : -INFINITY;
      mb = fmaxf(mb, sv[t]);
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    // lazy rescale: wave-uniform branch taken only when some row's max grew past the slack
    if (__any(mb > m + kMaxSlack)) {
      const float mn = fmaxf(m, mb);
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) acc[jj] *= alpha;
      m = mn;
    }
    float p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) p[t] = sv[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[t] - m);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])));

    // P.C: A = C^T tile jj (16 channels x 16 tokens) by transposed LDS read, B = P^T
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q8 = 0; q8 < 4; ++q8) {
      s16x4_t av[8];
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8)  // tile 8*q8 + r8: + 16 granules per 8 tiles
        av[r8] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tr_base[r8] + 16 * 8 * q8));
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8)
        acc[8 * q8 + r8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[r8], pb, acc[8 * q8 + r8], 0, 0, 0);
    }
    asm volatile("" ::: "memory");
  };

  for (int i = 0; i < nwb; i += NBUF) {
    process(bufA, i);
    process(bufB, i + 1);
    if (NBUF == 3) process(bufC, i + 2);
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
    if (mw != -INFINITY) Ltot += __builtin_amdgcn_exp2f(mw - M) * l_lds[ww][r16];
  }
  const float sw = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) acc[jj] *= sw;

  // NW/2 slots of 32 x 64 lanes x 16 B; a lane's accumulator tile jj sits at [jj][lane], so
  // that consecutive lanes touch consecutive 16-byte words (no bank conflicts)
  f32x4_t* slots = reinterpret_cast<f32x4_t*>(c_lds);
#pragma unroll
  for (int stride = NW / 2; stride >= 1; stride >>= 1) {
    if (w >= stride && w < 2 * stride) {
      f32x4_t* sl = slots + (w - stride) * (32 * 64);
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) sl[jj * 64 + lane] = acc[jj];
    }
    __syncthreads();
    if (w < stride) {
      const f32x4_t* sl = slots + w * (32 * 64);
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) acc[jj] += sl[jj * 64 + lane];
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
  const int grid = ((a.units + 7) >> 3) << 3;
  switch (waves) {
    case 2:
      decode_bf16_kernel<2, 2><<<grid, 128, 0, s>>>(a);
      break;
    case 4:
      decode_bf16_kernel<4, 2><<<grid, 256, 0, s>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
