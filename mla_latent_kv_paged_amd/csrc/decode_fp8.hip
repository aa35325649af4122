// S3-S6 over an FP8 latent cache -- split-KV paged MLA decode, 16 query rows per sequence and split.
//
// What is computed: the same as decode_bf16.hip (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收",
// 版本 3 and 设计取舍; 踩坑记录 坑 2 causal mask; vLLM learning book ch. 07 §2.3 paged cache shape;
// bxzpzcl.cn hybrid KV-cache page §2.1 block table), over cache rows that hold the normed latent
// as FP8 E4M3 codes in 4 groups of 128 channels with one fp32 scale per group (the vLLM learning
// book, ch. 07, lists an FP8 KV cache for MLA; the row layout and scale rule are this library's):
//   row (656 B) = [ 512 codes | 64 bf16 rope values | 4 fp32 scales ],  c_i = e4m3(code_i) * s_{i/128}
// Nothing is rounded on the way in: codes convert to bf16 exactly (e4m3 is a subset of bf16) and
// the scales are applied in fp32 to the MFMA results:
//   s[r,t] = sum_g s_{t,g} (q_lat[r, g] . code_t[g]) + q_pe'[r] . k_pe_t          (scores)
//   acc[r, g] += sum_t (P[r,t] s_{t,g}) code_t[g]                                  (P.C)
// with P[r,t] s_{t,g} rounded to bf16 as the MFMA operand, as P alone is in the bf16 kernel.
//
// How:
//  * A paged block is 16 rows of 656 bytes = 10,496 contiguous bytes.  Each wave streams its blocks
//    HBM -> LDS with global_load_lds_dwordx4 (11 transfers of 1 KB, the last one partly into padding)
//    into a private ring of NS stages, NS - 1 blocks ahead.  A 16-byte piece of a token past the
//    visible range is read from the zero block instead (rows are 41 pieces), so nothing stale or
//    NaN reaches the arithmetic.
//  * The codes are converted to bf16 in registers where they are consumed (exact), never staged:
//    - score MFMA k (v_mfma_f32_16x16x32_bf16, tokens on M): lane (t = l%16, g = l/16) reads the 8
//      codes of token t, channels 32k + 8g..+7, with one ds_read_b64 at a per-lane base + 32 k;
//    - P.C (v_mfma_f32_16x16x16_bf16): one ds_read_b64_tr_b8 gives lane i of group g the codes of
//      tokens 4g..4g+3 for channel 16p + i (lanes 0-7 of the group point at those tokens) and for
//      channel 16p + 64 + i (lanes 8-15 point 64 bytes further): the A operands of channel tiles
//      p and p + 4, both in the same scale group.  B = P^T times that group's scale, in bf16.
//    The rope part (bf16 as stored) is read with ds_read_b128 for the last two score MFMAs.
//  * Group scales: the four latent groups and the rope part accumulate separately; the lane's four
//    tokens' scales (one ds_read_b128 each) weigh the groups in fp32.
//  * NW waves (2 or 4) share one query tile and take every NW-th block of the split; at the end
//    they merge through LDS (each wave finalises 32 / NW channel tiles), then normalise and store
//    the fp16 partial rows as the bf16 kernel does.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kQTile = BLK * ROW * 2;            // bf16 query tile: 16 rows x 576
constexpr int kStage8 = 11 * 1024;               // fp8 stage: one block (10,496 B) + transfer padding
constexpr int kPieces = kFp8Row / 16;            // 41 sixteen-byte pieces per row
constexpr float kMaxSlack = 32.f;                // lazy-rescale slack (log2 units): P <= 2^32

typedef int int2v_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) int2v_t lds_i32x2_t;

__device__ __forceinline__ void wait_blocks8(int n) {  // at most n blocks (11 transfers each) in flight
  if (n <= 0)
    wait_vmcnt<0>();
  else if (n == 1)
    wait_vmcnt<11>();
  else if (n == 2)
    wait_vmcnt<22>();
  else
    wait_vmcnt<33>();
}

__device__ __forceinline__ s16x4_t codes4(uint32_t c) {
  return __builtin_bit_cast(s16x4_t, make_uint2(cvt2<false>(c), cvt2<true>(c)));
}

// P.C step on one accumulator tile pinned in AGPRs: with the builtin, the register allocator moves
// all 32 tiles through VGPRs once per block.  The compiler does not see an MFMA here, so the wait
// states are provided explicitly: s_nop 2 after the VALU that writes the A/B operands; a tile is
// used again 31 MFMAs later at the earliest; VALU access to the tiles follows mfma_drain().
__device__ __forceinline__ void mfma16_acc(f32x4_t& acc, s16x4_t a, s16x4_t b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_16x16x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// (mfma_drain, the wait states after the last asm MFMA before VALU touches its accumulator, is shared)

}  // namespace

template <int NW, int NS>
__global__ __launch_bounds__(NW * 64) void decode_fp8_kernel(DecodeArgs a) {
  static_assert(NW == 2 || NW == 4, "two or four waves share a query tile");
  static_assert(NS >= 2 && NS <= 4, "a wave keeps at most 3 blocks in flight");
  constexpr int TPW = 32 / NW;  // channel tiles each wave finalises
  static_assert(NW * NS * kStage8 >= NW * 32 * 1024, "the merge reuses the rings");
  __shared__ __attribute__((aligned(16))) char ring_mem[NW * NS * kStage8];
  __shared__ __attribute__((aligned(16))) char q_mem[kQTile];
  __shared__ float m_lds[NW][16];
  __shared__ float l_lds[NW][16];
  __shared__ float x_lds[NW][16];

  // work unit u = (sequence b, split j, row tile rt), rt fastest; contiguous unit ranges per XCD
  const int per_xcd = (a.units + 7) >> 3;
  const int u = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (u >= a.units) return;
  const int rt = u % a.n_rt;
  const int j = (u / a.n_rt) % a.n_split;
  const int b = u / (a.n_rt * a.n_split);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int lrow = lane & 7, lgr = lane >> 3;

  const int tiles_per_q = a.H >> 4;
  const int iq = rt / tiles_per_q;
  const int h0 = (rt % tiles_per_q) << 4;
  const int row = b * a.q_len + iq;
  const int kb0 = j * a.split_blocks;
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);  // >= 10,496 zero bytes
  lds_char_t* const ring = (lds_char_t*)ring_mem + w * (NS * kStage8);

  // start-up as in the bf16 kernel: context length, block ids and query tile requested together
  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;
  const int in_row = min(a.split_blocks, a.bt_stride - kb0) - w;
  const int nid = in_row > 0 ? (in_row + NW - 1) / NW : 0;
  const int phys_lo = lane < nid ? bt[kb0 + w + NW * lane] : 0;
  const int phys_hi = lane + 64 < nid ? bt[kb0 + w + NW * (lane + 64)] : 0;
  if (w < 2) {  // query tile -> LDS: wave w moves rows 8w..8w+7 (the bf16 kernel's stage layout)
    const char* src = static_cast<const char*>(a.qcat) + (int64_t(row) * a.H + h0 + 8 * w + lrow) * (ROW * 2) +
                      16 * lgr;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t((lds_char_t*)q_mem)));
#pragma unroll
    for (int gq = 0; gq < 9; ++gq) dma16(src + 128 * gq, dst + 1024 * (9 * w + gq));
  }
  asm volatile("" ::"v"(phys_lo), "v"(phys_hi));  // the ids are complete (see decode_bf16.hip)
  auto phys_of = [&](int i) {
    return i < 64 ? __builtin_amdgcn_readlane(phys_lo, i & 63) : __builtin_amdgcn_readlane(phys_hi, i & 63);
  };

  const int nblk = (ctx + BLK - 1) / BLK;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  if (j >= ns) {  // empty split: marked for the combine after the query transfer has landed
    if (w == 0 && lane < 16)
      a.part_ml[(int64_t(row) * a.H + h0 + lane) * a.n_split + j] = make_float2(-INFINITY, 0.f);
    wait_vmcnt<0>();
    return;
  }
  const int L = ctx - a.q_len + iq + 1;
  int kb1 = kb0 + a.split_blocks;
  const int lblk = (L + BLK - 1) / BLK;
  if (kb1 > lblk) kb1 = lblk;
  const int span = kb1 - kb0 - w;
  const int nwb = span > 0 ? (span + NW - 1) / NW : 0;

  // transfer of the wave's block i into ring stage i % NS: 16-byte piece pc of the block (token
  // pc / 41) comes from the zero block when that token is past the visible range or the block id
  // is out of range; 10 full kilobytes, then pieces 640..655 (lanes 16..63 fill stage padding)
  auto issue = [&](int i) {
    const int kb = kb0 + w + NW * i;
    const int phys = phys_of(i);
    const bool ok = unsigned(phys) < unsigned(a.num_blocks);
    const char* blk = cache + int64_t(ok ? phys : 0) * kFp8Block;
    int vis = (L - kb * BLK) * kPieces;
    vis = !ok ? 0 : vis > BLK * kPieces ? BLK * kPieces : vis;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(ring + (i % NS) * kStage8)));
    const int pc_last = lane < 16 ? 640 + lane : lane;
    if (vis == BLK * kPieces) {  // the common case: the whole block is visible
#pragma unroll
      for (int k = 0; k < 10; ++k) dma16_nt(blk + 16 * (64 * k + lane), dst + 1024 * k);
      dma16_nt(blk + 16 * pc_last, dst + 10240);
    } else {
#pragma unroll
      for (int k = 0; k < 10; ++k) {
        const int pc = 64 * k + lane;
        dma16_nt((pc < vis ? blk : zero) + 16 * pc, dst + 1024 * k);
      }
      dma16_nt((pc_last < vis ? blk : zero) + 16 * pc_last, dst + 10240);
    }
  };

  const int pre = nwb < NS - 1 ? nwb : NS - 1;
  for (int i = 0; i < pre; ++i) issue(i);
  wait_blocks8(pre);  // the query transfers precede the blocks'
  lds_barrier();

  u32x4_t qreg[18];  // B operand of score MFMA k: row r16, channels 32k + 8g .. + 7
  {
    const int q_off = 9216 * (r16 >> 3) + 128 * g + 16 * (r16 & 7);
    const lds_u32x4_t* qp = (const lds_u32x4_t*)((lds_char_t*)q_mem + q_off);
#pragma unroll
    for (int k = 0; k < 18; ++k) qreg[k] = qp[32 * k];
  }

  // per-lane offsets inside a stage
  const int s_off = kFp8Row * r16 + 8 * g;  // scores: token r16, codes 32k + 8g .. + 7
  const int r_off = kFp8Row * r16 + DC + 16 * g;  // rope: + 64 (k - 16)
  const int t_off = kFp8Row * (4 * g + ((lane >> 1) & 3)) + 8 * (lane & 1) + 64 * ((lane >> 3) & 1);  // P.C
  const int c_off = kFp8Row * (4 * g) + DC + 2 * DR;  // scales of tokens 4g .. 4g + 3

  f32x4_t acc[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) {
    acc[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    asm volatile("" : "+a"(acc[jj]));
  }
  float m = -INFINITY, lsum = 0.f;

  for (int i = 0; i < nwb; ++i) {
    if (i + NS - 1 < nwb) issue(i + NS - 1);
    const int ahead = nwb - 1 - i < NS - 1 ? nwb - 1 - i : NS - 1;
    wait_blocks8(ahead);
    asm volatile("" ::: "memory");
    const int kb = kb0 + w + NW * i;
    uint32_t sbase = uint32_t(uintptr_t(ring + (i % NS) * kStage8));
    asm volatile("" : "+v"(sbase));  // one base per block; the offsets stay per-lane constants
    lds_char_t* const st8 = (lds_char_t*)uintptr_t(sbase);

    // scores: latent groups G (MFMA k = 4G .. 4G+3) and the rope part (k = 16, 17) accumulate
    // apart; lane holds tokens 4g + t of row r16
    // MFMA n takes channels 32 k, k = 4 (n % 4) + n / 4: consecutive MFMAs feed different groups
    const u32x4_t rope0 = *(const lds_u32x4_t*)(st8 + r_off);
    const u32x4_t rope1 = *(const lds_u32x4_t*)(st8 + r_off + 64);
    constexpr int D = 4;
    auto kof = [](int n) { return 4 * (n & 3) + (n >> 2); };
    u32x2_t cg[D];
#pragma unroll
    for (int n = 0; n < D; ++n) cg[n] = *(const lds_u32x2_t*)(st8 + s_off + 32 * kof(n));
    f32x4_t scg[5];
#pragma unroll
    for (int G = 0; G < 5; ++G) scg[G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    scg[4] = mfma32v(rope0, qreg[16], scg[4]);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int k = kof(n);
      const u32x4_t x = codes8(cg[n % D]);
      if (n + D < 16) cg[n % D] = *(const lds_u32x2_t*)(st8 + s_off + 32 * kof(n + D));
      scg[k >> 2] = mfma32v(x, qreg[k], scg[k >> 2]);
      if (n == 7) scg[4] = mfma32v(rope1, qreg[17], scg[4]);
    }
    f32x4_t scl[4];  // group scales of tokens 4g + t (zero past the visible range, as their codes)
#pragma unroll
    for (int t = 0; t < 4; ++t) scl[t] = *(const __attribute__((address_space(3))) f32x4_t*)(st8 + c_off + kFp8Row * t);
    float sv[4];
    float ml = -INFINITY;  // this lane's max; m is the same in the four lanes of a row
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float s = scg[4][t];
#pragma unroll
      for (int G = 0; G < 4; ++G) s = fmaf(scl[t][G], scg[G][t], s);
      sv[t] = (kb * BLK + 4 * g + t < L) ? s : -INFINITY;
      ml = fmaxf(ml, sv[t]);
    }
    if (__any(ml > m + kMaxSlack)) {  // rare: a score rose by more than the slack above m
      const float mb = xor32_max(xor16_max(ml));
      const float mn = fmaxf(m, mb);
      if (!__all(m == -INFINITY)) {  // something accumulated: rescale it to the new reference
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        lsum *= alpha;
        mfma_drain();
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) acc_scale<f32x4_t, 4>(acc[jj], alpha);
      }
      m = mn;
    }
    float p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) p[t] = sv[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[t] - m);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    s16x4_t pb[4];  // B operand: P of the lane's tokens times their group-G scale
#pragma unroll
    for (int G = 0; G < 4; ++G)
      pb[G] = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0] * scl[0][G], p[1] * scl[1][G]),
                                                     cvt_pk_bf16(p[2] * scl[2][G], p[3] * scl[3][G])));

    // P.C: read q (q = 0..15) covers channel tiles p = 8 (q / 4) + q % 4 and p + 4 (group q / 4)
    constexpr int DT = 4;
    int2v_t tv[DT];
    auto tread = [&](int q) {
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(st8 + t_off + 128 * (q >> 2) + 16 * (q & 3)));
    };
#pragma unroll
    for (int q = 0; q < DT; ++q) tv[q] = tread(q);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int2v_t v = tv[q % DT];
      if (q + DT < 16) tv[q % DT] = tread(q + DT);
      const int pt = 8 * (q >> 2) + (q & 3);
      mfma16_acc(acc[pt], codes4(uint32_t(v[0])), pb[q >> 2]);
      mfma16_acc(acc[pt + 4], codes4(uint32_t(v[1])), pb[q >> 2]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage reads done before its reuse
  }

  // merge of the waves: every wave leaves its 32 tiles in the rings, wave w sums tiles
  // TPW w .. TPW w + TPW - 1 over the waves in wave order
  mfma_drain();
  lsum = xor32_add(xor16_add(lsum));
  if (g == 0) {
    m_lds[w][r16] = m;
    l_lds[w][r16] = lsum;
  }
  __syncthreads();  // every wave's transfers have landed, the rings are free
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
  f32x4_t* slots = reinterpret_cast<f32x4_t*>(ring_mem);  // slot (wave, tile): 1 KB
#pragma unroll
  for (int t = 0; t < 32; ++t) slots[(w * 32 + t) * 64 + lane] = acc[t] * sw;
  __syncthreads();
  f32x4_t fin[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    fin[t] = slots[(TPW * w + t) * 64 + lane];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) fin[t] += slots[(ww * 32 + TPW * w + t) * 64 + lane];
  }
  float mx = 0.f;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(fin[t][e]));
  mx = xor32_max(xor16_max(mx));
  if (g == 0) x_lds[w][r16] = mx;
  __syncthreads();
  float rmx = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) rmx = fmaxf(rmx, x_lds[ww][r16]);
  const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
  const float down = fp16_fit_scale(rmx * inv);
  const float sc = inv * down;
  lds_char_t* const otile = (lds_char_t*)q_mem;  // 16 rows x 1 KB of fp16, granules swizzled by row
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const f32x4_t v = fin[t] * sc;
    const int G = 2 * (TPW * w + t) + (g >> 1);
    *(lds_u32x2_t*)(otile + r16 * 1024 + 16 * (G ^ r16) + 8 * (g & 1)) =
        u32x2_t{cvt_pk_f16(v[0], v[1]), cvt_pk_f16(v[2], v[3])};
  }
  __syncthreads();
  constexpr int RPW = 16 / NW;
#pragma unroll
  for (int r = RPW * w; r < RPW * w + RPW; ++r) {
    const int64_t pr = (int64_t(row) * a.H + h0 + r) * a.n_split + j;
    *reinterpret_cast<u32x4_t*>(a.part_o16 + pr * DC + 8 * lane) =
        *(const lds_u32x4_t*)(otile + r * 1024 + 16 * (lane ^ r));
  }
  if (w == 0 && g == 0) {
    const int64_t pidx = (int64_t(row) * a.H + h0 + r16) * a.n_split + j;
    a.part_ml[pidx] = make_float2(M, Ltot);
    a.part_scale[pidx] = 1.f / down;
  }
}

hipError_t launch_decode_fp8(const DecodeArgs& a, int waves, hipStream_t s) {
  const int grid = ((a.units + 7) >> 3) << 3;
  switch (waves) {
    case 2:
      launch(decode_fp8_kernel<2, 4>, dim3(grid), dim3(128), 0, s, a);
      break;
    case 4:
      launch(decode_fp8_kernel<4, 3>, dim3(grid), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
