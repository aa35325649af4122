// S3-S6 in bf16 storage -- split-KV paged MLA decode on the CDNA4 matrix cores, one tile of 16
// query rows per sequence and split.
//
// What is computed (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收", 版本 3 and 设计取舍;
// 踩坑记录 坑 2 causal mask; vLLM learning book ch. 07 §2.3 paged cache shape; bxzpzcl.cn
// hybrid KV-cache page §2.1 block table): for one sequence b, one split of its context and one
// tile of 16 query rows r (16 heads of one query token),
//   s[r,t]  = [q_lat | q_pe'][r] . [c_t | k_pe_t]    (query pre-scaled by scale*log2 e)
//   masked for t > p (causal) and t >= ctx
//   m, l, acc[r, 0:512] = online-softmax state of sum_t 2^(s[r,t]-m) c_t
// and one partial per (row, split) is written for the combine pass: (m, l) and o = acc / l in
// fp16 (a convex combination of cache values: |o| <= max |c|).
//
// How (gfx950 specifics):
//  * A paged block is 16 tokens x 576 bf16 = 18,432 contiguous bytes.  Each wave streams its
//    blocks straight from HBM into a private ring of NS LDS stages with global_load_lds_dwordx4
//    (no register staging), NS - 1 blocks ahead of the one it computes on.  The waves of a
//    workgroup stride over the split's blocks independently: no barrier in the loop.
//  * Stage layout: two 8 x 9 grids of 1 KB chunks.  Chunk K = 9 tg + gq holds tokens 8tg..8tg+7 x
//    granules 8gq..8gq+7 (granule = 8 channels), granule c of token t at slot 8 (c % 8) + t % 8.
//    Lane l of a transfer writes slot l and reads token 8tg + l % 8, granule 8gq + l / 8: eight
//    rows x 128 contiguous bytes, whole cache lines.  Lanes whose token is not visible read the
//    library's zero block instead, so stale or NaN data never reaches the arithmetic.
//  * The query tile (16 rows x 576, contiguous in qcat) arrives the same way, once per workgroup,
//    and each wave keeps it in registers as the B operand of the score MFMA.
//  * Scores S^T[16 tok x 16 rows] = C Q^T on v_mfma_f32_16x16x32_bf16: the A operand of MFMA k
//    (token l%16, granule 4k + l/16) is one ds_read_b128 at a per-lane base + 512 k.  Lane l then
//    holds row l%16 at tokens 4(l/16)..+3, so the softmax state stays per lane; the row max (two
//    lane-pair steps, v_permlane16_swap and v_permlane32_swap) is formed only when a lane's max passes
//    the slack.
//  * P.C on v_mfma_f32_16x16x16_bf16: A = C^T tile jj (16 channels x 16 tokens) from one
//    ds_read_b64_tr_b16 at a per-lane base + 256 jj; B = P^T is exactly the score registers
//    rounded to bf16.  The accumulator lands with row r = lane%16 again, so the online-softmax
//    rescale is lane-local.
//  * At the end the two waves' states are merged in LDS in a fixed order (deterministic), each
//    wave summing and writing half of the channels.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kBlockBytes = BLK * ROW * 2;  // one paged block (and one query tile) in bf16
constexpr int kChunksPerBlock = kBlockBytes / 1024;

// Running-max slack of the online softmax (log2 units): the max used for the exponentials is
// only moved when a block's max exceeds it by more than this, so P <= 2^8 and the accumulator
// rescale (a multiply of all 128 accumulator registers) is skipped for most blocks.  The result
// is the same softmax; only the common factor carried in (acc, l) differs.
constexpr float kMaxSlack = 8.f;

// wait until at most n of this wave's block transfers (kChunksPerBlock instructions each) are in
// flight; n <= 3
__device__ __forceinline__ void wait_blocks(int n) {
  if (n <= 0)
    wait_vmcnt<0>();
  else if (n == 1)
    wait_vmcnt<kChunksPerBlock>();
  else if (n == 2)
    wait_vmcnt<2 * kChunksPerBlock>();
  else
    wait_vmcnt<3 * kChunksPerBlock>();
}

}  // namespace

// NW waves per workgroup (2 or 4), NS ring stages per wave.  With four waves the query tile is moved
// into the last stage of the last wave's ring (read into registers before that stage first takes a
// block), which keeps the workgroup within the 160 KiB of LDS at two stages per wave.
template <int NW, int NS>
__global__ __launch_bounds__(NW * 64) void decode_bf16_kernel(DecodeArgs a) {
  static_assert(NW == 2 || NW == 4, "two or four waves");
  static_assert(NS >= 2 && NS <= 4, "a wave keeps at most 3 blocks in flight (vmcnt range)");
  static_assert(NW * NS * kBlockBytes >= NW * 32 * 64 * 16 + 16 * 1024, "the merge reuses the rings");
  constexpr bool kQInRing = NW > 2;
  constexpr int kTilesPerWave = 32 / NW;  // channel tiles each wave finishes in the merge
  constexpr int kRowsPerWave = 16 / NW;   // partial rows each wave stores
  __shared__ __attribute__((aligned(16))) char ring_mem[NW * NS * kBlockBytes];
  __shared__ __attribute__((aligned(16))) char q_mem[kQInRing ? 16 : kBlockBytes];
  __shared__ float m_lds[NW][16];
  __shared__ float l_lds[NW][16];
  __shared__ float x_lds[NW][16];

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
  const int lrow = lane & 7, lgr = lane >> 3;  // transfer lane: token row and granule in a chunk

  const int tiles_per_q = a.H >> 4;
  const int iq = rt / tiles_per_q;
  const int h0 = (rt % tiles_per_q) << 4;
  const int row = b * a.q_len + iq;
  const int kb0 = j * a.split_blocks;
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);
  lds_char_t* const ring = (lds_char_t*)ring_mem + w * (NS * kBlockBytes);

  // Start-up: the context length, the block ids and the query tile are requested together (none
  // depends on another), so the first blocks wait for one memory round trip before they are
  // requested, not two.  The ids are read before the context length is known: the wave's blocks
  // kb0 + w + NW*i of the split that lie inside the block-table row (which holds every block of
  // a context, so this covers the wave's visible blocks).  Lane l holds the ids of the wave's
  // blocks l and 64 + l (at most 128: the host caps the split at 128 blocks per wave).
  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;
  const int in_row = min(a.split_blocks, a.bt_stride - kb0) - w;
  const int nid = in_row > 0 ? (in_row + NW - 1) / NW : 0;
  const int phys_lo = lane < nid ? bt[kb0 + w + NW * lane] : 0;
  const int phys_hi = lane + 64 < nid ? bt[kb0 + w + NW * (lane + 64)] : 0;
  lds_char_t* const qbuf = kQInRing ? (lds_char_t*)ring_mem + (NW * NS - 1) * kBlockBytes : (lds_char_t*)q_mem;
  {  // query tile -> LDS: rows 8 (w % 2) .. + 7; two waves move all 9 chunks of 128 bytes of their
     // rows, four waves split them 5 + 4
    const int rh = w % 2;
    const int gq0 = NW == 2 ? 0 : (w < 2 ? 0 : 5), gq1 = NW == 2 ? 9 : (w < 2 ? 5 : 9);
    const char* src = static_cast<const char*>(a.qcat) + (int64_t(row) * a.H + h0 + 8 * rh + lrow) * (ROW * 2) +
                      16 * lgr;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(qbuf)));
#pragma unroll
    for (int gq = 0; gq < 9; ++gq)
      if (gq >= gq0 && gq < gq1) dma16(src + 128 * gq, dst + 1024 * (9 * rh + gq));
  }
  // the ids are complete here: the compiler's wait for them must not land inside the transfer
  // pipeline below (it cannot tell them from the transfers and would wait for all of them)
  asm volatile("" ::"v"(phys_lo), "v"(phys_hi));
  auto phys_of = [&](int i) {
    return i < 64 ? __builtin_amdgcn_readlane(phys_lo, i & 63) : __builtin_amdgcn_readlane(phys_hi, i & 63);
  };

  const int nblk = (ctx + BLK - 1) / BLK;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  if (j >= ns) {  // a split past a short context: marked empty for the combine (which reads every
                  // split without the context length), after the query transfer has landed
    if (w == 0 && lane < 16)
      a.part_ml[(int64_t(row) * a.H + h0 + lane) * a.n_split + j] = make_float2(-INFINITY, 0.f);
    wait_vmcnt<0>();
    return;
  }
  const int L = ctx - a.q_len + iq + 1;  // tokens visible to every row of the tile
  int kb1 = kb0 + a.split_blocks;
  const int lblk = (L + BLK - 1) / BLK;
  if (kb1 > lblk) kb1 = lblk;
  // this wave's blocks: kb0 + w + NW*i, i < nwb (nwb <= nid)
  const int span = kb1 - kb0 - w;
  const int nwb = span > 0 ? (span + NW - 1) / NW : 0;

  // transfer of the wave's block i into ring stage i % NS
  auto issue = [&](int i) {
    const int kb = kb0 + w + NW * i;
    const int phys = phys_of(i);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(ring + (i % NS) * kBlockBytes)));
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int trow = 8 * tg + lrow;
      const bool ok = unsigned(phys) < unsigned(a.num_blocks) && kb * BLK + trow < L;
      const char* src =
          (ok ? cache + (int64_t(phys) * BLK + trow) * (ROW * 2) : zero + trow * (ROW * 2)) + 16 * lgr;
#pragma unroll
      for (int gq = 0; gq < 9; ++gq) dma16_nt(src + 128 * gq, dst + 1024 * (9 * tg + gq));
    }
  };

  // the first NS - 1 blocks of the wave
  const int pre = nwb < NS - 1 ? nwb : NS - 1;
  for (int i = 0; i < pre; ++i) issue(i);
  wait_blocks(pre);  // the query transfers precede the blocks'
  lds_barrier();

  // per-lane LDS offsets.  Score operand k (token r16, granule 4k + g): sc_off + 512 k.
  // Transposed read of channel tile jj (tokens 4g + r16/4, channels 16 jj + 4 (r16 % 4)):
  // tr_off + 256 jj.
  const int sc_off = 9216 * (r16 >> 3) + 128 * g + 16 * (r16 & 7);
  const int tr_off = 9216 * (g >> 1) + 64 * (g & 1) + 128 * ((r16 >> 1) & 1) + 16 * (r16 >> 2) + 8 * (r16 & 1);

  // query tile in registers, in the B-operand layout of the score MFMA: granule 4k + g of row r16
  u32x4_t qreg[18];
  {
    const lds_u32x4_t* qp = (const lds_u32x4_t*)(qbuf + sc_off);
#pragma unroll
    for (int k = 0; k < 18; ++k) qreg[k] = qp[32 * k];
  }
  // the query tile's LDS is the last wave's last stage: every wave has read it before it takes a block
  if constexpr (kQInRing) lds_barrier();

  f32x4_t acc[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) acc[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  for (int i = 0; i < nwb; ++i) {
    // keep NS - 1 blocks in flight behind this one
    if (i + NS - 1 < nwb) issue(i + NS - 1);
    const int ahead = nwb - 1 - i < NS - 1 ? nwb - 1 - i : NS - 1;
    wait_blocks(ahead);
    asm volatile("" ::: "memory");
    const uint32_t stage = uint32_t(uintptr_t(ring + (i % NS) * kBlockBytes));

    // scores: S^T[t][r] = sum_k C[t][k] * Q[r][k], two independent MFMA chains, operand reads
    // kept D ahead
    uint32_t spa = stage + uint32_t(sc_off);
    asm volatile("" : "+v"(spa));  // one base per block: the offsets fold into the reads
    const lds_u32x4_t* sp = (const lds_u32x4_t*)uintptr_t(spa);
    constexpr int D = 4;
    u32x4_t rg[D];
#pragma unroll
    for (int k = 0; k < D; ++k) rg[k] = sp[32 * k];
    f32x4_t sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const u32x4_t x = rg[k % D];
      if (k + D < 18) rg[k % D] = sp[32 * (k + D)];
      if (k & 1)
        sc1 = mfma32v(x, qreg[k], sc1);
      else
        sc0 = mfma32v(x, qreg[k], sc0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
#pragma unroll
    for (int k = 0; k < 18 - D; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, D, 0);
    const f32x4_t sc = sc0 + sc1;

    // mask + online softmax (row r16; this lane holds tokens 4g..4g+3 of the block)
    const int kb = kb0 + w + NW * i;
    float sv[4];
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sv[t] = (kb * BLK + 4 * g + t < L) ? sc[t] : -INFINITY;
      mb = fmaxf(mb, sv[t]);
    }
    // lazy rescale: wave-uniform branch taken only when some row's max grew past the slack (some lane's
    // max did); the row maximum over the row's four lanes is formed only then
    if (__any(mb > m + kMaxSlack)) {
      const float mn = fmaxf(m, xor32_max(xor16_max(mb)));
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
    uint32_t tpa = stage + uint32_t(tr_off);
    asm volatile("" : "+v"(tpa));
    lds_char_t* tp = (lds_char_t*)uintptr_t(tpa);
    constexpr int DT = 8;
    s16x4_t tv[DT];
#pragma unroll
    for (int jj = 0; jj < DT; ++jj) tv[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tp + 256 * jj));
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const s16x4_t av = tv[jj % DT];
      if (jj + DT < 32)
        tv[jj % DT] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tp + 256 * (jj + DT)));
      acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb, acc[jj], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, DT, 0);
#pragma unroll
    for (int jj = 0; jj < 32 - DT; ++jj) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, DT, 0);
    asm volatile("" ::: "memory");  // this stage's reads stay before the next transfer into it
  }

  // merge the two waves' states: row max, rescale, fixed-order sum through LDS
  lsum = xor32_add(xor16_add(lsum));
  if (g == 0) {
    m_lds[w][r16] = m;
    l_lds[w][r16] = lsum;
  }
  __syncthreads();  // also: every wave's transfers have landed, the rings are free
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

  // Each wave finishes kTilesPerWave of the 32 channel tiles (wave w: tiles kTilesPerWave w ..): every
  // wave writes its scaled accumulator to LDS ([wave][tile][lane] x 16 B: consecutive lanes,
  // consecutive words), and each tile is summed over the waves in wave order (deterministic).
  f32x4_t* slots = reinterpret_cast<f32x4_t*>(ring_mem);
#pragma unroll
  for (int t = 0; t < 32; ++t) slots[(w * 32 + t) * 64 + lane] = acc[t];
  __syncthreads();
  f32x4_t fin[kTilesPerWave];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    fin[t] = slots[(0 * 32 + kTilesPerWave * w + t) * 64 + lane];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) fin[t] += slots[(ww * 32 + kTilesPerWave * w + t) * 64 + lane];
  }
  // The partial is stored normalised, o = acc / l, in fp16 (a convex combination of cache
  // values), divided by a power of two when the row's largest |o| would not fit fp16.  The row
  // spans every wave (lanes r16 + 16 g of each): max over the lane's values, its row's four
  // lanes, then the waves through LDS.
  float mx = 0.f;
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(fin[t][e]));
  mx = xor32_max(xor16_max(mx));
  if (g == 0) x_lds[w][r16] = mx;
  __syncthreads();
  const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
  float xmax = x_lds[0][r16];
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) xmax = fmaxf(xmax, x_lds[ww][r16]);
  const float down = fp16_fit_scale(xmax * inv);
  const float sc = inv * down;
  // through an LDS tile (16 rows x 1 KB after the exchange slots; granule G of row r at slot
  // G ^ r) so that each store instruction writes one whole 1 KB row
  lds_char_t* const otile = (lds_char_t*)ring_mem + NW * 32 * 64 * 16;
  auto put = [&](int jj, f32x4_t v) {  // channels 16 jj + 4 g .. + 3 of row r16: granule 2 jj + g / 2
    v *= sc;
    const int G = 2 * jj + (g >> 1);
    *(lds_u32x2_t*)(otile + r16 * 1024 + 16 * (G ^ r16) + 8 * (g & 1)) =
        u32x2_t{cvt_pk_f16(v[0], v[1]), cvt_pk_f16(v[2], v[3])};
  };
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) put(kTilesPerWave * w + t, fin[t]);
  __syncthreads();
  const int64_t pidx = (int64_t(row) * a.H + h0 + r16) * a.n_split + j;  // this lane's row (r16)
#pragma unroll
  for (int r = kRowsPerWave * w; r < kRowsPerWave * w + kRowsPerWave; ++r) {  // wave w's rows
    const int64_t pr = (int64_t(row) * a.H + h0 + r) * a.n_split + j;
    *reinterpret_cast<u32x4_t*>(a.part_o16 + pr * DC + 8 * lane) =
        *(const lds_u32x4_t*)(otile + r * 1024 + 16 * (lane ^ r));
  }
  if (w == 0 && g == 0) a.part_scale[pidx] = 1.f / down;
  if (w == 0 && g == 0) a.part_ml[pidx] = make_float2(M, Ltot);
}

hipError_t launch_decode(bool bf16, const DecodeArgs& a, int waves, hipStream_t s) {
  if (!bf16) return launch_decode_f32(a, s);
  const int grid = ((a.units + 7) >> 3) << 3;
  switch (waves) {
    case 2:
      launch(decode_bf16_kernel<2, 3>, dim3(grid), dim3(128), 0, s, a);
      break;
    case 4:
      launch(decode_bf16_kernel<4, 2>, dim3(grid), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
