// The chunked prefill's attention on v_mfma_f32_32x32x16_bf16 (mini-infer 17 "MLA Attention：从 KV Cache
// 压缩到矩阵吸收", MLA 的数学结构 and 版本 1; 踩坑记录 坑 2 causal mask): over the expanded rows
// [K_nope | k_pe | V] that the expansion kernel wrote, the new tokens attend causally, MHA-style,
//   out[i, h] = softmax_{t <= p_i}(scale (q_nope[i,h] . K_nope[t,h] + RoPE(q_pe[i,h], p_i) . k_pe_t)) V[t, h].
// Two kernels: the rotation of the queries' q_pe (prefill_qprep_kernel), then the attention
// (prefill_attn32_kernel), which reads q_nope as given and that rotated q_pe.  Built with MFMA results in
// VGPRs (the scores feed the softmax arithmetic); the P.V accumulators are pinned to the AGPRs by hand.
#include "prefill_common.h"

namespace mla {

namespace {

// RoPE(q_pe) of the chunk's rows at their positions, in fp64 with the decode's table, rounded to bf16 once
// (round to nearest even), unscaled; a position outside the table gives NaN.  The attention reads q_nope
// as given and applies the softmax scale to the scores.  Lane -> (row, head, granule of 8 values): eight
// (row, head) units per wave, so that a wave reads whole 128-byte runs of q_pe; kQpUnits units per
// workgroup, every load issued before the arithmetic.  Grid y = the sequence.
constexpr int kQpUnits = 128;
__global__ __launch_bounds__(256) void prefill_qprep_kernel(PrefillArgs a) {
  const int b = blockIdx.y;
  int c0;
  const int n = chunk_of(a, b, &c0);
  const int tid = threadIdx.x;
  const int gq = tid & 7;  // granule of q_pe: rope pairs 4 gq .. 4 gq + 3
  const int ctx = clamp_ctx(a.seq_lens[b], n, a.max_seq_len);
  const uint32_t nu = uint32_t(n) * uint32_t(a.H);
  constexpr int kIt = kQpUnits / 32;
  u32x4_t x[kIt];
  uint32_t uu[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    uu[it] = blockIdx.x * uint32_t(kQpUnits) + 32 * it + (tid >> 3);  // row in the chunk * H + head
    const int64_t off = (int64_t(c0) * a.H + (uu[it] < nu ? uu[it] : 0)) * QW + DN + 8 * gq;
    x[it] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q) + off);
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    if (uu[it] >= nu) break;
    const int pos = ctx - n + int(uu[it] / uint32_t(a.H));
    const bool ok = pos >= 0 && pos <= a.max_position;
    const double2* cs = a.rope + int64_t(ok ? pos : 0) * NPAIR + 4 * gq;
    u32x4_t y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // values 2 e, 2 e + 1 of the granule
      const double2 c = cs[e];
      const double x0 = __uint_as_float(x[it][e] << 16), x1 = __uint_as_float(x[it][e] & 0xffff0000u);
      const float y0 = ok ? float(x0 * c.x - x1 * c.y) : __builtin_nanf("");
      const float y1 = ok ? float(x0 * c.y + x1 * c.x) : __builtin_nanf("");
      y[e] = cvt_pk_bf16(y0, y1);
    }
    *reinterpret_cast<u32x4_t*>(a.qpe + (int64_t(c0) * a.H + uu[it]) * DR + 8 * gq) = y;
  }
}

// The attention on v_mfma_f32_32x32x16_bf16, one wave per SIMD.  A workgroup of four waves takes 256
// query rows of one (sequence, head); wave w owns rows 64 w .. 64 w + 63 as two tiles of 32, so that every
// key and value operand read from LDS feeds two MFMAs.  The ring holds eight pairs of 32 tokens (160 KiB),
// moved six ahead.  Scores S^T[token][row] (the pair's 32 tokens on M, a tile's 32 rows on N, K = 192 in
// 12 steps): lane (l32, hf) receives, for row l32 of the tile, tokens 8 i + 4 hf + e of the pair in
// register 4 i + e, so the softmax state is per lane and a row's other tokens are in lane l32 + 32
// (1 - hf): one exchange for the row maximum.  P.V as O^T[dim][row] = V^T[dim][token] P^T[token][row]
// (dims on M, rows on N, K = the pair's tokens in two steps): with the K index of step kk permuted to
// tokens 16 kk + 8 rd + 4 hf + e (rd = 0, 1), the B operand is exactly score registers 8 kk .. 8 kk + 7
// of the lane, as bf16, and the A operand two transposing reads of V.  The step of pair q: its score
// MFMAs, with the exponentials of pair q - 1, the reads of pair q - 1's V operands and the transfer of
// pair q + 6 issued between them; a barrier; pair q - 1's P.V MFMAs, with pair q's lane maxima, pair
// q - 1's row sums and the reads of pair q + 1's first key operands between them; the reference check.
constexpr int kA32Rows = 64;                   // query rows per wave
constexpr int kA32Tile = 4 * kA32Rows;         // per workgroup
constexpr int kA32Stages = 8;                  // 160 KiB
constexpr int kA32Ahead = kA32Stages - 2;      // pairs in flight ahead of the one computed
static_assert(kA32Stages * kPairBytes <= 160 * 1024, "ring");

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_attn32_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char ring_mem[kA32Stages * kPairBytes];

  // workgroup -> (sequence, head, query tile), as in the 16x16 kernel: pair bh on XCD bh % 8, each XCD
  // taking its query tiles longest first
  const int nqt = (a.max_q_len + kA32Tile - 1) / kA32Tile;
  const int nbh = a.batch * a.H;
  const int nbx = (nbh + 7) >> 3;
  const int j = int(blockIdx.x >> 3);
  const int bh = (j % nbx) * 8 + int(blockIdx.x & 7);
  if (bh >= nbh || j >= nbx * nqt) return;
  const int qt = nqt - 1 - j / nbx;
  const int h = bh % a.H;
  const int b = bh / a.H;
  int c0;
  const int n = chunk_of(a, b, &c0);
  const int r0 = qt * kA32Tile;
  if (r0 >= n) return;  // uniform per workgroup: before any barrier

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hf = lane >> 5;  // 32x32 MFMA lane: row / column l32, K half hf
  const int r16 = lane & 15, G = lane >> 4;   // transposing-read lane: 16-lane group G
  const int lrow = lane & 7, lgr = lane >> 3;
  const int ctx = clamp_ctx(a.seq_lens[b], n, a.max_seq_len);
  const int p0 = ctx - n;  // position of chunk row 0
  // the wave's rows: rw0 + 32 t + l32 for tile t; rows past the chunk compute row n - 1 and are not stored
  const int rw0 = r0 + kA32Rows * w;
  auto p_of = [&](int rw) { return p0 + (rw < n ? rw : n - 1); };
  const int p_wave = p_of(rw0 + kA32Rows - 1);  // last position among the wave's rows
  const int p_wmin = p_of(rw0);                 // first position among them
  const int p_wg = p_of(r0 + kA32Tile - 1);
  const int npair = p_wg / 32 + 1;  // key pairs 0 .. npair - 1 (32 tokens each) seen by the workgroup

  const char* kvb = reinterpret_cast<const char*>(a.kv + (int64_t(b) * a.H + h) * a.t_pad * kKV);
  const char* zero = static_cast<const char*>(a.zero_block);  // >= 640 zero bytes
  lds_char_t* const ring = (lds_char_t*)ring_mem;
  // transfer of pair q into stage q % kA32Stages: wave w moves tokens 32 q + 8 w .. + 7 (token group
  // w % 2 of sub-block w / 2), one chunk of 8 granules per group gq (groups 0..2 hold K, 3..4 V);
  // rows past the context read the zero block.  Every step issues one pair's transfers, also past the
  // last pair (npair and later: zeros into a stage no later pair uses), so that the count of transfers
  // issued after pair q is always the same and one wait fits every step.
  auto xfer_src = [&](int q) {
    const int t = 32 * q + 8 * w + lrow;
    return (q < npair && t < ctx ? kvb + int64_t(t) * kKVBytes : zero) + 16 * lgr;
  };
  auto xfer_dst = [&](int q) {
    return __builtin_amdgcn_readfirstlane(
        uint32_t(uintptr_t(ring + (q % kA32Stages) * kPairBytes + (w >> 1) * kSubBytes + 1024 * kGQ * (w & 1))));
  };
  auto issue = [&](int q) {
    const char* src = xfer_src(q);
    const uint32_t dst = xfer_dst(q);
#pragma unroll
    for (int gq = 0; gq < kGQ; ++gq) dma16(src + 128 * gq, dst + 1024 * gq);
  };
  auto stage = [&](int q) {
    uint32_t sa = uint32_t(uintptr_t(ring + (q % kA32Stages) * kPairBytes));
    asm volatile("" : "+v"(sa));
    return (const lds_char_t*)uintptr_t(sa);
  };

  // Per-lane LDS offsets in a stage (two 16-token sub-blocks of 2 x 5 chunks of 1 KiB; granule c of
  // token t at slot 8 (c % 8) + t % 8 of chunk (t / 8, c / 8)).
  //  * key operand of score step k (token l32, channels 16 k + 8 hf .. + 7 = granule 2 k + hf): sc_off + 256 k
  //  * transposing read of V for dimension tile dt (32 dims), token quartet 4 Q .. 4 Q + 3 of the pair, in
  //    16-lane group G: tokens 4 Q + r16 / 4, dims 32 dt + 16 (G % 2) + 4 (r16 % 4) .. + 3 read, dims
  //    32 dt + 16 (G % 2) + r16 received: tr_off + 512 dt + (Q / 4) kSubBytes + ((Q / 2) % 2) 1024 kGQ +
  //    64 (Q % 2), with Q = 4 kk + 2 rd + G / 2 for the two reads rd of K step kk (V starts at granule 24)
  const int sc_off = (l32 >> 4) * kSubBytes + 1024 * kGQ * ((l32 >> 3) & 1) + 16 * (l32 & 7) + 128 * hf;
  const int tr_off = 3072 + 256 * (G & 1) + 64 * (G >> 1) + 128 * ((r16 >> 1) & 1) + 16 * (r16 >> 2) + 8 * (r16 & 1);

  // O^T[dim][row] tiles, in the AGPRs: acc[t][dt] holds dims 32 dt + 8 i + 4 hf + e of row l32 of tile t in
  // register 4 i + e
  f32x16_t acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      acc[t][dt] = f32x16_t{};
      asm volatile("" : "+a"(acc[t][dt]));
    }
  // per row, in log2 units of the scaled scores (the MFMAs give the unscaled score s; its exponent is
  // scale * s - msub): the reference m (-inf before the row has one), the same as msub (0 before), the
  // row sum, and the threshold above which a lane's maximum asks for a new reference (-inf before the row
  // has one, else m + the slack); the reference moves only there
  float m[2] = {-INFINITY, -INFINITY}, msub[2] = {0.f, 0.f}, lsum[2] = {0.f, 0.f};
  float thr[2] = {-INFINITY, -INFINITY};

  // the first two pairs now, the rest of the first kA32Ahead after the query rows are in registers
  // (the compiler's wait for the query loads covers every transfer issued before them)
  for (int q = 0; q < 2; ++q) issue(q);

  // query rows in registers, the B operand of score step k (channels 16 k + 8 hf .. + 7) of tile t: q_nope
  // as given (k < 8), RoPE(q_pe) from the prep kernel (k >= 8); unscaled, in bf16
  u32x4_t qreg[2][12];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t rrow = int64_t(c0 + p_of(rw0 + 32 * t + l32) - p0) * a.H + h;
    const u32x4_t* qs = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q) + rrow * QW);
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.qpe + rrow * DR);
#pragma unroll
    for (int k = 0; k < 8; ++k) qreg[t][k] = qs[2 * k + hf];
#pragma unroll
    for (int k = 8; k < 12; ++k) qreg[t][k] = qp[2 * (k - 8) + hf];
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 12; ++k) asm volatile("" ::"v"(qreg[t][k]));
  for (int q = 2; q < kA32Ahead; ++q) issue(q);

  const int nq = p_wave / 32 + 1;  // pairs seen by the wave's rows (<= npair)
  f32x16_t sv[2];  // scores of the pending pair (masked)
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[t][e] = -INFINITY;
  u32x4_t kw[3];     // key operands: step k in kw[k % 3]
  u32x4_t vt[4][2];  // A operands of P.V: dimension tile dt, K step kk
  auto ld_key = [&](const lds_char_t* st, int k) { kw[k % 3] = *(const lds_u32x4_t*)(st + sc_off + 256 * k); };
  auto ld_vt = [&](const lds_char_t* st, int dt, int kk) {
    const lds_char_t* base = st + tr_off + 512 * dt + kk * kSubBytes;
    const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base));
    const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + 1024 * kGQ));
    const u32x2_t a0 = __builtin_bit_cast(u32x2_t, v0), a1 = __builtin_bit_cast(u32x2_t, v1);
    vt[dt][kk] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
  };
  // p = exp2(scale s - msub) of the pending pair for element pair j (tile j / 8, elements 2 (j % 8), + 1),
  // packed to bf16 into the B operand of its P.V step (exp2(-inf) = 0)
  auto exp_pair = [&](u32x4_t (&pb)[2][2], int j) {
    const int t = j >> 3, e = 2 * (j & 7);
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t][e], a.qscale, -msub[t]));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t][e + 1], a.qscale, -msub[t]));
    uint32_t x = cvt_pk_bf16(p0, p1);
    asm volatile("" : "+v"(x));  // computed here, in its slot (not sunk to the P.V that reads it)
    pb[t][e >> 3][(e & 7) >> 1] = x;
  };
  // First part of a step (its key steps 0..2 already read): the score MFMAs of pair st (both tiles: two chains fed by one key read), the
  // exponentials of the pending pair and the reads of its V operands (from vst), slot by slot, one score
  // K step per slot, pinned so that the VALU and LDS work issues between the MFMAs.
  // The transfer of pair xq is issued here too, one chunk in each of the first five slots, so that a
  // transfer held back by the memory pipeline stalls the wave between MFMAs.
  auto step_scores = [&](const lds_char_t* st, const lds_char_t* vst, f32x16_t (&sc)[2], u32x4_t (&pb)[2][2], int xq) {
    const char* xs = xfer_src(xq);
    const uint32_t xd = xfer_dst(xq);
#pragma unroll
    for (int k = 0; k < 12; ++k) {
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[t] = mfma32x32(kw[k % 3], qreg[t][k], k == 0 ? f32x16_t{} : sc[t]);
      if (k + 3 < 12) ld_key(st, k + 3);
      if (k < kGQ) dma16(xs + 128 * k, xd + 1024 * k);
      if (k < 4) {
        exp_pair(pb, 2 * k);
        exp_pair(pb, 2 * k + 1);
      } else {
        exp_pair(pb, k + 4);
        ld_vt(vst, (k - 4) >> 1, (k - 4) & 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // lane (l32, hf) holds the scores of tokens 8 i + 4 hf + e of the pair (register 4 i + e); the causal
  // mask of a diagonal pair (one not wholly visible to every row of the wave)
  auto mask = [&](f32x16_t (&sc)[2], int tpair) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int lim = p_of(rw0 + 32 * t + l32) - tpair - 4 * hf;  // token 8 i + 4 hf + e visible iff 8 i + e <= lim
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[t][4 * i + e] = 8 * i + e <= lim ? sc[t][4 * i + e] : -INFINITY;
    }
  };
  // Second part: the P.V MFMAs of the pending pair (one read of V feeds both tiles), with the lane maxima
  // of pair st's scores, the pending pair's row sums (the lane's half of the row's tokens) and the first
  // key reads of the next pair (stage nst) between them, slot by slot.
  auto step_pv = [&](const u32x4_t (&pb)[2][2], const f32x16_t (&sc)[2], float (&ml)[2], const lds_char_t* nst) {
    // operands written by VALU (the packed probabilities, any move that assembles a V operand) -> the
    // MFMAs that read them
    asm volatile("s_nop 4" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(vt[0][0]), "v"(vt[1][0]),
                 "v"(vt[2][0]), "v"(vt[3][0]), "v"(vt[0][1]), "v"(vt[1][1]), "v"(vt[2][1]), "v"(vt[3][1]));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = i >> 3, dt = (i >> 1) & 3, t = i & 1;
      mfma32x32_acc(acc[t][dt], vt[dt][kk], pb[t][kk]);
      if (i < 8) {
        const int tt = i >> 2, pp = i & 3;
        const f32x16_t& x = sc[tt];
        if (pp == 0) {
          ml[tt] = vmax3(vmax3(x[0], x[1], x[2]), x[3], x[4]);
        } else if (pp == 1) {
          ml[tt] = vmax3(vmax3(ml[tt], x[5], x[6]), x[7], x[8]);
        } else if (pp == 2) {
          ml[tt] = vmax3(vmax3(ml[tt], x[9], x[10]), x[11], x[12]);
        } else {
          ml[tt] = vmax(vmax3(ml[tt], x[13], x[14]), x[15]) * a.qscale;  // in log2 units
        }
      } else {
        const int j = i - 8, tt = j >> 2, k2 = (j >> 1) & 1, h2 = j & 1;
        lsum[tt] = add_pk_bf16(pb[tt][k2][2 * h2 + 1], add_pk_bf16(pb[tt][k2][2 * h2], lsum[tt]));
      }
      if (i >= 13) ld_key(nst, i - 13);  // the next step's first key operands
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P.V of the pending pair without new scores (its row sums as well)
  auto pv_only = [&](const lds_char_t* vst) {
    u32x4_t pb[2][2];
#pragma unroll
    for (int j = 0; j < 16; ++j) exp_pair(pb, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) ld_vt(vst, i >> 1, i & 1);
    asm volatile("s_nop 4" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(vt[0][0]), "v"(vt[1][0]),
                 "v"(vt[2][0]), "v"(vt[3][0]), "v"(vt[0][1]), "v"(vt[1][1]), "v"(vt[2][1]), "v"(vt[3][1]));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = i >> 3, dt = (i >> 1) & 3, t = i & 1;
      mfma32x32_acc(acc[t][dt], vt[dt][kk], pb[t][kk]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) lsum[t] = add_pk_bf16(pb[t][kk][r], lsum[t]);
  };
  // only the lane's own maximum is compared with the threshold; the row maximum is reduced across the
  // two halves only when some score passes it or the row has no reference yet (the reference, moved
  // only there, stays the same in the two lanes of a row).  Then pair st's scores become the pending ones.
  auto rebase = [&](const f32x16_t (&sc)[2], const float (&ml)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (__any(ml[t] > thr[t])) {
        const float mn = fmaxf(m[t], xor32_max(ml[t]));  // -inf: nothing visible yet
        if (mn != -INFINITY) {
          const float alpha = (m[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[t] - mn);
          lsum[t] *= alpha;
          mfma_drain();
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) acc_scale<f32x16_t, 16>(acc[t][dt], alpha);
          m[t] = mn;
          msub[t] = mn;
          thr[t] = mn + kMaxSlack;
        }
      }
      sv[t] = sc[t];
    }
  };
  // Barrier q + 1, in the middle of step q: pair q + 1 has landed (this wave's transfers of the
  // kA32Ahead - 1 pairs after it may still be out), then every wave's part of it has, and every wave has
  // read the values of pair q - 1 (the scores part of step q), so that the transfer of pair q + 7 (step
  // q + 1) may go into its stage.
  auto enter = [&]() {
    wait_vmcnt<(kA32Ahead - 1) * kGQ>();
    lds_barrier();
  };
  // The pairs the wave's rows see, in two loops: those visible to every row of the wave (no mask), then
  // the diagonal ones (masked per element); each loop body holds the accumulators' code once (at a
  // control-flow merge inside the loop the register allocator would copy the AGPR tiles).  Then the step
  // of pair nq (P.V of pair nq - 1 only), the later pairs (transfers and barriers only), and the last P.V
  // when the wave sees every pair.
  const int nfull = min(nq, max(0, (p_wmin + 1) / 32));  // pairs q with 32 q + 31 <= p_wmin
  enter();  // barrier 0: pair 0 has landed
#pragma unroll
  for (int k = 0; k < 3; ++k) ld_key(stage(0), k);
  int q = 0;
  for (; q < nfull; ++q) {
    f32x16_t sc[2];
    u32x4_t pb[2][2];
    float ml[2];
    // before pair 0 the pending scores are -inf: its P.V adds exact zeros times this pair's (finite)
    // values
    step_scores(stage(q), stage(q == 0 ? 0 : q - 1), sc, pb, q + kA32Ahead);
    enter();
    step_pv(pb, sc, ml, stage(q + 1));
    rebase(sc, ml);
  }
  for (; q < nq; ++q) {
    f32x16_t sc[2];
    u32x4_t pb[2][2];
    float ml[2];
    step_scores(stage(q), stage(q == 0 ? 0 : q - 1), sc, pb, q + kA32Ahead);
    enter();
    mask(sc, 32 * q);
    step_pv(pb, sc, ml, stage(q + 1));
    rebase(sc, ml);
  }
  // P.V of the wave's last pair: in the step of pair nq when there is one (its transfer and barrier go
  // on for the other waves), else after the loops; then the later steps' transfers and barriers
  if (q < npair) {
    issue(q + kA32Ahead);
    pv_only(stage(nq - 1));
    enter();
    for (++q; q < npair; ++q) {
      issue(q + kA32Ahead);
      enter();
    }
  } else {
    pv_only(stage(nq - 1));
  }
  wait_vmcnt<0>();  // no transfer into this workgroup's LDS outlives it

  // out = acc / l for the rows of the chunk; lane (l32, hf) holds dims 32 dt + 8 i + 4 hf .. + 3 of row l32
  mfma_drain();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float l = xor32_add(lsum[t]);
    const int rw = rw0 + 32 * t + l32;
    if (rw < n) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* o = static_cast<uint16_t*>(a.out) + (int64_t(c0 + rw) * a.H + h) * DV + 4 * hf;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x2_t*>(o + 32 * dt + 8 * i) =
              u32x2_t{cvt_pk_bf16(acc[t][dt][4 * i] * inv, acc[t][dt][4 * i + 1] * inv),
                      cvt_pk_bf16(acc[t][dt][4 * i + 2] * inv, acc[t][dt][4 * i + 3] * inv)};
    }
  }
}

}  // namespace

hipError_t launch_prefill_qprep(PrefillArgs a, hipStream_t s) {
  const int64_t per_seq = int64_t(a.max_q_len) * a.H;  // (row, head) units of the longest chunk
  const int64_t gx = (per_seq + kQpUnits - 1) / kQpUnits;
  if (per_seq >= (int64_t(1) << 31) || a.batch > 65535) return hipErrorInvalidValue;
  launch(prefill_qprep_kernel, dim3(unsigned(gx), unsigned(a.batch)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_attn32(PrefillArgs a, hipStream_t s) {
  const int64_t nbx = (int64_t(a.batch) * a.H + 7) / 8;
  const int64_t grid = 8 * nbx * ((a.max_q_len + kA32Tile - 1) / kA32Tile);
  if (grid > 0x7ffffff0) return hipErrorInvalidValue;
  a.units = int32_t(grid);
  launch(prefill_attn32_kernel, dim3(int(grid)), dim3(256), 0, s, a);  // 160 KiB of LDS: one workgroup per CU
  return hipGetLastError();
}

}  // namespace mla
