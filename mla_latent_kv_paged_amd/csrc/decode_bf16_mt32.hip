// S3-S6 in bf16 storage for 32-row tiles (32 heads of one query, or 16 heads of two queries):
// the same computation as decode_bf16.hip (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收",
// 版本 3 and 设计取舍; 踩坑记录 坑 2 causal mask; vLLM learning book ch. 07 §2.3 paged cache shape;
// bxzpzcl.cn hybrid KV-cache page §2.1 block table), organised for many rows per sequence.
//
//  * A workgroup owns one (sequence, split) and T tiles of 32 rows; wave w owns tile w: its query
//    tile (registers), its (m, l) per row and acc[32 rows x 512] (the AGPR file), and writes its
//    own partial.
//  * A step covers 32 tokens (two paged blocks).  The workgroup moves the step's 36 KB straight from
//    HBM into one LDS stage with global_load_lds_dwordx4 (no register staging), NSTAGE - 1 steps
//    ahead; masked lanes read the library's zero block.  The block ids of a piece are staged in LDS.
//  * Stage layout: 8 x 8 tiles of 16-byte granules (8 channels).  Chunk K = 9 tg + gq (1 KB) holds
//    tokens 8tg..8tg+7 x granules 8gq..8gq+7, granule c of token t at slot 8 (c % 8) + t % 8.  Lane
//    l of a DMA instruction writes slot l and reads token 8tg + l % 8, granule 8gq + l / 8: eight
//    rows x 128 contiguous bytes, i.e. whole cache lines.  Both operand reads below are a per-lane
//    base plus immediate offsets (score operand k at + 256 k) and run at the LDS's full rate.
//  * Scores S^T[32 tok x 32 rows] = C Q^T on v_mfma_f32_32x32x16_bf16: A = chunk k as read, B = the
//    query tile's granules 2k, 2k+1.  Lane l then holds row l%32 at tokens 8(r/4) + 4(l/32) + r%4.
//  * Causal mask per row; softmax against a per-row reference max that moves only when a score
//    exceeds it by more than 64 (log2 units), exp2; P is at most 2^64, well inside bf16 and fp32.
//    When it moves, what was accumulated is rescaled to the new reference.
//  * P.C: acc^T[32 ch x 32 rows] += C^T[32 ch x 16 tok] P^T[16 tok x 32 rows], two K steps of 16
//    tokens per step.  The K order inside a step is {4h..4h+3, 8+4h..8+4h+3} for lane half h, which
//    is exactly the order in which the score registers hold P, so B is the score registers rounded
//    to bf16; A is two ds_read_b64_tr_b16 per MFMA.
#include "mla_internal.h"


namespace mla {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kReset = 64.f;    // reference-max headroom (log2 units): P <= 2^64
constexpr int kChunks = 36;       // 1 KB chunks per stage (72 granules x 32 tokens)
constexpr int kStageBytes = kChunks * 1024;
constexpr int kIdCap = 2048;      // block ids of one piece held in LDS (a range is <= kIdCap / 2 steps)

}  // namespace

template <int T, int NSTAGE>
__global__ __launch_bounds__(T * 64) void decode_bf16_mt32_kernel(DecodeArgs a) {
  constexpr int CPW = kChunks / T;  // DMA chunks per wave per step
  constexpr int RP = 32 * T;        // rows of a piece (one tile group)
  static_assert(kChunks % T == 0, "chunks split evenly over the waves");
  static_assert(NSTAGE >= 2, "a step is read while a later one is loaded");
  static_assert(T * 32 * 1024 <= NSTAGE * kStageBytes, "the partial tiles fit the stages");
  static_assert(kIdCap >= 2 * kMt32MaxSteps, "a workgroup's block ids fit the LDS table");
  __shared__ __attribute__((aligned(16))) char stage_mem[NSTAGE * kStageBytes];
  __shared__ int ids_lds[kIdCap];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_grp = a.n_rt / T;  // tile groups per sequence (n_rt = tiles of 32 rows)
  const int n_wg = a.units;

  // ---- balanced partition.  Stream (b, grp) = tile group grp of sequence b, L_b steps of two
  // blocks, preceded by kPieceCost units that stand for a piece's setup; streams are ordered
  // (b, grp) and the workgroups take equal contiguous ranges of the concatenated units.  A range
  // cuts streams into pieces; the piece of stream s in range g keeps its partial under
  // id g + s (unique: between consecutive pieces g or s grows), so the pieces of a stream have
  // consecutive ids.
  constexpr int c = kPieceCost;
  auto steps_of = [&](int b) {
    const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
    return (((ctx + BLK - 1) / BLK) + 1) >> 1;
  };
  int S = 0;  // total units (uniform)
  for (int c0 = 0; c0 < a.batch; c0 += 64) {
    int v = c0 + lane < a.batch ? steps_of(c0 + lane) + c : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    S += __builtin_amdgcn_readfirstlane(v);
  }
  S *= n_grp;
  const int W = (S + n_wg - 1) / n_wg;
  // range index of this workgroup: workgroup i runs on XCD i % 8, and each XCD takes a contiguous block of
  // ranges (when n_wg is a multiple of 8), so that the pieces of one stream, which cut consecutive ranges,
  // mostly share an L2: their query tile and block ids come from HBM once
  const int bid = int(blockIdx.x);
  const int gr = (n_wg & 7) == 0 ? (bid & 7) * (n_wg >> 3) + (bid >> 3) : bid;
  const int lo = gr * W;
  const int hi = min(lo + W, S);
  // the sequence holding unit lo: the last b whose streams start at or before lo; workgroup 0
  // also records each stream's first piece id and piece count for the combine
  int bstar = 0, Cstar = 0, Lstar = 0;
  {
    int C = 0;  // units of the sequences before this chunk, per tile group
    for (int c0 = 0; c0 < a.batch; c0 += 64) {
      const int b = c0 + lane;
      const int L = b < a.batch ? steps_of(b) : 0;
      const int U = b < a.batch ? L + c : 0;
      int incl = U;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const int pre = C + incl - U;  // units before sequence b, per tile group
      const uint64_t before = __ballot(b < a.batch && n_grp * pre <= lo);
      if (before) {
        const int k = 63 - __builtin_clzll(before);  // the last such lane (prefixes grow with b)
        bstar = c0 + k;
        Cstar = __builtin_amdgcn_readlane(pre, k);
        Lstar = __builtin_amdgcn_readlane(L, k);
      }
      if (blockIdx.x == 0 && w == 0 && b < a.batch) {
        for (int grp = 0; grp < n_grp; ++grp) {
          const int st = n_grp * pre + grp * U + c, s = b * n_grp + grp;  // first step's unit
          const int gf = st / W, gl = (st + L - 1) / W;
          a.piece_tbl[s] = make_int2(gf + s, gl - gf + 1);
        }
      }
      C += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
    }
  }
  if (lo >= hi) return;

  lds_char_t* const stages = (lds_char_t*)stage_mem;
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);
  auto stage_addr = [&](int i) { return uint32_t(uintptr_t(stages + (i % NSTAGE) * kStageBytes)); };

  // row maximum over both lane halves (lanes l and l ^ 32 hold the same row)
  auto row_max = [&](float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };

  // ---- one piece: steps k0..k1-1 of stream (b, grp), partial under id pid
  auto piece = [&](const int b, const int grp, const int k0, const int k1, const int pid) {
    // the per-lane values are formed again for each piece from an opaque thread index: kept across the
    // piece loop they would be spilled (the step loops take every register)
    int tid_p = int(threadIdx.x);
    asm volatile("" : "+v"(tid_p));
    const int lane = tid_p & 63;
    const int h = lane >> 5;    // lane half: K block of the MFMA operands
    const int r32 = lane & 31;  // row of the tile (N index) / token of a score operand (M index)
    const int lrow = lane & 7, lgr = lane >> 3;
    // per-lane LDS offsets.  Score operand k (token r32, granule 2k + h): 9216 (r32 / 8) + 128 h +
    // 16 (r32 % 8) + 256 k.  Transposed read of K step s, half r, channel tile jt (tokens 16s + 8r +
    // 4 hh + li / 4, channels 32 jt + 16 cb + 4 (li % 4)): the base below + 18432 s + 9216 r + 512 jt.
    const int sc_off = 9216 * (r32 >> 3) + 128 * h + 16 * (r32 & 7);
    const int G = lane >> 4, li = lane & 15;
    const int tr_off = 128 * (2 * (G & 1) + ((li >> 1) & 1)) + 64 * (G >> 1) + 16 * (li >> 2) + 8 * (li & 1);
    const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
    const int nblk = (ctx + BLK - 1) / BLK;
    const int kb0 = 2 * k0;
    const int nb = min(2 * k1, nblk) - kb0;  // blocks of the piece
    const int steps = k1 - k0;

    // this lane's row: rr = tile row within the sequence, rows ordered (query, head)
    const int rr = (grp * T + w) * 32 + r32;
    const int iq = rr / a.H;
    // tokens visible to the row in this piece: causal limit and the piece's end (a step spans two
    // blocks, so an odd block count ends the last step one block past the piece)
    const int Lw = min(ctx - a.q_len + iq + 1, (kb0 + nb) * BLK);
    const int Lw_min = min(ctx - a.q_len + ((grp * T + w) * 32) / a.H + 1, (kb0 + nb) * BLK);
    const int64_t R = int64_t(b) * a.q_len * a.H + rr;

    // query tile: B operand of the score MFMA k is granule 2k + h of the row
    u32x4_t qreg[kChunks];
    {
      const u32x4_t* qsrc = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.qcat) + R * ROW);
#pragma unroll
      for (int k = 0; k < kChunks; ++k) qreg[k] = qsrc[2 * k + h];
    }
    // the piece's block ids, staged in LDS once (a miss in the table per step would otherwise
    // stall the barrier that precedes each transfer); nb <= kIdCap by the launch
    {
      const int* bt_row = a.block_table + int64_t(b) * a.bt_stride + kb0;
      for (int e = tid_p; e < nb; e += T * 64) ids_lds[e] = bt_row[e];
    }
    lds_barrier();
    // block ids of step i; the second is clamped into the piece (its lanes are masked when the
    // step has one block)
    auto ids = [&](int i, int& pa, int& pb) {
      pa = __builtin_amdgcn_readfirstlane(ids_lds[2 * i]);
      pb = __builtin_amdgcn_readfirstlane(ids_lds[min(2 * i + 1, nb - 1)]);
    };

    // DMA of step i into stage i % NSTAGE: wave w takes chunks K = w CPW .. w CPW + CPW - 1 (token
    // groups tg = K / 9); lane l of chunk K reads token 8 tg + l % 8, granule 8 (K % 9) + l / 8.
    // prep() computes the wave's source rows for step i, put(c) issues its chunk w CPW + c.
    constexpr int NTG = (CPW + 8) / 9;  // token groups this wave touches (CPW is 9, 18 or 36)
    struct Xfer {
      const char* src[NTG];
      uint32_t dst;
    };
    auto prep = [&](int i, int pa, int pb) {
      Xfer x;
      x.dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(stages + (i % NSTAGE) * kStageBytes + w * CPW * 1024)));
#pragma unroll
      for (int gi = 0; gi < NTG; ++gi) {
        const int tg = (w * CPW) / 9 + gi;     // token group of the step (uniform)
        const int bi = 2 * i + (tg >> 1);       // block index within the piece
        const int trow = 8 * (tg & 1) + lrow;   // token row within the block
        const int phys = (tg >> 1) ? pb : pa;
        const bool ok = bi < nb && unsigned(phys) < unsigned(a.num_blocks) && (kb0 + bi) * BLK + trow < ctx;
        x.src[gi] = (ok ? cache + (int64_t(phys) * BLK + trow) * (ROW * 2) : zero + trow * (ROW * 2)) + 16 * lgr;
      }
      return x;
    };
    auto put = [&](const Xfer& x, int c) { dma16_nt(x.src[c / 9] + 128 * (c % 9), x.dst + 1024 * c); };
    auto issue = [&](int i, int pa, int pb) {
      const Xfer x = prep(i, pa, pb);
#pragma unroll
      for (int c = 0; c < CPW; ++c) put(x, c);
    };

    // zeroed in place in the AGPRs (a zero tile built in VGPRs would be kept, or spilled, across the
    // pieces)
    f32x16_t acc[16];
#pragma unroll
    for (int jt = 0; jt < 16; ++jt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float z;
        asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(z));
        acc[jt][e] = z;
      }
      asm volatile("" : "+a"(acc[jt]));
    }
    float m = -INFINITY, lsum = 0.f;

    // reference-max update for a step with row max mb: returns whether the row's reference moves
    // with terms accumulated (they must then be scaled by alpha = 2^(m_old - m_new): the latest of
    // them may sit just below the new maximum, so they are rescaled, never dropped); sets m, lsum,
    // alpha and the exponent base
    auto ref_update = [&](float mb, float& msub, float& alpha) {
      const bool upd = mb > m + kReset;
      const bool rsc = upd && m != -INFINITY;
      alpha = rsc ? __builtin_amdgcn_exp2f(m - mb) : 1.f;
      lsum *= alpha;
      m = upd ? mb : m;
      msub = m == -INFINITY ? 0.f : m;  // a row with nothing visible yet: every p is exp2(-inf) = 0
      return rsc;
    };

    // scores of step i: S^T on v_mfma_f32_32x32x16_bf16, operand reads kept D ahead of the MFMAs;
    // masked only when the step reaches a row's limit (a uniform test)
    // When a transfer x is given, its CPW chunks are issued among the MFMAs (one after MFMA
    // SP c + 1 for chunk c), so that a transfer held back by the memory pipeline stalls the wave
    // between matrix instructions instead of in one block before them.
    constexpr int SP = kChunks / CPW;
    auto scores = [&](int i, float (&sv)[16], const Xfer* x) {
      uint32_t spa = stage_addr(i) + uint32_t(sc_off);
      asm volatile("" : "+v"(spa));  // one base per step: the 36 offsets fold into the reads
      lds_u32x4_t* sp = (lds_u32x4_t*)uintptr_t(spa);
      constexpr int D = 4;
      u32x4_t ring[D];
      f32x16_t sc = f32x16_t{};
#pragma unroll
      for (int k = 0; k < D; ++k) ring[k] = sp[16 * k];
      // one scheduling region per K step (MFMA k and the read of operand k + D), so that the reads
      // stay D steps ahead: left free, the scheduler moved each read next to its own MFMA
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {
        const u32x4_t xr = ring[k % D];
        sc = mfma32x32(xr, qreg[k], sc);
        if (k + D < kChunks) ring[k % D] = sp[16 * (k + D)];
        if (x && k % SP == SP / 2) put(*x, k / SP);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = sc[r];
      const int tok0 = (kb0 + 2 * i) * BLK;
      if (tok0 + 32 > Lw_min) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = tok0 + 8 * (r >> 2) + 4 * h + (r & 3);
          sv[r] = t < Lw ? sv[r] : -INFINITY;
        }
      }
    };

    // P.C of step i, with the step's softmax folded in.  Before the MFMAs: the row max, the
    // reference update and P for the step's first 16 tokens (the first K step's B operand).  Then
    // 32 slots of one MFMA each (two K steps of 16 tokens x 16 channel tiles); slots 0-11 also
    // compute P for the second 16 tokens (needed from slot 16 on), pinned slot by slot so that the
    // VALU work runs under the MFMAs.
    auto step = [&](int i, float (&sv)[16]) {
      float t0 = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      float t1 = fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7]));
      float t2 = fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11]));
      float t3 = fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15]));
      float msub, alpha;
      const bool rsc = ref_update(row_max(fmaxf(fmaxf(t0, t1), fmaxf(t2, t3))), msub, alpha);
      if (__any(rsc)) {  // rare: a reference moved (rows whose reference stayed have alpha = 1)
        mfma_drain();
#pragma unroll
        for (int jt = 0; jt < 16; ++jt) acc_scale<f32x16_t, 16>(acc[jt], alpha);
      }
      uint32_t pw[8];
#pragma unroll
      for (int r = 0; r < 8; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sv[r] - msub), p1 = __builtin_amdgcn_exp2f(sv[r + 1] - msub);
        lsum += p0 + p1;
        pw[r >> 1] = cvt_pk_bf16(p0, p1);
      }
      asm volatile("" : "+v"(sv[8]));

      uint32_t tpa = stage_addr(i) + uint32_t(tr_off);
      asm volatile("" : "+v"(tpa));  // one base per step: the 64 offsets fold into the reads
      lds_char_t* tp = (lds_char_t*)uintptr_t(tpa);
      auto tr = [&](int k, int r) {  // slot k = 16 s + jt, read r: tokens 16s + 8r + 4(l/32) + 0..3
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tp + 512 * (k & 15) + 18432 * (k >> 4) + 9216 * r));
      };
      constexpr int D = 3;
      s16x4_t ra[D], rb[D];
#pragma unroll
      for (int k = 0; k < D; ++k) {
        ra[k] = tr(k, 0);
        rb[k] = tr(k, 1);
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int s = k >> 4;
        const u32x4_t pb = u32x4_t{pw[4 * s], pw[4 * s + 1], pw[4 * s + 2], pw[4 * s + 3]};
        if ((k & 15) == 0) asm volatile("s_nop 4" ::"v"(pb));  // VALU-written B operand -> MFMA read
        const u32x4_t av = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(ra[k % D], rb[k % D], 0, 1, 2, 3, 4, 5, 6, 7));
        mfma32x32_acc(acc[k & 15], av, pb);
        if (k + D < 32) {
          ra[k % D] = tr(k + D, 0);
          rb[k % D] = tr(k + D, 1);
        }
        if (k < 8) {  // p_r for r = 8 + k, in place
          sv[8 + k] = __builtin_amdgcn_exp2f(sv[8 + k] - msub);
          asm volatile("" : "+v"(sv[8 + k]));
          if (k < 7) asm volatile("" : "+v"(sv[9 + k]));
        } else if (k < 12) {  // pack and sum pairs of the second half
          const int q = k - 4;
          lsum += sv[2 * q] + sv[2 * q + 1];
          pw[q] = cvt_pk_bf16(sv[2 * q], sv[2 * q + 1]);
          asm volatile("" : "+v"(pw[q]), "+v"(lsum));
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // the query tile is in registers (and the previous piece's stores are out) before the first
    // transfer: from here on every outstanding vector memory operation is a transfer of this piece
    wait_vmcnt<0>();
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i) {
      if (i < steps) {
        int pa, pb;
        ids(i, pa, pb);
        issue(i, pa, pb);
      }
    }
    float sv[16];
    // steady state: step i's chunks have landed for this wave (newer steps' transfers may stay in
    // flight), then for every wave; the barrier also retires the stage read at step i - 1, which
    // then takes step i + NSTAGE - 1, issued among the score MFMAs of step i
    int i = 0;
    for (; i + NSTAGE - 1 < steps; ++i) {
      int pa, pb;
      ids(i + NSTAGE - 1, pa, pb);
      wait_vmcnt<(NSTAGE - 2) * CPW>();
      lds_barrier();
      const Xfer x = prep(i + NSTAGE - 1, pa, pb);
      scores(i, sv, &x);
      step(i, sv);
    }
    // the last NSTAGE - 1 steps: nothing left to load
    for (; i < steps; ++i) {
      if (i + NSTAGE - 2 < steps)
        wait_vmcnt<(NSTAGE - 2) * CPW>();
      else
        wait_vmcnt<0>();
      lds_barrier();
      scores(i, sv, nullptr);
      step(i, sv);
    }

    // partial of this wave's rows: channel 32jt + 8q + 4h + e sits in acc[jt][4q + e]; stored
    // normalised, o = acc / l, in fp16 (a convex combination of cache values).  It goes through
    // the (then idle) stages so that each store instruction writes one whole 1 KB row: written
    // straight from the accumulator layout, a store touches 32 rows with 16 bytes each.  Tile of
    // wave w: 32 rows x 1 KB at w * 32 KB, granule G of row r at slot G ^ r.
    mfma_drain();
    lsum = xor32_add(lsum);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    // divided by a power of two when the row's largest |o| would not fit fp16 (the row's values
    // sit in lanes r32 and r32 + 32)
    float mx = 0.f;
#pragma unroll
    for (int jt = 0; jt < 16; ++jt) {
      f32x16_t v = acc[jt];
      asm volatile("" : "+v"(v));
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(v[e]));
    }
    mx = row_max(mx);
    const float down = fp16_fit_scale(mx * inv);
    const float sc = inv * down;
    lds_barrier();  // every wave is done with the last step's stage
    // (the swizzle keys are opaque here so that the 96 addresses are formed at their use, not
    // hoisted out of the piece loop and spilled)
    uint32_t wbase = uint32_t(uintptr_t(stages + w * (32 * 1024))) + r32 * 1024 + 8 * h, wkey = r32;
    uint32_t rbase = uint32_t(uintptr_t(stages + w * (32 * 1024))), rkey = lane;
    asm volatile("" : "+v"(wbase), "+v"(wkey), "+v"(rbase), "+v"(rkey));
#pragma unroll
    for (int jt = 0; jt < 16; ++jt) {
      f32x16_t v = acc[jt];
      asm volatile("" : "+v"(v));  // one tile at a time out of the AGPRs
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t G = 4 * jt + q;
        *(lds_u32x2_t*)uintptr_t(wbase + 16 * (G ^ wkey)) =
            u32x2_t{cvt_pk_f16(v[4 * q] * sc, v[4 * q + 1] * sc), cvt_pk_f16(v[4 * q + 2] * sc, v[4 * q + 3] * sc)};
      }
    }
    const int64_t pidx = int64_t(pid) * RP + w * 32;
    uint16_t* dst = a.part_o16 + pidx * DC + 8 * lane;
#pragma unroll
    for (int r = 0; r < 32; ++r)
      *reinterpret_cast<u32x4_t*>(dst + r * DC) =
          *(const lds_u32x4_t*)uintptr_t(rbase + r * 1024 + 16 * (rkey ^ uint32_t(r)));
    if (h == 0) {
      a.part_ml[pidx + r32] = make_float2(m, lsum);
      a.part_scale[pidx + r32] = 1.f / down;
    }
    lds_barrier();  // every wave is done with the stages before the next piece refills them
  };

  // ---- walk this workgroup's range stream by stream: the steps of stream (b, grp) are units
  // [st, st + L_b) with st = its first unit + c
  int b = bstar, Lb = Lstar;
  int grp = (lo - n_grp * Cstar) / (Lb + c);
  int pos = n_grp * Cstar + grp * (Lb + c);  // first unit of stream (b, grp)
  while (pos < hi) {
    const int st = pos + c;
    const int k0 = max(lo, st) - st, k1 = min(hi, st + Lb) - st;
    if (k1 > k0) piece(b, grp, k0, k1, gr + b * n_grp + grp);
    pos += Lb + c;
    if (++grp == n_grp) {
      grp = 0;
      if (++b == a.batch) break;
      Lb = steps_of(b);
    }
  }
}

hipError_t launch_decode_mt32(const DecodeArgs& a, int T, hipStream_t s) {
  const int grid = a.units;  // one workgroup per resident slot, each with an equal share
  switch (T) {
    case 1:
      launch(decode_bf16_mt32_kernel<1, 2>, dim3(grid), dim3(64), 0, s, a);
      break;
    case 2:
      launch(decode_bf16_mt32_kernel<2, 2>, dim3(grid), dim3(128), 0, s, a);
      break;
    case 4:
      launch(decode_bf16_mt32_kernel<4, 4>, dim3(grid), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
