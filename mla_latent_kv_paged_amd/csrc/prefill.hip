// Chunked prefill over the latent cache, naive form: K and V are expanded from the cached latent
// once per chunk and the new tokens attend to them causally, MHA-style.
//
// What is computed (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收", MLA 的数学结构 and
// 版本 1; 踩坑记录 坑 2 causal mask; vLLM learning book ch. 07 §2.3 paged cache shape, §2.4
// Decoupled RoPE; bxzpzcl.cn hybrid KV-cache page §2.1 block table):
//   K_nope[t, h] = W_uk[h] c_t,  V[t, h] = W_uv[h] c_t,  K[t, h] = [K_nope[t, h] | k_pe_t]
//   out[i, h]    = softmax_{t <= p_i}(scale (q_nope[i,h] . K_nope[t,h] + RoPE(q_pe[i,h], p_i) . k_pe_t)) V[t, h]
// for the n_b new tokens of sequence b at positions p_i = ctx_b - n_b + i, whose rows are already in
// the cache.  Per (row, token) this costs 2 (192 + 128) flops, against 2 (576 + 512) for the
// absorbed form the decode uses: with many query rows per token the expansion pays for itself.
//
// The expansion here (the attention, and the rotation of the queries' q_pe it reads, are in
// prefill_attn.hip): per (sequence, 1,024 tokens, head) one workgroup computes K_nope and V of every token
// (W_uk[h] and W_uv[h], 128 x 512 each, times the latent row) and copies its rope keys, writing rows
// [K_nope | k_pe | V] (320 bf16, rounded once) per (sequence, head, token).  Over bf16 cache rows on
// v_mfma_f32_32x32x16_bf16 with the W rows in registers and the tokens through an LDS ring; over FP8 rows
// on v_mfma_f32_16x16x32_bf16 with the group scales applied per K group (the kernels below say how).
#include "prefill_common.h"

namespace mla {

namespace {

constexpr int kExpandTokens = kPrefillTokens;  // tokens per expansion workgroup (256 per wave)
constexpr int kSubPerWave = kExpandTokens / 64;  // 16-token sub-tiles per wave

}  // namespace

// ----------------------------------------------------------------------------------------- expand

// Expansion over bf16 rows.  One workgroup of eight waves per (sequence, 1,024 tokens, head): waves 0-3
// compute K_nope (W_uk[h]), waves 4-7 V (W_uv[h]), wave w taking output dimensions 32 (w % 4) .. + 31 of its
// part for every token, on v_mfma_f32_32x32x16_bf16 (the 16x16x32 shape issues at half the flop rate on this
// device): dimensions on M, 32 tokens on N, K = 512 in 32 steps.  The wave's W rows (32 x 512) stay in
// registers, 32 A operands of 16 bytes per lane.
// The tokens move HBM -> LDS by DMA, 32 per stage through a ring of kXNS stages, one token row per transfer
// (a 1 KiB row, granule c of token t at slot c ^ (t % 16), so that the 16 lanes of a B-operand read hit
// distinct banks), the rope values 8 tokens per transfer; the B operand of step s is one 16-byte LDS read
// per lane, shared by the eight waves through LDS.  The stage's output (32 tokens x [K_nope | V], bf16) is
// turned to token-major order in LDS and stored 256 contiguous bytes at a time; the K waves also store the
// rope values straight from the stage.  Rows past the context are computed from the zero block and stored
// like the others: they lie inside the (sequence, head) slab of the workspace, whose rows past the context
// are never read.
// Per iteration i of the stage loop: wait for stage i and synchronise; DMA stage i + kXNS - 1; store the
// output tile of stage i - 1 (from LDS); compute stage i; store stage i's rope values (K waves); synchronise
// (every wave has read the previous tile); write stage i's tile to LDS.  Every wave issues the same
// transfers and stores in every iteration, so the wait for stage i is a fixed count of later vector-memory
// instructions (exp_wait); before the first iteration the wave waits for all it has in flight (the first
// kXNS - 1 stages and its W rows).  Three stages are in flight while one is computed.
constexpr int kXTok = 32;                        // tokens per stage
constexpr int kXNS = 4;                          // ring stages
constexpr int kXLat = kXTok * DC * 2;            // 32 KiB: the stage's latent rows
constexpr int kXStage = kXLat + kXTok * DR * 2;  // + 4 KiB of rope values
constexpr int kXRowOut = 2 * DN * 2;             // 512 bytes of output per token in LDS: K_nope | V
constexpr int kXOut = kXTok * kXRowOut;          // 16 KiB: one stage's output tile
constexpr int kXLds = kXNS * kXStage + kXOut;
static_assert(kXLds <= 160 * 1024, "LDS");
static_assert(kExpandTokens % kXTok == 0, "whole stages");

// wait until stage i's transfers have landed: the vector-memory instructions the wave issued after them are
// D (its transfers of a stage) + R (rope stores) + 2 (tile stores) per iteration, in the loop order above.
// Iteration 0 waits for everything in flight, which covers stages 1 and 2 as well.
template <int D, int R>
__device__ __forceinline__ void exp_wait(int i) {
  static_assert(kXNS == 4, "counts for a four-stage ring");
  if (i >= 4)
    wait_vmcnt<2 * D + 6 + 3 * R>();
  else if (i == 3)
    wait_vmcnt<2 * D + 4 + 3 * R>();
  else if (i == 0)
    wait_vmcnt<0>();
}

// the body of wave wv (0..7), whose part is PART (wv / 4)
template <int PART>
__device__ __forceinline__ void expand_body(const PrefillArgs& a, char* smem, int b, int h, int ck, int ctx, int wv) {
  constexpr int D = 4 + (PART == 0 ? 1 : 0);  // transfers per wave and stage (latent rows + rope values)
  constexpr int R = PART == 0 ? 1 : 0;        // rope stores per wave and stage
  const int w4 = wv & 3;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hf = lane >> 5;
  const int t0 = ck * kExpandTokens;
  const int nst = (min(kExpandTokens, ctx - t0) + kXTok - 1) / kXTok;  // stages with visible tokens
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);  // >= 1,152 zero bytes
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;
  char* kvrow0 = reinterpret_cast<char*>(a.kv + (int64_t(b) * a.H + h) * a.t_pad * kKV);
  lds_char_t* const lds = (lds_char_t*)smem;
  lds_char_t* const outl = lds + kXNS * kXStage;

  // block ids of the chunk's 64 blocks (lane i: block t0 / 16 + i; -1 past the context)
  const int ids = (t0 + 16 * lane < ctx) ? bt[t0 / BLK + lane] : -1;

  // DMA of stage k: wave wv moves token rows 4 wv .. 4 wv + 3 (one 1 KiB transfer each); K wave w4 also
  // the rope values of tokens 8 w4 .. 8 w4 + 7 (one transfer)
  auto issue = [&](int k) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(lds + (k % kXNS) * kXStage)));
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int t = 4 * wv + rr;
      const int tok = t0 + kXTok * k + t;
      const int phys = __builtin_amdgcn_readlane(ids, (kXTok * k + t) >> 4 & 63);  // k < nst: no wrap
      const bool ok = k < nst && tok < ctx && unsigned(phys) < unsigned(a.num_blocks);
      const char* row = ok ? cache + (int64_t(phys) * BLK + tok % BLK) * (ROW * 2) : zero;
      dma16(row + 16 * (lane ^ (t & 15)), st + t * (DC * 2));
    }
    if constexpr (PART == 0) {  // lane -> token 8 w4 + lane / 8, granule lane % 8 of its rope values
      const int t = 8 * w4 + (lane >> 3);
      const int tok = t0 + kXTok * k + t;
      const int phys = __shfl(ids, (kXTok * k + t) >> 4 & 63, 64);
      const bool ok = k < nst && tok < ctx && unsigned(phys) < unsigned(a.num_blocks);
      const char* row = ok ? cache + (int64_t(phys) * BLK + tok % BLK) * (ROW * 2) : zero;
      dma16(row + DC * 2 + 16 * (lane & 7), st + kXLat + 1024 * w4);
    }
  };
  // output tile of stage k from LDS: wave wv stores tokens 4 wv .. 4 wv + 3, two per instruction (K_nope:
  // granules 0..15 of the LDS row, row bytes 0..255; V: granules 16..31, row bytes 384..639)
  auto store_tile = [&](int k) {
    const lds_char_t* o = outl;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int t = 4 * wv + 2 * e + (lane >> 5), g = lane & 31;
      const u32x4_t v = *(const lds_u32x4_t*)(o + t * kXRowOut + 16 * (g ^ (t & 15)));
      *reinterpret_cast<u32x4_t*>(kvrow0 + int64_t(t0 + kXTok * k + t) * kKVBytes + (g < 16 ? 0 : (DN + DR) * 2 - 256) +
                                  16 * g) = v;
    }
  };

#pragma unroll
  for (int k = 0; k < kXNS - 1; ++k) issue(k);
  // the wave's W rows: A operand of step s = row 32 w4 + l32, channels 16 s + 8 hf .. + 7 (requested
  // after the first stages, and all waited for with them before the loop's first MFMA, so that the
  // compiler's own waits for them never wait for a later transfer)
  u32x4_t wf[32];
  {
    const char* W = reinterpret_cast<const char*>((PART ? a.W_uv : a.W_uk) + int64_t(h) * DN * DC) +
                    int64_t(32 * w4 + l32) * (DC * 2) + 16 * hf;
#pragma unroll
    for (int s = 0; s < 32; ++s) wf[s] = *reinterpret_cast<const u32x4_t*>(W + 32 * s);
  }
  for (int i = 0; i < nst; ++i) {
    exp_wait<D, R>(i);
    lds_barrier();
    issue(i + kXNS - 1);  // past the last stage: the zero block, so that every iteration issues the same
    if (i > 0) store_tile(i - 1);
    const lds_char_t* sg = lds + (i % kXNS) * kXStage;
    // B operand of step s: token l32, channels 16 s + 8 hf .. + 7 = granule 2 s + hf
    const lds_char_t* brow = sg + l32 * (DC * 2);
    auto ldb = [&](int s) { return *(const lds_u32x4_t*)(brow + 16 * ((2 * s + hf) ^ (l32 & 15))); };
    f32x16_t acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    constexpr int DB = 4;  // B reads kept ahead of the MFMAs
    u32x4_t bq[DB];
#pragma unroll
    for (int s = 0; s < DB; ++s) bq[s] = ldb(s);
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const u32x4_t bv = bq[s % DB];
      if (s + DB < 32) bq[s % DB] = ldb(s + DB);
      acc = mfma32x32(wf[s], bv, acc);
    }
    if constexpr (PART == 0) {  // rope values of stage i: lane -> token 8 w4 + lane / 8, granule lane % 8
      const int t = 8 * w4 + (lane >> 3);
      const u32x4_t v = *(const lds_u32x4_t*)(sg + kXLat + t * (DR * 2) + 16 * (lane & 7));
      *reinterpret_cast<u32x4_t*>(kvrow0 + int64_t(t0 + kXTok * i + t) * kKVBytes + DN * 2 + 16 * (lane & 7)) = v;
    }
    lds_barrier();  // every wave has read the previous tile out of LDS
    // D[dimension][token]: lane (token l32, half hf) holds dimensions 32 w4 + 8 q + 4 hf .. + 3 in
    // acc[4 q .. 4 q + 3]; token-major tile row t = 32 granules (K_nope 0..15, V 16..31), granule gi at
    // slot gi ^ (t % 16)
    lds_char_t* o = outl + l32 * kXRowOut;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int gi = 16 * PART + 4 * w4 + q;
      *(lds_u32x2_t*)(o + 16 * (gi ^ (l32 & 15)) + 8 * hf) =
          u32x2_t{cvt_pk_bf16(acc[4 * q], acc[4 * q + 1]), cvt_pk_bf16(acc[4 * q + 2], acc[4 * q + 3])};
    }
  }
  lds_barrier();
  store_tile(nst - 1);
  wait_vmcnt<0>();  // the transfers issued past the last stage land before the workgroup's LDS is released
}

// 160 KiB of LDS and 512 threads: one workgroup, two waves per SIMD, per CU.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_expand_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kXLds];
  // Work unit u = (sequence b, token chunk ck, head h), h fastest.  Workgroup i is dispatched to XCD i % 8;
  // each XCD gets a contiguous range of units, so that the H workgroups reading one chunk's latent rows
  // share an L2.
  const int per_xcd = (a.units + 7) >> 3;
  int u = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (u >= a.units) return;
  const int nck = a.t_pad / kExpandTokens;
  const int h = u % a.H;
  u /= a.H;
  const int ck = u % nck;
  const int b = u / nck;
  if (b >= a.batch) return;
  int c0;
  const int n = chunk_of(a, b, &c0);
  if (n == 0) return;
  const int ctx = clamp_ctx(a.seq_lens[b], n, a.max_seq_len);
  if (ck * kExpandTokens >= ctx) return;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv >= 4)
    expand_body<1>(a, smem, b, h, ck, ctx, wv);
  else
    expand_body<0>(a, smem, b, h, ck, ctx, wv);
}

// The expansion over FP8 rows (656 bytes: latent codes, bf16 rope values, four fp32 group scales;
// mla_cache_write), on v_mfma_f32_16x16x32_bf16 with the 128 output dimensions on M and 16 tokens on N.
// Every e4m3 value is a bf16 value, so the codes are the MFMA's B operand exactly, and the K steps of
// each group of 128 channels accumulate apart; the group's tile is then added to the output times that
// token's group scale (a lane holds one token: one scale per lane), in fp32.  (On the 32x32x16 shape the
// two accumulator sets of the bf16 kernel's tile do not fit beside the register ring.)  128 KiB of LDS:
// one workgroup, one wave per SIMD, per CU.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_expand_fp8_kernel(PrefillArgs a) {
  constexpr int kRowBytes = kFp8Row;  // one cache row
  constexpr int kRopeOff = DC;        // its rope values (bf16)
  // W_uk[h] or W_uv[h]: 128 rows of 512 values; granule c (8 values) of row r at slot c ^ (r % 16)
  __shared__ __attribute__((aligned(16))) char wl[DN * DC * 2];
  static_assert(DN == DV, "one staging buffer for both parts");
  const int nck = a.t_pad / kExpandTokens;
  const int per_xcd = (a.units + 7) >> 3;  // XCD-contiguous units, as in prefill_expand_kernel
  int u = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (u >= a.units) return;
  const int part = u & 1;  // 0: K (W_uk, also the rope keys), 1: V (W_uv)
  u >>= 1;
  const int h = u % a.H;
  u /= a.H;
  const int ck = u % nck;
  const int b = u / nck;
  if (b >= a.batch) return;
  int c0;
  const int n = chunk_of(a, b, &c0);
  if (n == 0) return;
  const int ctx = clamp_ctx(a.seq_lens[b], n, a.max_seq_len);
  const int t0 = ck * kExpandTokens;
  if (t0 >= ctx) return;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  {  // stage the weight part: wave w moves rows 32w .. 32w+31, one 1 KiB row per transfer
    const char* W = reinterpret_cast<const char*>((part ? a.W_uv : a.W_uk) + int64_t(h) * DN * DC);
    const uint32_t base = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t((lds_char_t*)wl)));
#pragma unroll 4
    for (int rr = 0; rr < 32; ++rr) {
      const int r = 32 * w + rr;
      dma16(W + r * (DC * 2) + 16 * (lane ^ (r & 15)), base + r * (DC * 2));
    }
    wait_vmcnt<0>();
    lds_barrier();
  }
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);  // >= 1,152 zero bytes
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;
  uint16_t* kvrow0 = a.kv + (int64_t(b) * a.H + h) * a.t_pad * kKV;
  // A operand of MFMA (dim tile jt, K step s): row 16 jt + r16, granule 4 s + g
  const lds_char_t* wa = (const lds_char_t*)wl + r16 * (DC * 2);

  // wave w: tokens t0 + 16 kSubPerWave w + 16 st + (lane % 16); the next sub-tile's latent rows are
  // loaded while the current one is multiplied (two register buffers, the loop unrolled by two)
  const int tw = t0 + 16 * kSubPerWave * w;
  // sub-tile st is one paged block: the wave's kSubPerWave block ids, read once (lane st holds id st)
  static_assert(kSubPerWave <= 64, "one id per lane");
  const int ids = (lane < kSubPerWave && tw + 16 * lane < ctx) ? bt[tw / BLK + lane] : -1;
  asm volatile("" ::"v"(ids));  // complete before the row loads
  // the latent part of one token row: 16 K steps of 8 codes per lane (8 bytes) and the row's four group
  // scales
  struct Brow {
    u32x2_t c[16];
    f32x4_t sc;
  };
  auto load_b = [&](int st, Brow& bq) {
    const int tb = tw + 16 * st;
    const int tok = tb + r16;
    const int phys = __builtin_amdgcn_readlane(ids, st);  // st <= kSubPerWave < 64: -1 past the range
    const bool ok = tok < ctx && unsigned(phys) < unsigned(a.num_blocks);
    // rows past the context or of an invalid block read the zero block: no divergent loads, which
    // would make the compiler wait for every load in flight
    const char* crow = ok ? cache + (int64_t(phys) * BLK + tok % BLK) * kRowBytes : zero;
#pragma unroll
    for (int s = 0; s < 16; ++s) bq.c[s] = *reinterpret_cast<const u32x2_t*>(crow + 32 * s + 8 * g);
    bq.sc = *reinterpret_cast<const f32x4_t*>(crow + DC + 2 * DR);
    return phys;
  };
  auto step = [&](int st, const Brow& cb, int phys) {
    const int tb = tw + 16 * st;
    const int tok = tb + r16;
    f32x4_t acc[8];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the eight A operands of K step s + 1 are read while the MFMAs of step s run
    u32x4_t av[2][8];
    auto load_a = [&](int s, u32x4_t (&d)[8]) {
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) d[jt] = *(const lds_u32x4_t*)(wa + jt * 16 * (DC * 2) + 16 * ((4 * s + g) ^ r16));
    };
    load_a(0, av[0]);
#pragma unroll
    for (int G = 0; G < 4; ++G) {  // scale group G: K steps 4G .. 4G + 3
      f32x4_t gacc[8];
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) gacc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s = 4 * G + q;
        if (s + 1 < 16) load_a(s + 1, av[(s + 1) & 1]);
        const u32x4_t bv = codes8(cb.c[s]);
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) gacc[jt] = mfma32v(av[s & 1][jt], bv, gacc[jt]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) acc[jt] += cb.sc[G] * gacc[jt];
    }
    // D[dim][token]: lane (token r16, g) holds dims 16 jt + 4 g .. + 3
    if (tok < ctx) {
      uint16_t* dst = kvrow0 + int64_t(tok) * kKV + (part ? DN + DR : 0) + 4 * g;
#pragma unroll
      for (int jt = 0; jt < 8; ++jt)
        *reinterpret_cast<u32x2_t*>(dst + 16 * jt) =
            u32x2_t{cvt_pk_bf16(acc[jt][0], acc[jt][1]), cvt_pk_bf16(acc[jt][2], acc[jt][3])};
    }
    if (part == 0) {  // rope keys of the 16 tokens: lane -> token lane / 4, values 16 (lane % 4) .. + 15
      const int rt = tb + (lane >> 2);
      if (rt < ctx) {
        const bool rok = unsigned(phys) < unsigned(a.num_blocks);
        const char* src = (rok ? cache + (int64_t(phys) * BLK + rt % BLK) * kRowBytes + kRopeOff : zero) + 32 * (lane & 3);
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(src);
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(src + 16);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(kvrow0 + int64_t(rt) * kKV + DN + 16 * (lane & 3));
        dst[0] = v0;
        dst[1] = v1;
      }
    }
  };
  if (tw >= ctx) return;
  // groups of four sub-tiles; within a group the buffers alternate at compile time, and the
  // prefetch is unconditional (past the wave's range it reads the zero block: lane kSubPerWave's id
  // is -1), so that no branch guards a load
  Brow bq[2];
  int ph[2];
  ph[0] = load_b(0, bq[0]);
  for (int G = 0; G < kSubPerWave / 4; ++G) {
    if (tw + 64 * G >= ctx) break;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int cur = 4 * G + st;
      ph[(st + 1) & 1] = load_b(cur + 1, bq[(st + 1) & 1]);
      if (tw + 16 * cur < ctx) step(cur, bq[st & 1], ph[st & 1]);
    }
  }
}

hipError_t launch_prefill_expand(PrefillArgs a, bool fp8, hipStream_t s) {
  // bf16: a workgroup per (sequence, chunk, head); FP8: per (sequence, chunk, head, part)
  const int64_t units = int64_t(a.batch) * (a.t_pad / kExpandTokens) * a.H * (fp8 ? 2 : 1);
  if (units > 0x7fffffff) return hipErrorInvalidValue;
  a.units = int32_t(units);
  const int grid = ((a.units + 7) >> 3) << 3;
  if (fp8)
    launch(prefill_expand_fp8_kernel, dim3(grid), dim3(256), 0, s, a);
  else
    launch(prefill_expand_kernel, dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(PrefillArgs a, hipStream_t s) { return launch_prefill_attn32(a, s); }

}  // namespace mla
