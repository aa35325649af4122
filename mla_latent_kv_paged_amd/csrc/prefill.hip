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
// [K_nope | k_pe | V] (320 bf16, rounded once) per (sequence, head, token), on v_mfma_f32_32x32x16_bf16 with
// the W rows in registers and the tokens through an LDS ring.  Over an FP8 cache the context rows are
// first dequantised to bf16 rows (code x group scale, rounded once) in the workspace, which the same
// expansion then reads in place of the cache.
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
  // over an FP8 cache: the sequence's dequantised rows, token t at row t (no block table)
  const char* lat = a.lat ? reinterpret_cast<const char*>(a.lat + int64_t(b) * a.t_pad * ROW) : nullptr;
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
      const bool ok = k < nst && tok < ctx && (lat || unsigned(phys) < unsigned(a.num_blocks));
      const char* row = ok ? (lat ? lat + int64_t(tok) * (ROW * 2) : cache + (int64_t(phys) * BLK + tok % BLK) * (ROW * 2))
                           : zero;
      dma16(row + 16 * (lane ^ (t & 15)), st + t * (DC * 2));
    }
    if constexpr (PART == 0) {  // lane -> token 8 w4 + lane / 8, granule lane % 8 of its rope values
      const int t = 8 * w4 + (lane >> 3);
      const int tok = t0 + kXTok * k + t;
      const int phys = __shfl(ids, (kXTok * k + t) >> 4 & 63, 64);
      const bool ok = k < nst && tok < ctx && (lat || unsigned(phys) < unsigned(a.num_blocks));
      const char* row = ok ? (lat ? lat + int64_t(tok) * (ROW * 2) : cache + (int64_t(phys) * BLK + tok % BLK) * (ROW * 2))
                           : zero;
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

// Over an FP8 cache (rows of 656 bytes: 512 e4m3 codes, 64 bf16 rope values, four fp32 group scales;
// mla_cache_write): the context rows of each sequence are first dequantised into lat [batch, t_pad, 576] bf16,
// code x its group's scale in fp32 rounded once to nearest even, the rope values as stored.  Rows past the
// context are not written (the expansion reads the zero block there); a row of an invalid block id becomes
// zeros, as the bf16 path reads such a row from the zero block.  Grid (t_pad / 32, batch): four waves of
// eight tokens, lane l converting codes 8 l .. 8 l + 7 of each token; all loads are issued first.
__global__ __launch_bounds__(256) void prefill_dequant_fp8_kernel(PrefillArgs a) {
  const int b = blockIdx.y;
  int c0;
  const int n = chunk_of(a, b, &c0);
  if (n == 0) return;
  const int ctx = clamp_ctx(a.seq_lens[b], n, a.max_seq_len);
  const int lane = threadIdx.x & 63;
  const int tb = int(blockIdx.x) * 32 + 8 * (threadIdx.x >> 6);  // the wave's first token, 8 | tb
  if (tb >= ctx) return;
  const char* zero = static_cast<const char*>(a.zero_block);  // >= 1,152 zero bytes
  const int phys = a.block_table[int64_t(b) * a.bt_stride + tb / BLK];  // the wave's eight tokens share a block
  const bool okb = unsigned(phys) < unsigned(a.num_blocks);
  const char* base = okb ? static_cast<const char*>(a.cache) + (int64_t(phys) * BLK + tb % BLK) * kFp8Row : zero;
  const int64_t rstep = okb ? kFp8Row : 0;  // the zero block stands for every row of an invalid block
  u32x2_t cw[8];
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    cw[i] = *reinterpret_cast<const u32x2_t*>(base + i * rstep + 8 * lane);
    sc[i] = *reinterpret_cast<const float*>(base + i * rstep + DC + 2 * DR + 4 * (lane >> 4));
  }
  // rope values: lane -> token lane / 8, granule lane % 8
  const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(base + (lane >> 3) * rstep + DC + 16 * (lane & 7));
  uint16_t* lat = a.lat + (int64_t(b) * a.t_pad + tb) * ROW;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (tb + i >= ctx) break;
    const u32x4_t v = codes8(cw[i]);  // the codes as bf16, exactly
    u32x4_t y;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y[e] = cvt_pk_bf16(__uint_as_float(v[e] << 16) * sc[i], __uint_as_float(v[e] & 0xffff0000u) * sc[i]);
    *reinterpret_cast<u32x4_t*>(lat + i * ROW + 8 * lane) = y;
  }
  if (tb + (lane >> 3) < ctx) *reinterpret_cast<u32x4_t*>(lat + (lane >> 3) * ROW + DC + 8 * (lane & 7)) = rv;
}

hipError_t launch_prefill_expand(PrefillArgs a, bool fp8, hipStream_t s) {
  // a workgroup per (sequence, chunk, head)
  const int64_t units = int64_t(a.batch) * (a.t_pad / kExpandTokens) * a.H;
  if (units > 0x7fffffff || a.batch > 65535 || (fp8 && !a.lat)) return hipErrorInvalidValue;
  a.units = int32_t(units);
  if (fp8) {
    launch(prefill_dequant_fp8_kernel, dim3(a.t_pad / 32, a.batch), dim3(256), 0, s, a);
  } else {
    a.lat = nullptr;
  }
  const int grid = ((a.units + 7) >> 3) << 3;
  launch(prefill_expand_kernel, dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(PrefillArgs a, hipStream_t s) { return launch_prefill_attn32(a, s); }

}  // namespace mla
