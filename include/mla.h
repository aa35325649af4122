/*
 * mla.h -- C ABI of libmla: DeepSeek-V2-style Multi-head Latent Attention (MLA) decode over a
 * paged latent KV cache with matrix absorption, for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *  [P-vllm]   vLLM learning book ch. 07 "模型架构特异：MLA / Mamba / MoE 在 vLLM 源码层",
 *             §2.1 算法核心, §2.2 vLLM 源码挂载点 (wrapper forward: down-projection, decoupled
 *             RoPE, cache write by slot_mapping, attention), §2.3 (cache shape
 *             (n_blocks, block, 1, latent_d + rope_d)), §2.4 Decoupled RoPE.
 *  [P-mini]   mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收", sections
 *             "MLA 的数学结构", 版本 1 (Naive), 版本 3 (矩阵吸收, _build_absorbed),
 *             踩坑记录 坑 2 (causal mask) and 坑 3 (norm before absorption), 设计取舍.
 *  [P-hybrid] bxzpzcl.cn, KV-cache management for hybrid models, §2.1 (block table maps
 *             logical to physical pages; one cache per layer, pages shared by all requests).
 *
 * Conventions shared by every call
 *  - Dimensions supported: kv_lora_rank (dc) 512, qk_rope_head_dim (dr) 64,
 *    qk_nope_head_dim (dn) 128, v_head_dim (dv) 128, block_size 16, num_heads a multiple of 16.
 *    Anything else returns MLA_EUNSUPPORTED.
 *  - Storage dtype (mla_config.dtype) applies to q, c_kv, k_pe, the cache, the weights, gamma
 *    and out.  MLA_BF16 computes scores and P*c_kv with bf16 MFMA inputs and fp32 accumulation;
 *    MLA_F32 computes in fp32 throughout.  cache_write evaluates each row in fp64 and rounds once
 *    (round to nearest even) in both modes.
 *  - Every data pointer is DEVICE memory owned by the caller, borrowed until the work queued on
 *    `stream` has completed.  `stream` is a hipStream_t passed as void* (NULL = default stream).
 *  - cache_write and decode are asynchronous: no host synchronisation, no allocation.
 *  - Device-resident indices (positions, slot_mapping, block_table, seq_lens) are not read by
 *    the host.  Out-of-range values are handled as documented per call, never by faulting.
 *  - The context is not thread-safe: it owns one decode workspace.  Calls on one context must be
 *    serialised on one stream.
 *  - No C++ exception crosses this boundary; errors are returned as mla_status.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mla_ctx mla_ctx; /* opaque, library-owned */

/* MLA_BF16_FP8: bf16 like MLA_BF16 for q, c_kv, k_pe, the weights, gamma and out; the cache holds
 * FP8 rows (see mla_cache_write).  The vLLM learning book (ch. 07) lists an FP8 KV cache for MLA;
 * the pages fix no scale convention or layout, so both are this library's. */
typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_BF16_FP8 = 2 } mla_dtype;

typedef enum {
  MLA_OK = 0,
  MLA_EINVAL = -1,       /* null pointer, negative size, inconsistent argument */
  MLA_EUNSUPPORTED = -2, /* dims or dtype outside the supported set */
  MLA_ENOMEM = -3,       /* device allocation failed */
  MLA_EHIP = -4,         /* a HIP runtime call or kernel launch failed */
  MLA_ECAP = -5          /* a size exceeds the caps fixed at mla_absorb_weights */
} mla_status;

typedef struct {
  int32_t num_heads;        /* H, multiple of 16 */
  int32_t kv_lora_rank;     /* dc = 512 */
  int32_t qk_nope_head_dim; /* dn = 128 */
  int32_t qk_rope_head_dim; /* dr = 64 */
  int32_t v_head_dim;       /* dv = 128 */
  int32_t block_size;       /* 16 */
  int32_t dtype;            /* mla_dtype */
  float softmax_scale;      /* <= 0 selects 1/sqrt(dn + dr) */
  float rms_eps;            /* RMSNorm epsilon, e.g. 1e-6 */
  float rope_theta;         /* RoPE base, e.g. 10000 */
  int32_t max_q_tokens;     /* cap on batch * q_len per decode (sizes the workspace) */
  int32_t max_batch;        /* cap on batch per decode */
  int32_t max_position;     /* RoPE positions 0..max_position are supported */
  int32_t max_seq_len;      /* cap on a context length (incl. new tokens) per decode */
} mla_config;

/*
 * mla_absorb_weights -- S0 of the decode path: split kv_b_proj into the absorbed factors and
 * build a context.  [P-mini] 版本 3 _build_absorbed views kv_b_proj as (H, dn + dv, dc): per
 * head, the first dn rows form W_uk (folded into the query: q_lat = q_nope . W_uk) and the next
 * dv rows form W_uv (applied last: out = o_lat . W_uv^T).  The copy is exact (no arithmetic);
 * the library repacks both into its own kernel layouts.
 *
 *  cfg           host pointer, read during the call only.
 *  kv_b_proj_w   device [H*(dn+dv), dc] row-major in the storage dtype, per-head row blocks of
 *                dn nope rows then dv value rows.  May be freed after the call returns.
 *  kv_norm_gamma device [dc] RMSNorm weight (kv_a_layernorm) in the storage dtype, or NULL for
 *                all-ones.  Copied; may be freed after the call returns.
 *  stream        hipStream_t; the call synchronises this stream once before returning.
 *  out           receives the new context on MLA_OK, NULL otherwise.
 * Returns MLA_EINVAL (null cfg/weights/out, non-positive caps), MLA_EUNSUPPORTED (dims, dtype),
 * MLA_ENOMEM, MLA_EHIP.  The context owns W_uk/W_uv, gamma, an fp64 RoPE table for positions
 * 0..max_position and the split-KV workspace (sized from the caps).
 */
mla_status mla_absorb_weights(const mla_config* cfg, const void* kv_b_proj_w, const void* kv_norm_gamma,
                              void* stream, mla_ctx** out);

/*
 * mla_cache_write -- S1: [P-vllm] §2.2 steps 2-3 and §2.3.  For each new token j:
 *   row = [ RMSNorm(c_kv[j]) * gamma  |  RoPE(k_pe[j], positions[j]) ]   (dc + dr values)
 * stored at slot s = slot_mapping[j] = physical_block * 16 + offset, i.e. in
 * kv_cache[s / 16][s % 16][0][:].  RMSNorm: x / sqrt(mean(x^2) + eps) ([P-mini] 坑 3, the
 * kv_a_layernorm); RoPE: interleaved pairs (x[2i], x[2i+1]) rotated by p * theta^(-2i/dr)
 * ([P-vllm] §2.4; the pairing is this library's reading, the pages leave it open).
 * The row is evaluated in fp64 and rounded once to the storage dtype (round to nearest even).
 *
 *  c_kv, c_kv_row_stride  device [T, dc] raw (un-normed) latent; stride in elements (>= dc).
 *  k_pe, k_pe_row_stride  device [T, dr] un-rotated rope key; stride in elements (>= dr).
 *  positions              device int32 [T] RoPE position of each token.
 *  slot_mapping           device int32 [T]; a negative slot skips the token (padding).
 *  num_tokens             T >= 0 (0 is a no-op).
 *  kv_cache, num_blocks   device [num_blocks, 16, 1, dc + dr] in the storage dtype; with
 *                         MLA_BF16_FP8, [num_blocks, 16, 1, 656] bytes, one row per slot:
 *                           bytes   0..511  the normed latent as FP8 E4M3 codes (OCP: bias 7, max
 *                                           448, no infinities), channel order;
 *                           bytes 512..639  the rotated rope values, bf16 (round to nearest even);
 *                           bytes 640..655  4 fp32 scales, one per group of 128 latent channels.
 *                         Channel i holds e4m3(code_i) * scale[i / 128].  Per group, scale =
 *                         fp32(amax / 448) (amax = largest |value|; stepped up one fp32 value if
 *                         amax / scale would exceed 448; 1 for an all-zero group) and code_i =
 *                         the E4M3 value nearest value_i / scale (quotient in fp64), ties to the
 *                         even code.  A position outside 0..max_position writes NaN codes, rope
 *                         values and scales.
 * Device-side handling: a slot at or beyond num_blocks*16 is skipped; a position outside
 * 0..max_position writes a row of NaN so that the error is visible downstream.
 * Slots not named in slot_mapping are not touched.  Two tokens naming one slot race.
 * Returns MLA_EINVAL (null ctx/pointers with T > 0, strides too small, num_blocks <= 0),
 * MLA_EHIP on launch failure.
 */
mla_status mla_cache_write(mla_ctx* ctx, const void* c_kv, int64_t c_kv_row_stride, const void* k_pe,
                           int64_t k_pe_row_stride, const int32_t* positions, const int32_t* slot_mapping,
                           int32_t num_tokens, void* kv_cache, int32_t num_blocks, void* stream);

/*
 * mla_decode -- S2..S7: absorbed MLA attention over the paged latent cache ([P-mini] 版本 3
 * reassociated; [P-hybrid] §2.1 paging).  For query i of sequence b (row n = b*q_len + i),
 * position p = seq_lens[b] - q_len + i, and head h:
 *   q_lat   = q[n,h,:dn] . W_uk[h]                         (dc values)
 *   q_pe'   = RoPE(q[n,h,dn:], p)
 *   s_t     = scale * (q_lat . c_t + q_pe' . k_pe_t)        for cache tokens t <= p, else masked
 *             ([P-mini] 设计取舍 two-part score, 坑 2 causal mask)
 *   o_lat   = softmax(s) . C                                 (dc values)
 *   out[n,h]= o_lat . W_uv[h]^T                             (dv values)
 * Cache token t of sequence b is the row kv_cache[block_table[b*stride + t/16]][t%16][0].
 * The context is cut into splits processed in parallel; their (max, sum, acc) partials are
 * merged by a log-sum-exp combine.  Results are deterministic for fixed inputs and split count.
 *
 *  q                    device [batch*q_len, H, dn + dr], per head [nope | rope] (rope un-rotated).
 *  batch, q_len         batch >= 1, 1 <= q_len; batch <= max_batch, batch*q_len <= max_q_tokens.
 *  kv_cache, num_blocks device [num_blocks, 16, 1, dc + dr] (already written for every t < ctx);
 *                       MLA_BF16_FP8: the 656-byte rows of mla_cache_write, whose latent values are
 *                       e4m3(code) * scale exactly (the kernel rounds nothing on the way in).
 *  block_table, stride  device int32 [batch, stride]; entries for t >= ctx are not read.
 *  seq_lens             device int32 [batch]: context length ctx_b INCLUDING the q_len new
 *                       tokens (which must already be in the cache), q_len <= ctx_b <= max_seq_len.
 *  max_seq_len          host int: an upper bound of every seq_lens[b] (sizes the launch).
 *  out                  device [batch*q_len, H, dv] in the storage dtype (round to nearest even).
 * Device-side handling: a block_table entry outside [0, num_blocks) reads as a block of zeros;
 * seq_lens[b] is clamped to [q_len, max_seq_len].
 * Returns MLA_EINVAL (null pointers, batch < 1, q_len < 1, max_seq_len < q_len, stride smaller
 * than ceil(max_seq_len/16)), MLA_ECAP (batch, batch*q_len or max_seq_len above the caps, or
 * max_seq_len - 1 above max_position), MLA_EHIP.
 */
mla_status mla_decode(mla_ctx* ctx, const void* q, int32_t batch, int32_t q_len, const void* kv_cache,
                      int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                      const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream);

/*
 * mla_decode_noalloc -- mla_decode for callers that cannot allocate device memory during the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, semantics, launch shape and kernels as mla_decode, so the output is bit for bit the
 * same; the decode's scratch (the [q_lat | q_pe'] rows, the split or piece partials, their
 * (max, sum) pairs and scales, the piece table) lives in a static device region of 64 MiB that the
 * library holds on every GPU it runs on until the process ends, instead of the context's workspace.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *  - A decode whose scratch would exceed 64 MiB returns MLA_ECAP (for example, 16 heads: a batch of
 *    64 at 4,097 tokens uses about 5.4 MB; 128 heads x 128 sequences do not fit).
 *  - Every call on one GPU shares that GPU's region and leaves its contents behind: calls that
 *    overlap on one GPU (other streams, other contexts, other threads) race and must be serialised
 *    by the caller.  Nothing in the region needs clearing between calls.
 *  - MLA_EHIP if the region's address could not be looked up when the context was made.
 * Returns what mla_decode returns otherwise.
 */
mla_status mla_decode_noalloc(mla_ctx* ctx, const void* q, int32_t batch, int32_t q_len, const void* kv_cache,
                              int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream);

/*
 * mla_decode_step -- one decode step of the layer ([P-vllm] §2.2 wrapper forward: the new tokens'
 * cache write by slot_mapping, then attention): exactly mla_cache_write(ctx, c_kv, ..., num_tokens,
 * kv_cache, num_blocks) followed by mla_decode(ctx, q, ..., kv_cache, num_blocks, ...), with the
 * same arguments, semantics and results (cache rows and out bit for bit).  With bf16 storage (and
 * MLA_BF16_FP8 rows) the cache write runs in the query absorption's launch: the two are
 * independent, and only the attention kernel after them reads the new rows.  fp32 storage
 * launches them one after the other.  num_tokens may be 0 (no write).
 * Every argument is checked before anything is launched: a failing call writes nothing.
 * Returns what either call returns for its arguments.
 */
mla_status mla_decode_step(mla_ctx* ctx, const void* c_kv, int64_t c_kv_row_stride, const void* k_pe,
                           int64_t k_pe_row_stride, const int32_t* positions, const int32_t* slot_mapping,
                           int32_t num_tokens, const void* q, int32_t batch, int32_t q_len, void* kv_cache,
                           int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                           const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream);

/*
 * mla_layer_weights -- attach one layer's projections to a context, for mla_layer_decode_step: the
 * weight path q_proj, kv_a_proj_with_mqa, kv_b_proj, o_proj of [P-mini] 版本 1 (kv_b_proj and the
 * kv_a_layernorm gamma are the context's own, from mla_absorb_weights), and the input_layernorm of
 * the decoder layer ([P-vllm] DeepseekV3DecoderLayer listing).  bf16 contexts (MLA_BF16 and
 * MLA_BF16_FP8) only.
 *
 *  hidden_dim        D, the hidden size: a positive multiple of 512 (DeepSeek-V2-Lite: 2,048).
 *  q_proj_w          device bf16 [H*(dn+dr), D]: per head [nope | rope] query rows (no query
 *                    low-rank step, the V2-Lite shape).
 *  kv_a_proj_w       device bf16 [dc + dr, D]: compressed_kv rows then k_pe rows.
 *  o_proj_w          device bf16 [D, H*dv]: columns head-major (head h owns h*dv .. h*dv + dv - 1).
 *  input_norm_gamma  device bf16 [D] or NULL (all ones); used with MLA_LAYER_INPUT_NORM.
 *  flags             MLA_LAYER_INPUT_NORM: RMSNorm the hidden states first (with the context's
 *                    rms_eps); MLA_LAYER_RESIDUAL: add the hidden states to the output.  Both: the
 *                    attention half of the decoder layer; neither: the bare attention module of
 *                    [P-vllm] §2.2.
 *  stream            the call synchronises it once before returning.
 * The context keeps its own copies (the q_proj and kv_a_proj rows multiplied by input_norm_gamma
 * and rounded to bf16 once); the caller's buffers may be freed after the call.  It also sizes the
 * step's workspace from the context's max_q_tokens.  A second call replaces the first.
 * Returns MLA_EINVAL (null ctx or weights, unknown flags), MLA_EUNSUPPORTED (fp32 context, hidden_dim
 * not a positive multiple of 512), MLA_ENOMEM, MLA_EHIP.
 */
enum { MLA_LAYER_INPUT_NORM = 1, MLA_LAYER_RESIDUAL = 2 };
mla_status mla_layer_weights(mla_ctx* ctx, int32_t hidden_dim, const void* q_proj_w, const void* kv_a_proj_w,
                             const void* o_proj_w, const void* input_norm_gamma, int32_t flags, void* stream);

/*
 * mla_layer_decode_step -- one decode step of one attention layer from hidden states ([P-vllm] §2.2
 * wrapper forward: down-projection, decoupled RoPE, cache write by slot_mapping, attention; the
 * DeepseekV3DecoderLayer listing for input_layernorm and the residual; [P-mini] 版本 1 for the
 * kv_a_proj_with_mqa split [:dc] | [dc:] and o_proj).  For the N = batch * q_len new tokens
 * (row n = b*q_len + i):
 *   x      = RMSNorm(hidden[n]) * input_norm_gamma          (MLA_LAYER_INPUT_NORM; else hidden[n])
 *   q[n]   = x . q_proj^T                                    ([H, dn + dr])
 *   [c | k] = x . kv_a_proj^T,  split at dc
 *   mla_cache_write(c, k, positions[n], slot_mapping[n])     (kv_a_layernorm, RoPE, scatter)
 *   a[n]   = mla_decode(q)[n]                                ([H, dv], the absorbed attention)
 *   out[n] = a[n] . o_proj^T (+ hidden[n] with MLA_LAYER_RESIDUAL)
 * Intermediate values: q is rounded to bf16 (the query mla_decode takes), c and k stay fp32 until the
 * cache row is evaluated in fp64 and rounded once, a is rounded to bf16; out is bf16 (nearest even).
 *
 *  hidden                    device bf16 [N, D]
 *  positions, slot_mapping   device int32 [N]: RoPE position and cache slot of each new token (as
 *                            mla_cache_write; position ctx_b - q_len + i for the decode to be causal)
 *  batch, q_len, kv_cache, num_blocks, block_table, block_table_stride, seq_lens, max_seq_len
 *                            as mla_decode (seq_lens include the new tokens)
 *  out                       device bf16 [N, D]; may be the same buffer as hidden
 * Asynchronous on `stream`, no allocation; the context's workspace is used, so calls on one context
 * must be serialised.  Returns MLA_EINVAL (no layer weights attached, null pointers), and what
 * mla_decode_step returns for the rest.
 */
mla_status mla_layer_decode_step(mla_ctx* ctx, const void* hidden, const int32_t* positions,
                                 const int32_t* slot_mapping, int32_t batch, int32_t q_len, void* kv_cache,
                                 int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                                 const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream);

/*
 * mla_prefill -- chunked prefill over the latent cache, naive form: K and V are expanded from the
 * cached latent once per chunk and the new tokens attend to them causally, MHA-style.  The pages'
 * naive MLA ([P-mini] MLA 的数学结构 and 版本 1: K_nope = C W_uk^T, V = C W_uv^T per head, K_pe
 * shared by all heads) with the causal mask of [P-mini] 踩坑记录 坑 2, over the paged cache of
 * [P-vllm] §2.3 and the block table of [P-hybrid] §2.1:
 *   out[i, h] = softmax_{t <= p_i}(scale (q_nope . K_nope[t, h] + RoPE(q_pe, p_i) . k_pe_t)) V[t, h]
 * Sequence b's n_b = cu_q_lens[b+1] - cu_q_lens[b] new tokens sit at positions ctx_b - n_b ..
 * ctx_b - 1 and must already be in the cache (mla_cache_write), as for mla_decode.  bf16 contexts
 * (MLA_BF16 and MLA_BF16_FP8) only; over FP8 rows the latent values are the dequantised ones,
 * code x group scale, here rounded once to bf16 (the decode applies the scales to its fp32 results).
 *
 *  q           device bf16 [total_q, H, dn + dr], un-rotated queries, rows in sequence order
 *  cu_q_lens   device int32 [batch + 1], prefix sums of the chunk lengths (cu_q_lens[0] = 0,
 *              cu_q_lens[batch] = total_q); every chunk length must be <= max_q_len
 *  kv_cache .. max_seq_len   as in mla_decode (seq_lens[b] = ctx_b, the chunk included)
 *  workspace   device memory of at least mla_prefill_workspace_size(...) bytes, caller-owned;
 *              its contents on entry do not matter and are overwritten
 *  out         device bf16 [total_q, H, dv]
 * Asynchronous on `stream`; no host synchronisation and no allocation.  Device-resident values are
 * trusted like mla_decode's; a chunk whose prefix sums are inconsistent is skipped (its rows are not
 * written).  Returns MLA_EINVAL (null pointer, batch < 1, total_q < 1, max_q_len < 1,
 * max_seq_len < max_q_len, num_blocks <= 0, stride smaller than ceil(max_seq_len/16), workspace too
 * small), MLA_EUNSUPPORTED (an MLA_F32 context), MLA_ECAP (max_seq_len - 1 >
 * max_position), MLA_EHIP.
 */
mla_status mla_prefill(mla_ctx* ctx, const void* q, const int32_t* cu_q_lens, int32_t batch, int32_t total_q,
                       int32_t max_q_len, const void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                       int32_t block_table_stride, const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                       size_t workspace_bytes, void* out, void* stream);

/* Bytes of workspace mla_prefill needs for `batch` sequences of contexts up to max_seq_len tokens
 * and total_q new tokens: the expanded rows [K_nope | k_pe | V], batch * H * ceil1024(max_seq_len)
 * * 320 bf16, then the rotated q_pe, total_q * H * 64 bf16, then, for an FP8 cache (MLA_BF16_FP8),
 * the context rows dequantised to bf16, batch * ceil1024(max_seq_len) * 576 bf16.  MLA_EINVAL for a
 * null pointer or a size < 1. */
mla_status mla_prefill_workspace_size(const mla_ctx* ctx, int32_t batch, int32_t total_q, int32_t max_seq_len,
                                      size_t* bytes);

/*
 * mla_free -- synchronises the device, then releases everything the context owns.
 * NULL is accepted.  Using the context afterwards is undefined.
 */
void mla_free(mla_ctx* ctx);

/* ------------------------------------------------------------------------------------------
 * Inspection and tuning helpers (not part of the compute path).
 * ------------------------------------------------------------------------------------------ */

/* Human-readable name of a status code (static string). */
const char* mla_status_string(int32_t status);

/* Force the decode launch shape for subsequent decodes: split size in 16-token blocks and
 * waves per workgroup of the 16-row kernels (2; the FP8-cache kernel also 4, its default);
 * 0 keeps the automatic choice for each.
 * For the 32-row bf16 kernel the split size is read as its workgroup count.
 * Any split size gives the same result up to fp32 summation order.  Returns MLA_EINVAL for a
 * negative split size or an unsupported wave count. */
mla_status mla_set_decode_tuning(mla_ctx* ctx, int32_t split_blocks, int32_t waves_per_group);

/* Launch shape of the most recent decode: split size in blocks, number of splits launched
 * (grid x) and waves per workgroup.  Any pointer may be NULL. */
mla_status mla_last_decode_shape(const mla_ctx* ctx, int32_t* split_blocks, int32_t* n_split,
                                 int32_t* waves_per_group);

/* Kernel timing with HIP events recorded on the launch stream around each kernel.
 * enable != 0 starts recording (clears the totals); 0 stops.  Kernel ids: */
enum {
  MLA_K_CACHE_WRITE = 0,
  MLA_K_Q_ABSORB = 1,
  MLA_K_DECODE = 2,
  MLA_K_COMBINE = 3,
  MLA_K_PF_EXPAND = 4, /* mla_prefill: K/V expansion */
  MLA_K_PF_ATTN = 5,   /* mla_prefill: causal attention (queries prepared in it) */
  MLA_K_PREP = 6,      /* mla_decode_step: cache write and query absorption in one launch */
  MLA_K_LAYER_QKV = 7, /* mla_layer_decode_step: input norm, q_proj and kv_a_proj */
  MLA_K_LAYER_O = 8,   /* mla_layer_decode_step: o_proj and the residual */
  MLA_K_COUNT = 9
};
mla_status mla_profile_enable(mla_ctx* ctx, int32_t enable);
/* Synchronises the recorded events and returns the summed milliseconds and launch count of
 * kernel `kernel_id` since profiling was enabled. */
mla_status mla_profile_read(mla_ctx* ctx, int32_t kernel_id, double* total_ms, int64_t* launches);
/* Synchronises the recorded events and copies the durations (ms) of the most recent launches of
 * kernel `kernel_id` (at most 1024 are kept, and at most `max` are copied, oldest first) to the
 * host array `ms`; *n receives the number copied.  MLA_EINVAL for a bad id, max < 0, or NULL ms
 * with max > 0. */
mla_status mla_profile_samples(mla_ctx* ctx, int32_t kernel_id, float* ms, int32_t max, int32_t* n);

/* ------------------------------------------------------------------------------------------
 * Measurement kernels (not part of the compute path): the practical ceilings of the decode's
 * latent-cache stream and of the matrix cores on this device.
 * ------------------------------------------------------------------------------------------ */

/* A plain streaming read of `bytes` (a positive multiple of 16) contiguous device bytes at `src` by
 * 1,024 workgroups of 256 threads, each reading a contiguous range 32 KiB at a time (eight 16-byte
 * loads per thread in flight); each thread writes one word to `sink` (device, at least 1 MiB) so that
 * the loads are kept.  Asynchronous on `stream`.
 * MLA_EINVAL for a null pointer, a size that is not a positive multiple of 16, or a sink too small. */
mla_status mla_ceiling_read(const void* src, int64_t bytes, void* sink, int64_t sink_bytes, void* stream);

/* The matrix cores' issue rate for one MFMA shape: 1,024 workgroups of four waves (four waves per SIMD),
 * each wave running `iterations` (1 .. 2^20) rounds of independent chains on register operands: shape 0,
 * eight chains of v_mfma_f32_16x16x32_bf16 (the decode's score MFMA); shape 1, four chains of
 * v_mfma_f32_32x32x16_bf16.  Either way a round is 8 x 2 x 16 x 16 x 32 flops per wave; *flops (if not NULL)
 * receives the launch's count, 1,024 x 4 x iterations x 8 x 2 x 16 x 16 x 32.  `sink` (device, at least
 * 1 MiB) receives one word per thread.  Asynchronous on `stream`.  MLA_EINVAL for a null sink, a sink too
 * small, an unknown shape or an iteration count out of range. */
mla_status mla_ceiling_mfma(int32_t shape, int32_t iterations, void* sink, int64_t sink_bytes, double* flops,
                            void* stream);

/* The data movement of mla_decode's 16-row bf16 decode kernel and nothing else, for the decode those
 * arguments describe (same split, work units, unit order, waves, LDS ring and zero-block substitution):
 * every visible latent-cache block is moved HBM -> LDS by global_load_lds_dwordx4 and read once from LDS;
 * no MFMA, softmax or partial store.  `sink` (device, at least 512 bytes per workgroup: 128 KiB covers
 * 256 workgroups) receives one word per thread.  bf16 contexts whose decode shape runs the 16-row
 * kernel only (MLA_EUNSUPPORTED otherwise); MLA_EINVAL / MLA_ECAP as mla_decode for the rest. */
mla_status mla_ceiling_gather(mla_ctx* ctx, int32_t batch, int32_t q_len, const void* kv_cache, int32_t num_blocks,
                              const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                              int32_t max_seq_len, void* sink, int64_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
