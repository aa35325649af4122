"""Plain, slow fp64 CPU oracle for DeepSeek-V2-style MLA decode over a paged latent cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product path: it depends on NumPy alone.

Sources (cited by page title and section; no line numbers):

* [P-vllm]  vLLM learning book, ch. 07 "模型架构特异：MLA / Mamba / MoE 在 vLLM 源码层"
  - §2.1 算法核心: only the low-rank latent c_kv is cached; K and V are
    re-expanded from it with layer-fixed up-projections.
  - §2.2 vLLM 源码挂载点: the MLA wrapper forward = down-projection, decoupled
    RoPE, cache write by slot_mapping, attention with up-projection.
  - §2.3 与 KV manager 的接缝: MLA cache shape (n_blocks, block, 1, latent_d + rope_d).
  - §2.4 Decoupled RoPE: each head splits into a RoPE part and a no-RoPE part.
* [P-mini]  mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收"
  - "MLA 的数学结构": C_KV = X W_dkv; K_nope = C_KV W_uk; V = C_KV W_uv;
    K_pe is RoPE'd and shared by all heads; K = concat(K_nope, K_pe);
    V2-Lite dims kv_lora_rank 512, qk_rope_head_dim 64; 1,152 B/token/layer.
  - 版本 1 (MLAAttentionNaive): kv_a split [:kv_lora_rank] | [kv_lora_rank:],
    kv_a_layernorm before kv_b_proj, per-head view (nope rows, then v rows).
  - 版本 3 (MLAAttentionAbsorbed): kv_b_proj viewed as (H, d_nope + d_v, d_c);
    the nope rows give W_uk, the v rows give W_uv; scores and output are formed
    from the normed latent.
  - 踩坑记录 坑 2: causal mask = -inf strictly above the diagonal.
  - 踩坑记录 坑 3: the latent must be RMS-normed before absorption.
  - 设计取舍: nope and rope score parts are computed separately and summed.
  - 实验结果, KV Cache 压缩比 table: 2,048 / 10,240 / 1,152 bytes per token per layer.
* [P-hybrid] bxzpzcl.cn, KV-cache management for hybrid (GDN/KDA) models
  - §2.1 当前逻辑: paged physical pages shared by all requests, one cache per
    layer, a block table maps logical to physical blocks.
  - §2.3 cache的存储大小对比: MLA cache bytes = 2 * seq_len * (kv_lora_rank + qk_rope_head_dim).

Readings taken where the pages are silent:

* RoPE: interleaved consecutive pairs (x[2i], x[2i+1]) rotated by p * theta^(-2i/d_rope)
  (the RoFormer formulation); the pages never define the pairing.
* RMSNorm: x / sqrt(mean(x^2) + eps) * gamma, eps inside the root.
* The cache stores the RMS-normed latent and the RoPE'd k_pe ([P-mini] 设计取舍 stores
  the raw latent and norms at attention time; the two are equivalent).
* A decode query i of a sequence with context length ctx (which already includes
  the q_len new tokens) sits at position ctx - q_len + i and sees cache tokens
  t <= that position.
* q_pe is RoPE'd inside decode at the query position.
* softmax scale = 1/sqrt(qk_nope_head_dim + qk_rope_head_dim).
* slot = physical_block * block_size + offset; a negative slot is skipped.

Every function works in float64.  Storage rounding (to bf16 or fp32) is
round-to-nearest-even of the exact fp64 value, applied once.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "round_to_bf16",
    "round_to_f32",
    "absorb",
    "rms_norm",
    "rope",
    "cache_write",
    "gather_sequence",
    "query_positions",
    "softmax",
    "decode_naive",
    "decode_absorbed",
    "split_partials",
    "combine_partials",
    "decode_absorbed_split",
    "latent_bytes_per_token",
    "naive_bytes_per_token",
    "gqa_bytes_per_token",
    "mla_cache_bytes",
]


# ----------------------------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------------------------

def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and the fp32 exponent range.  For a normal value
    x = m * 2**e with 0.5 <= |m| < 1, the bf16 neighbours are multiples of 2**(e-8);
    below the smallest normal 2**-126 the spacing is fixed at 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    m, e = np.frexp(xf)                       # xf = m * 2**e, 0.5 <= |m| < 1
    e = e.astype(np.int64)
    # exponent of the spacing: normal -> e - 8, subnormal range -> -133
    spacing_exp = np.maximum(e - 8, -133)
    scaled = np.ldexp(xf, -spacing_exp)       # exact (power-of-two scaling)
    r = np.rint(scaled)                       # numpy rint rounds half to even
    y = np.ldexp(r, spacing_exp)
    bf16_max = float.fromhex("0x1.fep127")
    y = np.where(np.abs(y) > bf16_max, np.copysign(np.inf, y), y)
    out[finite] = y
    return out


def round_to_f32(x):
    """Round float64 values to the nearest float32 value (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# S0: weight absorption split ([P-mini] 版本 3, _build_absorbed; 版本 1 per-head view)
# ----------------------------------------------------------------------------------------------

def absorb(kv_b_proj, num_heads, qk_nope_head_dim, v_head_dim):
    """Split kv_b_proj [H*(dn+dv), dc] into W_uk [H, dn, dc] and W_uv [H, dv, dc].

    Row block h of kv_b_proj holds dn "nope" rows followed by dv "value" rows
    ([P-mini] 版本 1 view(bsz, q_len, H, dn + dv) and 版本 3 view(H, dn + dv, dc)).
    K_nope[t, h, :] = W_uk[h] @ c[t]  and  V[t, h, :] = W_uv[h] @ c[t].
    """
    W = np.asarray(kv_b_proj, dtype=np.float64)
    H, dn, dv = num_heads, qk_nope_head_dim, v_head_dim
    dc = W.shape[1]
    if W.shape[0] != H * (dn + dv):
        raise ValueError("kv_b_proj must have H*(dn+dv) rows")
    W = W.reshape(H, dn + dv, dc)
    return W[:, :dn, :].copy(), W[:, dn:, :].copy()


# ----------------------------------------------------------------------------------------------
# S1 pieces: RMSNorm and RoPE
# ----------------------------------------------------------------------------------------------

def rms_norm(x, gamma, eps):
    """kv_a_layernorm as an RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope(x, positions, theta):
    """Rotary embedding on the last axis (length d, even) with interleaved pairs.

    Pair i = (x[2i], x[2i+1]) is rotated by the angle p * theta**(-2i/d), where p is
    the token position.  ``positions`` broadcasts against x.shape[:-1].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / d)                 # [d/2]
    p = np.asarray(positions, dtype=np.float64)[..., None]          # [..., 1]
    ang = p * inv_freq                                              # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------------------------
# S1: cache write ([P-vllm] §2.2 steps 2-3, §2.3 cache shape; [P-mini] 版本 1 kv_a split, 坑 3)
# ----------------------------------------------------------------------------------------------

def cache_write(cache, c_kv, k_pe, positions, slot_mapping, gamma, eps, theta, storage):
    """Write new tokens into a copy of the paged latent cache and return it.

    cache        : [n_blocks, block_size, 1, dc + dr] float64 (values of the storage dtype)
    c_kv, k_pe   : [T, dc], [T, dr] raw latent and un-rotated rope key
    positions    : [T] token positions (for RoPE)
    slot_mapping : [T] slot = block * block_size + offset; negative -> skipped
    storage      : "bf16" or "f32" -- the row [rms_norm(c_kv) | rope(k_pe)] is rounded once.
    Untouched slots keep their previous contents.
    """
    out = np.array(cache, dtype=np.float64, copy=True)
    n_blocks, block_size, _, width = out.shape
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    dc = c_kv.shape[1]
    if width != dc + k_pe.shape[1]:
        raise ValueError("cache row width must be kv_lora_rank + qk_rope_head_dim")
    rnd = round_to_bf16 if storage == "bf16" else round_to_f32
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    idx = np.nonzero(slots >= 0)[0]
    if np.any(slots[idx] // block_size >= n_blocks):
        raise IndexError("slot outside the cache pool")
    # a slot written twice keeps the later token: store only each slot's last writer
    _, last = np.unique(slots[idx][::-1], return_index=True)
    idx = idx[len(idx) - 1 - last]
    positions = np.asarray(positions).reshape(-1)
    flat = out.reshape(-1, width)
    # RMSNorm and RoPE act on each row on its own: many rows at a time, in batches that bound the
    # temporaries
    for lo in range(0, len(idx), 8192):
        j = idx[lo:lo + 8192]
        flat[slots[j]] = np.concatenate([rnd(rms_norm(c_kv[j], gamma, eps)), rnd(rope(k_pe[j], positions[j], theta))],
                                        axis=1)
    return out


# ----------------------------------------------------------------------------------------------
# Paged gather ([P-hybrid] §2.1 logical -> physical through the block table)
# ----------------------------------------------------------------------------------------------

def gather_sequence(cache, block_table_row, ctx, dc):
    """Return the logical latent rows C [ctx, dc] and rope keys R [ctx, dr] of one sequence:
    token t is row t % block_size of physical block block_table_row[t // block_size]."""
    cache = np.asarray(cache, dtype=np.float64)
    block_size = cache.shape[1]
    t = np.arange(ctx)
    blk = np.asarray(block_table_row)[t // block_size].astype(np.int64)
    rows = cache[blk, t % block_size, 0, :]
    return rows[:, :dc], rows[:, dc:]


def query_positions(ctx, q_len):
    """Positions of the q_len new tokens of a sequence whose context (incl. them) is ctx."""
    return np.arange(ctx - q_len, ctx, dtype=np.int64)


def softmax(s):
    """Max-shifted softmax over the last axis; -inf entries get weight 0."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _causal_scores_mask(ctx, pos):
    """True where cache token t is visible to a query at position pos ([P-mini] 坑 2)."""
    return np.arange(ctx) <= pos


# ----------------------------------------------------------------------------------------------
# Decode, naive form ([P-mini] MLA 的数学结构 + 版本 1): expand K and V explicitly
# ----------------------------------------------------------------------------------------------

def decode_naive(q, cache, block_table, seq_lens, q_len, W_uk, W_uv, scale, theta):
    """Causal softmax attention with K = [C W_uk^T | R] and V = C W_uv^T expanded per head.

    q           : [B*q_len, H, dn + dr] un-rotated queries ([nope | rope] per head)
    cache       : [n_blocks, block, 1, dc + dr] (already written)
    block_table : [B, max_blocks] physical block ids
    seq_lens    : [B] context length ctx_b including the q_len new tokens
    returns out : [B*q_len, H, dv] float64
    """
    q = np.asarray(q, dtype=np.float64)
    H, dn, dc = W_uk.shape
    dv = W_uv.shape[1]
    B = len(seq_lens)
    out = np.zeros((B * q_len, H, dv), dtype=np.float64)
    for b in range(B):
        ctx = int(seq_lens[b])
        C, R = gather_sequence(cache, block_table[b], ctx, dc)
        for i in range(q_len):
            pos = ctx - q_len + i
            vis = _causal_scores_mask(ctx, pos)
            row = b * q_len + i
            for h in range(H):
                K_nope = C @ W_uk[h].T                     # [ctx, dn]
                V = C @ W_uv[h].T                          # [ctx, dv]
                K = np.concatenate([K_nope, R], axis=1)    # [ctx, dn + dr]
                qn = q[row, h, :dn]
                qr = rope(q[row, h, dn:], pos, theta)
                qf = np.concatenate([qn, qr])
                s = scale * (K @ qf)
                s = np.where(vis, s, -np.inf)
                out[row, h] = softmax(s) @ V
    return out


def prefill_naive(q, cu_q_lens, cache, block_table, seq_lens, W_uk, W_uv, scale, theta):
    """Chunked prefill in the naive form: K = [C W_uk^T | R] and V = C W_uv^T expanded once per
    sequence and head ([P-mini] MLA 的数学结构 and 版本 1), causal softmax attention of every new
    token over the cache ([P-mini] 踩坑记录 坑 2).

    Sequence b owns query rows cu_q_lens[b] .. cu_q_lens[b+1]-1: its n_b new tokens, at positions
    ctx_b - n_b .. ctx_b - 1, whose rows are already in the cache (as for the decode).  Row i of the
    chunk sees cache tokens t <= its position.  Same inputs and output layout as decode_naive, with
    per-sequence chunk lengths instead of one q_len.

    q          : [total_q, H, dn + dr] un-rotated queries
    cu_q_lens  : [B + 1] prefix sums of the chunk lengths
    seq_lens   : [B] context length ctx_b including the chunk
    returns    : [total_q, H, dv] float64
    """
    q = np.asarray(q, dtype=np.float64)
    H, dn, dc = W_uk.shape
    dv = W_uv.shape[1]
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    out = np.zeros((int(cu[-1]), H, dv), dtype=np.float64)
    for b in range(len(seq_lens)):
        ctx = int(seq_lens[b])
        r0, r1 = int(cu[b]), int(cu[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        C, R = gather_sequence(cache, block_table[b], ctx, dc)
        pos = query_positions(ctx, n)                                   # [n]
        vis = np.arange(ctx)[None, :] <= pos[:, None]                   # [n, ctx]
        for h in range(H):
            K = np.concatenate([C @ W_uk[h].T, R], axis=1)              # [ctx, dn + dr]
            V = C @ W_uv[h].T                                           # [ctx, dv]
            Q = np.concatenate([q[r0:r1, h, :dn], rope(q[r0:r1, h, dn:], pos, theta)], axis=1)
            S = np.where(vis, scale * (Q @ K.T), -np.inf)                # [n, ctx]
            out[r0:r1, h] = softmax(S) @ V
    return out


# ----------------------------------------------------------------------------------------------
# Decode, absorbed form ([P-mini] 版本 3 reassociated; 设计取舍 two-part score)
# ----------------------------------------------------------------------------------------------

def _absorbed_scores(q_row_h, C, R, W_uk_h, pos, scale, theta):
    dn = W_uk_h.shape[0]
    q_lat = q_row_h[:dn] @ W_uk_h                          # [dc]: q_nope folded through W_uk
    qr = rope(q_row_h[dn:], pos, theta)
    return scale * (C @ q_lat + R @ qr)                    # nope part + rope part


def decode_absorbed(q, cache, block_table, seq_lens, q_len, W_uk, W_uv, scale, theta):
    """Same result as decode_naive, computed from the latent: q_lat = q_nope W_uk,
    s_t = scale (q_lat . c_t + q_pe' . k_pe_t), o_lat = P C, out = o_lat W_uv^T."""
    q = np.asarray(q, dtype=np.float64)
    H, dn, dc = W_uk.shape
    dv = W_uv.shape[1]
    B = len(seq_lens)
    out = np.zeros((B * q_len, H, dv), dtype=np.float64)
    for b in range(B):
        ctx = int(seq_lens[b])
        C, R = gather_sequence(cache, block_table[b], ctx, dc)
        for i in range(q_len):
            pos = ctx - q_len + i
            vis = _causal_scores_mask(ctx, pos)
            row = b * q_len + i
            for h in range(H):
                s = _absorbed_scores(q[row, h], C, R, W_uk[h], pos, scale, theta)
                s = np.where(vis, s, -np.inf)
                o_lat = softmax(s) @ C                     # [dc]
                out[row, h] = W_uv[h] @ o_lat              # [dv]
    return out


# ----------------------------------------------------------------------------------------------
# Split-KV partials and their log-sum-exp combine (a reassociation of the softmax sum)
# ----------------------------------------------------------------------------------------------

def split_partials(s, C, bounds):
    """For score vector s [ctx] (masked entries -inf) and latent rows C [ctx, dc], return one
    (m, l, acc) per split [lo, hi): m = max s, l = sum exp(s - m), acc = sum exp(s - m) c_t.
    A split with no visible token gives m = -inf, l = 0, acc = 0."""
    parts = []
    for lo, hi in bounds:
        seg = s[lo:hi]
        if seg.size == 0 or not np.any(np.isfinite(seg)):
            parts.append((-np.inf, 0.0, np.zeros(C.shape[1])))
            continue
        m = np.max(seg)
        w = np.exp(seg - m)
        parts.append((m, float(np.sum(w)), w @ C[lo:hi]))
    return parts


def combine_partials(parts):
    """o_lat = sum_j e^(m_j - M) acc_j / sum_j e^(m_j - M) l_j with M = max_j m_j."""
    M = max(p[0] for p in parts)
    num = sum(np.exp(p[0] - M) * p[2] for p in parts if np.isfinite(p[0]))
    den = sum(np.exp(p[0] - M) * p[1] for p in parts if np.isfinite(p[0]))
    return num / den


def decode_absorbed_split(q, cache, block_table, seq_lens, q_len, W_uk, W_uv, scale, theta,
                          split_bounds):
    """decode_absorbed with the context cut into splits; split_bounds(ctx) -> [(lo, hi), ...]."""
    q = np.asarray(q, dtype=np.float64)
    H, dn, dc = W_uk.shape
    dv = W_uv.shape[1]
    B = len(seq_lens)
    out = np.zeros((B * q_len, H, dv), dtype=np.float64)
    for b in range(B):
        ctx = int(seq_lens[b])
        C, R = gather_sequence(cache, block_table[b], ctx, dc)
        bounds = split_bounds(ctx)
        for i in range(q_len):
            pos = ctx - q_len + i
            vis = _causal_scores_mask(ctx, pos)
            row = b * q_len + i
            for h in range(H):
                s = _absorbed_scores(q[row, h], C, R, W_uk[h], pos, scale, theta)
                s = np.where(vis, s, -np.inf)
                o_lat = combine_partials(split_partials(s, C, bounds))
                out[row, h] = W_uv[h] @ o_lat
    return out


# ----------------------------------------------------------------------------------------------
# Closed forms for cache size ([P-mini] MLA 的数学结构, 版本 1/2, 压缩比 table;
# [P-hybrid] §2.3)
# ----------------------------------------------------------------------------------------------

def latent_bytes_per_token(kv_lora_rank, qk_rope_head_dim, elem_bytes):
    """Bytes per token per layer of the latent cache: one row of (dc + dr) elements."""
    return (kv_lora_rank + qk_rope_head_dim) * elem_bytes


def naive_bytes_per_token(num_heads, qk_nope_head_dim, qk_rope_head_dim, v_head_dim, elem_bytes):
    """Bytes per token per layer when expanded keys (dn + dr) and values (dv) are cached per head."""
    return num_heads * (qk_nope_head_dim + qk_rope_head_dim + v_head_dim) * elem_bytes


def gqa_bytes_per_token(num_kv_heads, head_dim, elem_bytes):
    """Bytes per token per layer of a GQA cache: K and V per kv head."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def mla_cache_bytes(seq_len, kv_lora_rank, qk_rope_head_dim, elem_bytes=2):
    """Cache bytes of one MLA layer for seq_len tokens."""
    return seq_len * latent_bytes_per_token(kv_lora_rank, qk_rope_head_dim, elem_bytes)

