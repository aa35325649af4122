"""Plain fp64 oracle of one MLA attention layer's decode step from hidden states, and of a decode step
through a stack of such layers.

TEST INFRASTRUCTURE ONLY, like mla_oracle.py: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It depends on NumPy and mla_oracle alone
and shares no code with the HIP library.

Sources (cited by page title and section):

* [P-vllm]  vLLM learning book, ch. 07 "模型架构特异：MLA / Mamba / MoE 在 vLLM 源码层"
  - §2.2 vLLM 源码挂载点: the MLA wrapper's forward takes hidden states, positions and the cache:
    1. down-projection to c_kv, 2. decoupled RoPE, 3. c_kv written to the cache by slot_mapping,
    4. attention (up-projection inside), returning the layer output.
  - the DeepseekV3DecoderLayer listing: residual = h; h = input_layernorm(h); h = self_attn(h);
    h = residual + h; then the MLP / MoE half (not part of this path).
* [P-mini]  mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收"
  - "MLA 的数学结构": C_KV = X W_dkv; K_pe = RoPE(X W_kr), one rope key shared by all heads.
  - 版本 1: kv_a_proj_with_mqa(hidden) gives [compressed_kv | k_pe], split at kv_lora_rank; the
    kv_a_layernorm acts on compressed_kv; the weight path is q_proj, kv_a_proj, kv_b_proj, o_proj.
  - 版本 3: W_uk and W_uv come from kv_b_proj; attention is computed from the normed latent.
  - 踩坑记录 坑 3: dropping kv_a_layernorm changes the output by O(0.1).
* [P-hybrid] bxzpzcl.cn, KV-cache management for hybrid (GDN/KDA) models
  - §2.1 当前逻辑: one cache per layer, pages shared by all requests, a block table per request.

Readings taken where the pages are silent:

* q_proj maps hidden (D) straight to H * (dn + dr) query values, per head [nope | rope]: the
  DeepSeek-V2-Lite shape (the pages name q_proj and no query low-rank step).
* kv_a_proj_with_mqa maps D to dc + dr = 576: [compressed_kv (dc) | k_pe (dr)].
* o_proj maps the concatenated head outputs (H * dv, head-major) to D: out = A W_o^T.
* input_layernorm is an RMSNorm over D with its own gamma and the same epsilon as kv_a_layernorm.
* The new tokens of a sequence sit at the positions the caller passes; their rows are written to the
  cache before the attention reads it (as for mla_decode: seq_lens include them).

Every value is float64.  The only storage rounding is that of the cache rows (mla_oracle.cache_write).
"""

from __future__ import annotations

import numpy as np

from . import mla_oracle as O


def layer_decode_step(hidden, positions, slot_mapping, cache, block_table, seq_lens, q_len, weights, *,
                      input_norm=True, residual=True, attention="absorbed", kv_norm=True):
    """One decode step of one attention layer.

    hidden        : [N, D] hidden states of the N = batch * q_len new tokens (row b*q_len + i)
    positions     : [N] RoPE positions of the new tokens
    slot_mapping  : [N] cache slots of the new tokens
    cache         : [n_blocks, block, 1, dc + dr] latent cache before the step (history written)
    block_table, seq_lens, q_len : as mla_oracle.decode_absorbed (seq_lens include the new tokens)
    weights       : dict with q_proj [H*(dn+dr), D], kv_a_proj [dc+dr, D], kv_b_proj [H*(dn+dv), dc],
                    kv_norm_gamma [dc], o_proj [D, H*dv], input_norm_gamma [D], num_heads, eps, theta,
                    scale, storage ("bf16" or "f32": the cache rows' rounding)
    input_norm    : apply input_layernorm to hidden first (the decoder layer); False: the bare module
    residual      : add hidden to the output (the decoder layer's residual); False: the bare module
    attention     : "absorbed" ([P-mini] 版本 3) or "naive" (K and V expanded, [P-mini] 版本 1)
    kv_norm       : False drops kv_a_layernorm (the mistake of [P-mini] 坑 3), for the negative pin
    returns (out [N, D], cache after the step)
    """
    w = weights
    H = int(w["num_heads"])
    h = np.asarray(hidden, dtype=np.float64)
    x = O.rms_norm(h, w["input_norm_gamma"], w["eps"]) if input_norm else h
    q = (x @ np.asarray(w["q_proj"], dtype=np.float64).T).reshape(h.shape[0], H, -1)     # [N, H, dn + dr]
    kv = x @ np.asarray(w["kv_a_proj"], dtype=np.float64).T                              # [N, dc + dr]
    kvb = np.asarray(w["kv_b_proj"], dtype=np.float64)
    dc = kvb.shape[1]
    c_raw, k_raw = kv[:, :dc], kv[:, dc:]
    gamma = np.asarray(w["kv_norm_gamma"], dtype=np.float64)
    if kv_norm:
        cache = O.cache_write(cache, c_raw, k_raw, positions, slot_mapping, gamma, w["eps"], w["theta"],
                              w["storage"])
    else:  # the latent stored without its norm (rounded like a cache row), the rope part as usual
        rnd = O.round_to_bf16 if w["storage"] == "bf16" else O.round_to_f32
        cache = np.array(cache, dtype=np.float64, copy=True)
        rows = np.concatenate([rnd(c_raw), rnd(O.rope(k_raw, np.asarray(positions), w["theta"]))], axis=1)
        bs = cache.shape[1]
        for j, s in enumerate(slot_mapping):
            if s >= 0:
                cache[s // bs, s % bs, 0, :] = rows[j]
    dn = q.shape[2] - k_raw.shape[1]
    dv = kvb.shape[0] // H - dn
    W_uk, W_uv = O.absorb(kvb, H, dn, dv)
    dec = O.decode_absorbed if attention == "absorbed" else O.decode_naive
    a = dec(q, cache, block_table, seq_lens, q_len, W_uk, W_uv, w["scale"], w["theta"])   # [N, H, dv]
    out = a.reshape(a.shape[0], H * dv) @ np.asarray(w["o_proj"], dtype=np.float64).T      # [N, D]
    if residual:
        out = out + h
    return out, cache


def folded_query_weights(weights):
    """W_uk folded into q_proj (the absorption of the DeepSeek-V2 report that [P-mini] 版本 3 cites):
    per head, the [D, dc] matrix Wq_nope[h]^T W_uk[h], so that q_lat[h] = x . Wqk[h] in one product."""
    w = weights
    H = int(w["num_heads"])
    Wq = np.asarray(w["q_proj"], dtype=np.float64)
    kvb = np.asarray(w["kv_b_proj"], dtype=np.float64)
    dc = kvb.shape[1]
    dr = np.asarray(w["kv_a_proj"]).shape[0] - dc
    dn = Wq.shape[0] // H - dr
    W_uk, _ = O.absorb(kvb, H, dn, kvb.shape[0] // H - dn)
    Wq = Wq.reshape(H, dn + dr, -1)
    return np.stack([Wq[hh, :dn, :].T @ W_uk[hh] for hh in range(H)])                   # [H, D, dc]


def folded_output_weights(weights):
    """W_uv folded into o_proj: per head, the [dc, D] matrix W_uv[h]^T Wo_h^T, so that
    out = sum_h o_lat[h] . Wvo[h]."""
    w = weights
    H = int(w["num_heads"])
    kvb = np.asarray(w["kv_b_proj"], dtype=np.float64)
    Wo = np.asarray(w["o_proj"], dtype=np.float64)
    dv = Wo.shape[1] // H
    dn = kvb.shape[0] // H - dv
    _, W_uv = O.absorb(kvb, H, dn, dv)
    return np.stack([W_uv[hh].T @ Wo[:, hh * dv:(hh + 1) * dv].T for hh in range(H)])     # [H, dc, D]


def model_decode_step(hidden, positions, slot_mapping, caches, block_table, seq_lens, q_len, layers, **kw):
    """A decode step through a stack of attention layers: layer l takes layer l-1's output as its
    hidden states and reads and writes its own cache (one cache per layer, [P-hybrid] §2.1; the
    decoder layer's MLP / MoE half is left out).  Returns (out, [caches after the step])."""
    h = np.asarray(hidden, dtype=np.float64)
    new = []
    for wl, cache in zip(layers, caches):
        h, c = layer_decode_step(h, positions, slot_mapping, cache, block_table, seq_lens, q_len, wl, **kw)
        new.append(c)
    return h, new
