"""Pins for the fp64 oracle against things other than itself: the pages' printed numbers,
closed forms, textbook identities, brute force on tiny inputs, and invariants that a dropped
term, a wrong sign or index, or a transposed operand would break."""

import json
import math
import os

import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import mla_inputs as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers

def _small_problem(rng, H=2, dc=8, dr=4, dn=3, dv=5, ctx_list=(5,), q_len=1, block=4, pool_extra=3):
    """A tiny random problem with generic dims (the oracle is dimension-generic)."""
    B = len(ctx_list)
    need = [(c + block - 1) // block for c in ctx_list]
    n_blocks = sum(need) + pool_extra
    perm = rng.permutation(n_blocks)
    table = np.zeros((B, max(need)), dtype=np.int64)
    pos = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    cache = np.full((n_blocks, block, 1, dc + dr), np.nan)
    for b, ctx in enumerate(ctx_list):
        for t in range(ctx):
            cache[table[b, t // block], t % block, 0, :] = rng.standard_normal(dc + dr)
    kvb = rng.standard_normal((H * (dn + dv), dc)) / math.sqrt(dc)
    W_uk, W_uv = O.absorb(kvb, H, dn, dv)
    q = rng.standard_normal((B * q_len, H, dn + dr))
    return dict(q=q, cache=cache, block_table=table, seq_lens=np.array(ctx_list), q_len=q_len,
                W_uk=W_uk, W_uv=W_uv, scale=1.0 / math.sqrt(dn + dr), theta=10000.0, kvb=kvb,
                dims=(H, dc, dr, dn, dv, block))


def _decode(fn, p, **over):
    args = dict(q=p["q"], cache=p["cache"], block_table=p["block_table"], seq_lens=p["seq_lens"],
                q_len=p["q_len"], W_uk=p["W_uk"], W_uv=p["W_uv"], scale=p["scale"], theta=p["theta"])
    args.update(over)
    return fn(**args)


# ----------------------------------------------------------------------------- storage rounding

def test_round_to_bf16_ties_and_known_values():
    one = 1.0
    assert O.round_to_bf16(one + 2.0 ** -8) == 1.0                   # tie -> even mantissa
    assert O.round_to_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6    # tie -> even mantissa (up)
    assert O.round_to_bf16(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    assert O.round_to_bf16(-(one + 2.0 ** -8)) == -1.0
    assert O.round_to_bf16(0.0) == 0.0
    assert O.round_to_bf16(2.0 ** -130) == 2.0 ** -130                # subnormal, exact
    assert O.round_to_bf16(3.0 * 2.0 ** -135) == 2.0 ** -133          # subnormal spacing 2^-133 (3/4 of it -> up)
    assert np.isinf(O.round_to_bf16(3.5e38))


def test_round_to_bf16_matches_torch_on_fp32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                        rng.standard_normal(2000) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_bf16(x.astype(np.float64)), ref)


def test_round_to_f32_is_nearest():
    x = 1.0 + 2.0 ** -24          # tie between 1 and 1 + 2^-23 -> even (1.0)
    assert O.round_to_f32(x) == 1.0
    assert O.round_to_f32(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22


# ----------------------------------------------------------------------------- closed forms (pages' numbers)

def test_cache_bytes_match_printed_table():
    g = json.load(open(os.path.join(GOLDEN, "cache_bytes.json")))["bytes_per_token_per_layer"]
    gq, nv, lt = g["gqa_qwen2_5_7b"], g["mla_naive_v2_lite"], g["mla_latent_v2_lite"]
    assert O.gqa_bytes_per_token(gq["num_kv_heads"], gq["head_dim"], gq["elem_bytes"]) == gq["value"]
    assert O.naive_bytes_per_token(nv["num_heads"], nv["qk_nope_head_dim"], nv["qk_rope_head_dim"],
                                   nv["v_head_dim"], nv["elem_bytes"]) == nv["value"]
    lat = O.latent_bytes_per_token(lt["kv_lora_rank"], lt["qk_rope_head_dim"], lt["elem_bytes"])
    assert lat == lt["value"]
    assert lat / gq["value"] == lt["relative_to_gqa"]
    assert nv["value"] / gq["value"] == nv["relative_to_gqa"]
    assert 1 - lat / nv["value"] == pytest.approx(lt["saving_vs_naive"], abs=1e-12)
    # the hybrid page's formula: 2 * seq_len * (kv_lora_rank + qk_rope_head_dim)
    for s in (1, 1024, 4097):
        assert O.mla_cache_bytes(s, 512, 64, 2) == 2 * s * (512 + 64)


def test_concurrency_and_gqa_total_reproduce():
    g = json.load(open(os.path.join(GOLDEN, "cache_bytes.json")))
    mem = 32 * 2 ** 30
    layers = 27
    gqa = O.gqa_bytes_per_token(4, 128, 2) * 1024 * layers
    mla = O.latent_bytes_per_token(512, 64, 2) * 1024 * layers
    assert mem // gqa == g["concurrency_32gb_seq1024"]["gqa"]
    assert mem // mla == g["concurrency_32gb_seq1024"]["mla"]
    assert round((mem // mla) / (mem // gqa), 2) == g["concurrency_32gb_seq1024"]["ratio"]
    assert int(O.gqa_bytes_per_token(4, 128, 2) * 1024 * 28 / 1e6) == g["gqa_28_layers_1024_tokens_mb"]


def test_oracle_cache_tensor_is_1152_bytes_per_token():
    w = W.tiny()
    cache = np.zeros((w.n_blocks, 16, 1, 576), dtype=np.uint16)   # a bf16 pool of the page's shape
    assert cache.nbytes / (w.n_blocks * 16) == 1152


# ----------------------------------------------------------------------------- absorb split

def test_absorb_split_rows():
    H, dn, dv, dc = 3, 2, 4, 5
    kvb = np.arange(H * (dn + dv) * dc, dtype=np.float64).reshape(H * (dn + dv), dc)
    W_uk, W_uv = O.absorb(kvb, H, dn, dv)
    for h in range(H):
        for r in range(dn):
            assert np.array_equal(W_uk[h, r], kvb[h * (dn + dv) + r])
        for r in range(dv):
            assert np.array_equal(W_uv[h, r], kvb[h * (dn + dv) + dn + r])


# ----------------------------------------------------------------------------- RMSNorm and RoPE

def test_rmsnorm_closed_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 512)) * rng.uniform(0.1, 10, size=(7, 1))
    eps = 1e-6
    y = O.rms_norm(x, np.ones(512), eps)
    ms = np.mean(x * x, axis=1)
    rms_y = np.sqrt(np.mean(y * y, axis=1))
    assert np.allclose(rms_y, (1 + eps / ms) ** -0.5, rtol=1e-13, atol=0)
    # gamma multiplies per channel; direction of x is kept
    g = rng.uniform(0.5, 1.5, 512)
    assert np.allclose(O.rms_norm(x, g, eps), y * g, rtol=1e-14)
    assert np.allclose(np.sign(y), np.sign(x))


def test_rope_identity_norm_and_known_angles():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(64)
    assert np.array_equal(O.rope(x, 0, 10000.0), x)
    y = O.rope(x, 123, 10000.0)
    assert np.allclose(y[0::2] ** 2 + y[1::2] ** 2, x[0::2] ** 2 + x[1::2] ** 2, rtol=1e-13)
    # pair 0 has frequency 1: a unit vector on x[0] turns by p radians towards x[1]
    e0 = np.zeros(64); e0[0] = 1.0
    y = O.rope(e0, 1.0, 10000.0)
    assert y[0] == pytest.approx(math.cos(1.0), abs=1e-15) and y[1] == pytest.approx(math.sin(1.0), abs=1e-15)
    assert np.all(y[2:] == 0)
    # pair i has period 2*pi*theta^(2i/64); after one period the pair is back
    for i in (1, 16, 31):
        ei = np.zeros(64); ei[2 * i] = 1.0
        period = 2 * math.pi * 10000.0 ** (2 * i / 64)
        z = O.rope(ei, period, 10000.0)
        assert z[2 * i] == pytest.approx(1.0, abs=1e-9) and abs(z[2 * i + 1]) < 1e-9
        quarter = O.rope(ei, period / 4, 10000.0)
        assert abs(quarter[2 * i]) < 1e-9 and quarter[2 * i + 1] == pytest.approx(1.0, abs=1e-9)


def test_rope_composition_and_relative_positions():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.allclose(O.rope(O.rope(q, 5, 1e4), 11, 1e4), O.rope(q, 16, 1e4), atol=1e-12)
    base = O.rope(q, 40, 1e4) @ O.rope(k, 17, 1e4)
    for d in (1, 100, 3000):
        assert O.rope(q, 40 + d, 1e4) @ O.rope(k, 17 + d, 1e4) == pytest.approx(base, abs=1e-11)


# ----------------------------------------------------------------------------- softmax

def test_softmax_matches_brute_force():
    rng = np.random.default_rng(4)
    for n in (1, 2, 17, 300):
        s = rng.standard_normal(n) * 3
        brute = [math.exp(v) / sum(math.exp(u) for u in s) for v in s]
        assert np.allclose(O.softmax(s), brute, rtol=1e-13, atol=0)
    s = np.array([0.5, -np.inf, 1.0])
    p = O.softmax(s)
    assert p[1] == 0 and p[0] == pytest.approx(math.exp(0.5) / (math.exp(0.5) + math.e), rel=1e-14)


# ----------------------------------------------------------------------------- cache_write

def test_cache_write_places_rows_and_skips_negative_slots():
    rng = np.random.default_rng(5)
    n_blocks, dc, dr = 3, 8, 4
    cache = np.full((n_blocks, 4, 1, dc + dr), 7.0)
    c = rng.standard_normal((3, dc)); k = rng.standard_normal((3, dr))
    pos = np.array([0, 9, 2]); slots = np.array([5, -1, 11])
    out = O.cache_write(cache, c, k, pos, slots, np.ones(dc), 1e-6, 1e4, "f32")
    assert np.array_equal(out[1, 1, 0, :dc], O.round_to_f32(O.rms_norm(c[0], np.ones(dc), 1e-6)))
    assert np.array_equal(out[1, 1, 0, dc:], O.round_to_f32(k[0]))           # position 0: no rotation
    assert np.array_equal(out[2, 3, 0, dc:], O.round_to_f32(O.rope(k[2], 2, 1e4)))
    untouched = np.ones(out.shape[:3], bool); untouched[1, 1, 0] = untouched[2, 3, 0] = False
    assert np.all(out[untouched] == 7.0)


# ----------------------------------------------------------------------------- decode forms

def test_brute_force_attention_tiny():
    """Pure-Python loops over a 2-head, 3-token problem vs the naive and absorbed forms."""
    rng = np.random.default_rng(6)
    p = _small_problem(rng, H=2, dc=4, dr=2, dn=2, dv=3, ctx_list=(3,), block=2)
    H, dc, dr, dn, dv, block = p["dims"]
    kvb, q, cache, table = p["kvb"], p["q"], p["cache"], p["block_table"]
    ctx = 3
    expect = np.zeros((1, H, dv))
    for h in range(H):
        rows = [cache[table[0, t // block], t % block, 0] for t in range(ctx)]
        # K_nope[t][j] = sum_c kvb[h*(dn+dv)+j][c] * c_t[c];  V[t][j] = sum_c kvb[h*(dn+dv)+dn+j][c] * c_t[c]
        K, V = [], []
        for t in range(ctx):
            kn = [sum(kvb[h * (dn + dv) + j][cc] * rows[t][cc] for cc in range(dc)) for j in range(dn)]
            K.append(kn + list(rows[t][dc:]))
            V.append([sum(kvb[h * (dn + dv) + dn + j][cc] * rows[t][cc] for cc in range(dc)) for j in range(dv)])
        pos = ctx - 1
        qr = list(q[0, h, dn:])
        ang = pos * 1.0   # dr = 2: one pair with frequency theta^0 = 1
        qr = [qr[0] * math.cos(ang) - qr[1] * math.sin(ang), qr[0] * math.sin(ang) + qr[1] * math.cos(ang)]
        qf = list(q[0, h, :dn]) + qr
        s = [p["scale"] * sum(qf[j] * K[t][j] for j in range(dn + dr)) for t in range(ctx)]
        e = [math.exp(v) for v in s]
        z = sum(e)
        for j in range(dv):
            expect[0, h, j] = sum(e[t] / z * V[t][j] for t in range(ctx))
    assert np.allclose(_decode(O.decode_naive, p), expect, rtol=1e-12, atol=1e-13)
    assert np.allclose(_decode(O.decode_absorbed, p), expect, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("H,ctxs,q_len", [(1, (1,), 1), (2, (7, 1, 33), 1), (16, (40,), 1),
                                          (2, (4, 17, 9), 4), (3, (12, 30), 2)])
def test_naive_equals_absorbed(H, ctxs, q_len):
    rng = np.random.default_rng(100 + H + q_len)
    p = _small_problem(rng, H=H, dc=16, dr=8, dn=6, dv=5, ctx_list=ctxs, q_len=q_len, block=4)
    a = _decode(O.decode_naive, p)
    b = _decode(O.decode_absorbed, p)
    assert np.max(np.abs(a - b)) <= 1e-10


def test_naive_equals_absorbed_tiny_workload():
    w = W.tiny()
    kvb = w.kv_b_proj().astype(np.float64)
    W_uk, W_uv = O.absorb(kvb, w.num_heads, w.qk_nope_head_dim, w.v_head_dim)
    tok = w.all_tokens()
    cache = O.cache_write(np.full((w.n_blocks, 16, 1, 576), np.nan), tok["c_kv"], tok["k_pe"],
                          tok["positions"], tok["slot_mapping"], w.gamma(), w.eps, w.theta, "f32")
    args = (w.queries(), cache, w.block_table, w.seq_lens, w.q_len, W_uk, W_uv, w.scale, w.theta)
    a, b = O.decode_naive(*args), O.decode_absorbed(*args)
    assert np.max(np.abs(a - b)) <= 1e-10
    assert np.all(np.isfinite(a))


def test_single_token_context_is_value_projection():
    rng = np.random.default_rng(8)
    p = _small_problem(rng, H=3, dc=12, dr=4, dn=5, dv=6, ctx_list=(1,), block=4)
    out = _decode(O.decode_absorbed, p)
    H, dc = p["dims"][0], p["dims"][1]
    c0 = p["cache"][p["block_table"][0, 0], 0, 0, :dc]
    for h in range(H):
        assert np.allclose(out[0, h], p["W_uv"][h] @ c0, rtol=1e-14, atol=1e-15)


def test_zero_query_gives_uniform_average():
    rng = np.random.default_rng(9)
    p = _small_problem(rng, H=2, dc=12, dr=4, dn=5, dv=6, ctx_list=(9, 6), q_len=3, block=4)
    q0 = np.zeros_like(p["q"])
    out = _decode(O.decode_naive, p, q=q0)
    dc = p["dims"][1]
    for b, ctx in enumerate(p["seq_lens"]):
        C, _ = O.gather_sequence(p["cache"], p["block_table"][b], ctx, dc)
        for i in range(3):
            pos = ctx - 3 + i
            mean = C[:pos + 1].mean(axis=0)
            for h in range(2):
                assert np.allclose(out[b * 3 + i, h], p["W_uv"][h] @ mean, rtol=1e-13, atol=1e-14)


def test_paging_relabel_is_bitwise_invariant():
    rng = np.random.default_rng(10)
    p = _small_problem(rng, H=2, dc=16, dr=8, dn=6, dv=5, ctx_list=(13, 22), q_len=2, block=4, pool_extra=5)
    base = _decode(O.decode_absorbed, p)
    n = p["cache"].shape[0]
    perm = rng.permutation(n)             # physical block j moves to perm[j]
    cache2 = np.empty_like(p["cache"])
    cache2[perm] = p["cache"]
    table2 = perm[p["block_table"]]
    out = _decode(O.decode_absorbed, p, cache=cache2, block_table=table2)
    assert np.array_equal(out, base)


def test_split_combine_equals_unsplit():
    rng = np.random.default_rng(11)
    p = _small_problem(rng, H=2, dc=16, dr=8, dn=6, dv=5, ctx_list=(37, 5), q_len=2, block=4)
    base = _decode(O.decode_absorbed, p)
    for cuts in ([0.3, 0.6], [0.1], [0.5, 0.51, 0.9]):
        def bounds(ctx, cuts=cuts):
            pts = [0] + [int(c * ctx) for c in cuts] + [ctx]
            return list(zip(pts[:-1], pts[1:]))
        out = O.decode_absorbed_split(p["q"], p["cache"], p["block_table"], p["seq_lens"], p["q_len"],
                                      p["W_uk"], p["W_uv"], p["scale"], p["theta"], bounds)
        assert np.max(np.abs(out - base)) <= 1e-13


def test_split_with_only_masked_tokens_contributes_nothing():
    s = np.array([1.0, 2.0, -np.inf, -np.inf])
    C = np.arange(8.0).reshape(4, 2)
    parts = O.split_partials(s, C, [(0, 2), (2, 4)])
    assert parts[1][0] == -np.inf and parts[1][1] == 0.0
    assert np.allclose(O.combine_partials(parts), O.softmax(s) @ C, rtol=1e-15)


def test_causal_locality():
    rng = np.random.default_rng(12)
    p = _small_problem(rng, H=2, dc=16, dr=8, dn=6, dv=5, ctx_list=(19,), q_len=4, block=4)
    base = _decode(O.decode_absorbed, p)
    ctx = 19
    dc = p["dims"][1]
    cache2 = p["cache"].copy()
    t = ctx - 1                                  # the last token: only query 3 may see it
    cache2[p["block_table"][0, t // 4], t % 4, 0, :] += 5.0
    out = _decode(O.decode_absorbed, p, cache=cache2)
    assert np.array_equal(out[:3], base[:3])
    assert np.max(np.abs(out[3] - base[3])) > 1e-3
    t = ctx - 3                                  # visible to queries 1, 2, 3, not to 0
    cache3 = p["cache"].copy()
    cache3[p["block_table"][0, t // 4], t % 4, 0, :dc] *= -1.0
    out = _decode(O.decode_absorbed, p, cache=cache3)
    assert np.array_equal(out[0], base[0])
    assert np.all(np.max(np.abs(out[1:] - base[1:]), axis=(1, 2)) > 1e-6)


def test_missing_norm_changes_outputs():
    """Absorbing from an un-normed latent gives a visibly different answer (the pages report
    a max diff of 0.165 on real weights)."""
    w = W.custom("nn", "f32", 16, [40], seed=77)
    kvb = w.kv_b_proj().astype(np.float64)
    W_uk, W_uv = O.absorb(kvb, 16, 128, 128)
    tok = w.all_tokens()
    pool = np.full((w.n_blocks, 16, 1, 576), np.nan)
    normed = O.cache_write(pool, tok["c_kv"] * 3.0, tok["k_pe"], tok["positions"], tok["slot_mapping"],
                           w.gamma(), w.eps, w.theta, "f32")
    raw = normed.copy()
    for j, s in enumerate(tok["slot_mapping"]):
        raw[s // 16, s % 16, 0, :512] = tok["c_kv"][j] * 3.0
    args = (w.queries(), w.block_table, w.seq_lens, 1, W_uk, W_uv, w.scale, w.theta)
    a = O.decode_absorbed(args[0], normed, *args[1:])
    b = O.decode_absorbed(args[0], raw, *args[1:])
    assert np.max(np.abs(a - b)) > 0.1


def test_relative_position_shift_of_whole_sequence():
    """Writing the cache at positions +D and querying at +D leaves the output unchanged."""
    rng = np.random.default_rng(13)
    dc, dr, dn, dv, H = 16, 8, 6, 5, 2
    ctx = 11
    c = rng.standard_normal((ctx, dc)); k = rng.standard_normal((ctx, dr))
    kvb = rng.standard_normal((H * (dn + dv), dc)) / 4
    W_uk, W_uv = O.absorb(kvb, H, dn, dv)
    q = rng.standard_normal((1, H, dn + dr))
    outs = []
    for D in (0, 1000):
        pool = np.full((3, 4, 1, dc + dr), np.nan)
        cache = O.cache_write(pool, c, k, np.arange(ctx) + D, np.arange(ctx), np.ones(dc), 1e-6, 1e4, "f32")
        # decode the same context, with the query also shifted by D: emulate by shifting
        # the rotary angle of q through the absorbed score definition
        C, R = O.gather_sequence(cache, np.arange(3), ctx, dc)
        out = np.zeros((H, dv))
        for h in range(H):
            q_lat = q[0, h, :dn] @ W_uk[h]
            qr = O.rope(q[0, h, dn:], ctx - 1 + D, 1e4)
            s = (C @ q_lat + R @ qr) / math.sqrt(dn + dr)
            out[h] = W_uv[h] @ (O.softmax(s) @ C)
        outs.append(out)
    # the rotated k_pe rows are stored as fp32 (relative rounding <= 2^-24), nothing else differs
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-6


# ----------------------------------------------------------------------------- chunked prefill

def _prefill(p, cu, **over):
    args = dict(q=p["q"], cu_q_lens=cu, cache=p["cache"], block_table=p["block_table"], seq_lens=p["seq_lens"],
                W_uk=p["W_uk"], W_uv=p["W_uv"], scale=p["scale"], theta=p["theta"])
    args.update(over)
    return O.prefill_naive(**args)


@pytest.mark.parametrize("H,ctxs,q_len", [(2, (7, 9, 33), 1), (3, (13, 5), 5), (2, (16,), 16)])
def test_prefill_equals_decode_forms_at_uniform_chunks(H, ctxs, q_len):
    """With every chunk of length q_len, prefill_naive (K and V expanded once per sequence and head,
    the softmax of whole rows) must equal decode_naive (K recomputed per query row) and
    decode_absorbed (no expansion at all)."""
    rng = np.random.default_rng(300 + H + q_len)
    p = _small_problem(rng, H=H, dc=16, dr=8, dn=6, dv=5, ctx_list=ctxs, q_len=q_len, block=4)
    cu = np.arange(len(ctxs) + 1) * q_len
    a = _prefill(p, cu)
    assert np.max(np.abs(a - _decode(O.decode_naive, p))) <= 1e-12
    assert np.max(np.abs(a - _decode(O.decode_absorbed, p))) <= 1e-10


def test_prefill_variable_chunks_equal_per_sequence_decodes():
    """Chunk lengths 5, 0, 1 and 11 (an empty chunk included): each sequence's rows equal
    decode_naive run on that sequence alone with its own q_len, so the row offsets, the
    per-sequence positions and the empty chunk are all checked."""
    rng = np.random.default_rng(310)
    ctxs, lens = (12, 8, 3, 11), (5, 0, 1, 11)
    p = _small_problem(rng, H=2, dc=16, dr=8, dn=6, dv=5, ctx_list=ctxs, q_len=1, block=4)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((int(cu[-1]), 2, 14))
    out = _prefill(p, cu, q=q)
    for b, (ctx, n) in enumerate(zip(ctxs, lens)):
        if n == 0:
            continue
        ref = O.decode_naive(q[cu[b]:cu[b + 1]], p["cache"], p["block_table"][b:b + 1], np.array([ctx]), n,
                             p["W_uk"], p["W_uv"], p["scale"], p["theta"])
        assert np.max(np.abs(out[cu[b]:cu[b + 1]] - ref)) <= 1e-12


def test_prefill_fresh_sequence_first_row_is_value_projection():
    """A chunk that is the whole context: its first row sees only token 0, so its output is
    W_uv c_0 exactly (softmax of a single score), whatever the query."""
    rng = np.random.default_rng(320)
    ctx = 10
    p = _small_problem(rng, H=3, dc=12, dr=4, dn=5, dv=6, ctx_list=(ctx,), q_len=ctx, block=4)
    out = _prefill(p, np.array([0, ctx]))
    dc = p["dims"][1]
    c0 = p["cache"][p["block_table"][0, 0], 0, 0, :dc]
    for h in range(3):
        assert np.allclose(out[0, h], p["W_uv"][h] @ c0, rtol=1e-14, atol=1e-15)


def test_prefill_causal_locality():
    """Changing the chunk's last token changes only the chunk's last row; changing the token at
    position ctx-3 leaves the rows before it unchanged and changes the rows after it."""
    rng = np.random.default_rng(330)
    ctx, n = 21, 6
    p = _small_problem(rng, H=2, dc=16, dr=8, dn=6, dv=5, ctx_list=(ctx,), q_len=n, block=4)
    cu = np.array([0, n])
    base = _prefill(p, cu)
    c2 = p["cache"].copy()
    t = ctx - 1
    c2[p["block_table"][0, t // 4], t % 4, 0, :] += 5.0
    out = _prefill(p, cu, cache=c2)
    assert np.array_equal(out[:n - 1], base[:n - 1])
    assert np.max(np.abs(out[n - 1] - base[n - 1])) > 1e-3
    c3 = p["cache"].copy()
    t = ctx - 3                                  # position of chunk row n - 3
    c3[p["block_table"][0, t // 4], t % 4, 0, :16] *= -1.0
    out = _prefill(p, cu, cache=c3)
    assert np.array_equal(out[:n - 3], base[:n - 3])
    assert np.all(np.max(np.abs(out[n - 3:] - base[n - 3:]), axis=(1, 2)) > 1e-6)
