"""Pins of the layer-level oracle (oracle/mla_layer.py) against things other than itself:

* a pure-Python brute force of the whole layer step on tiny dimensions (lists and the math module:
  RMSNorm, the q / kv_a projections, the [:dc] | [dc:] split, RoPE, the cache write, K and V expanded
  per head, softmax without a max shift, o_proj, the residual), in both the decoder-layer form and
  the bare attention module;
* the naive form (K / V expanded, [P-mini] 版本 1) against the absorbed form (版本 3) at layer level;
* W_uk folded into q_proj and W_uv folded into o_proj (the absorption of the DeepSeek-V2 report that
  [P-mini] 版本 3 cites) against the unfolded layer, by associativity;
* closed cases: o_proj = 0 leaves the residual stream unchanged; kv_a_proj = identity exposes the
  split order; RMSNorm's scale invariance at eps = 0; dropping kv_a_layernorm changes the output by
  O(0.1) ([P-mini] 坑 3);
* a stack of layers: one layer equals the layer step; two layers equal the brute force applied
  twice; zero o_proj in every layer leaves the hidden states unchanged.
"""

import math
import struct

import numpy as np

from oracle import mla_layer as L
from oracle import mla_oracle as O


# ------------------------------------------------------------------------------------ tiny problems

def _tiny(seed=0, H=2, D=6, dc=4, dr=2, dn=2, dv=3, bs=2, ctxs=(5, 3), q_len=1, storage="f32"):
    """A tiny layer problem with arbitrary (small) dimensions, histories written into a pool."""
    rng = np.random.default_rng(seed)
    B = len(ctxs)
    nbs = [(c + bs - 1) // bs for c in ctxs]
    n_blocks = sum(nbs) + 2
    perm = rng.permutation(n_blocks)
    bt = np.zeros((B, max(nbs)), dtype=np.int64)
    p = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[p:p + nb]
        p += nb
    w = dict(num_heads=H, eps=1e-6, theta=10000.0, scale=1.0 / math.sqrt(dn + dr), storage=storage,
             q_proj=rng.standard_normal((H * (dn + dr), D)) / math.sqrt(D),
             kv_a_proj=rng.standard_normal((dc + dr, D)) / math.sqrt(D),
             kv_b_proj=rng.standard_normal((H * (dn + dv), dc)) / math.sqrt(dc),
             kv_norm_gamma=1 + 0.1 * rng.standard_normal(dc),
             o_proj=rng.standard_normal((D, H * dv)) / math.sqrt(H * dv),
             input_norm_gamma=1 + 0.1 * rng.standard_normal(D))
    cache = np.full((n_blocks, bs, 1, dc + dr), np.nan)
    for b, ctx in enumerate(ctxs):      # history: tokens before the q_len new ones
        hist = ctx - q_len
        t = np.arange(hist)
        cache = O.cache_write(cache, rng.standard_normal((hist, dc)), rng.standard_normal((hist, dr)), t,
                              bt[b, t // bs] * bs + t % bs, w["kv_norm_gamma"], w["eps"], w["theta"], storage)
    hidden = rng.standard_normal((B * q_len, D))
    pos = np.array([ctx - q_len + i for ctx in ctxs for i in range(q_len)])
    slots = np.array([bt[b, int(pp) // bs] * bs + int(pp) % bs for b in range(B) for pp in pos[b * q_len:(b + 1) * q_len]])
    return dict(w=w, cache=cache, bt=bt, seq_lens=np.array(ctxs), q_len=q_len, hidden=hidden, pos=pos, slots=slots,
                dims=(H, D, dc, dr, dn, dv, bs))


def _f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


def _brute_layer(pr, input_norm=True, residual=True, cache=None):
    """The layer step with Python lists and the math module only (fp32 cache rows).  Returns
    (out rows, cache as a dict {(block, offset): row})."""
    H, D, dc, dr, dn, dv, bs = pr["dims"]
    w = pr["w"]
    eps, theta, scale = w["eps"], w["theta"], w["scale"]
    tolist = lambda a: np.asarray(a, dtype=np.float64).tolist()
    Wq, Wkv, Wkvb, Wo = tolist(w["q_proj"]), tolist(w["kv_a_proj"]), tolist(w["kv_b_proj"]), tolist(w["o_proj"])
    g_in, g_kv = tolist(w["input_norm_gamma"]), tolist(w["kv_norm_gamma"])
    if cache is None:
        src = pr["cache"]
        cache = {(bb, o): [float(v) for v in src[bb, o, 0]] for bb in range(src.shape[0]) for o in range(bs)}
    else:
        cache = dict(cache)

    def rope(vals, p):
        out = list(vals)
        for i in range(len(vals) // 2):
            a = p * theta ** (-2.0 * i / len(vals))
            x0, x1 = vals[2 * i], vals[2 * i + 1]
            out[2 * i] = x0 * math.cos(a) - x1 * math.sin(a)
            out[2 * i + 1] = x0 * math.sin(a) + x1 * math.cos(a)
        return out

    def rmsnorm(vals, g):
        ms = sum(v * v for v in vals) / len(vals)
        return [v / math.sqrt(ms + eps) * gg for v, gg in zip(vals, g)]

    hid = tolist(pr["hidden"])
    xs = [rmsnorm(r, g_in) if input_norm else list(r) for r in hid]
    qs = [[sum(x[k] * Wq[n][k] for k in range(D)) for n in range(H * (dn + dr))] for x in xs]
    # cache write of the new tokens: kv_a projection, split at dc, kv_a_layernorm, RoPE, fp32 rows
    for j, x in enumerate(xs):
        kv = [sum(x[k] * Wkv[n][k] for k in range(D)) for n in range(dc + dr)]
        row = rmsnorm(kv[:dc], g_kv) + rope(kv[dc:], int(pr["pos"][j]))
        s = int(pr["slots"][j])
        cache[(s // bs, s % bs)] = [_f32(v) for v in row]
    outs = []
    for b, ctx in enumerate(pr["seq_lens"]):
        ctx = int(ctx)
        toks = [cache[(int(pr["bt"][b][t // bs]), t % bs)] for t in range(ctx)]
        for i in range(pr["q_len"]):
            n = b * pr["q_len"] + i
            p = ctx - pr["q_len"] + i
            a = []
            for hh in range(H):
                rows = Wkvb[hh * (dn + dv):(hh + 1) * (dn + dv)]
                qh = qs[n][hh * (dn + dr):(hh + 1) * (dn + dr)]
                qf = qh[:dn] + rope(qh[dn:], p)
                es, vs = [], []
                for t in range(p + 1):
                    c, r = toks[t][:dc], toks[t][dc:]
                    k_nope = [sum(rows[d][e] * c[e] for e in range(dc)) for d in range(dn)]
                    v = [sum(rows[dn + d][e] * c[e] for e in range(dc)) for d in range(dv)]
                    es.append(math.exp(scale * sum(qq * kk for qq, kk in zip(qf, k_nope + r))))
                    vs.append(v)
                z = sum(es)
                a += [sum(es[t] * vs[t][d] for t in range(p + 1)) / z for d in range(dv)]
            o = [sum(a[k] * Wo[m][k] for k in range(H * dv)) for m in range(D)]
            if residual:
                o = [oo + hh_ for oo, hh_ in zip(o, hid[n])]
            outs.append(o)
    return np.array(outs), cache


# ------------------------------------------------------------------------------------ pins

def test_layer_against_brute_force():
    for seed, q_len, ctxs in ((1, 1, (5, 3)), (2, 2, (6, 2, 9))):
        for input_norm, residual in ((True, True), (False, False)):
            pr = _tiny(seed=seed, q_len=q_len, ctxs=ctxs)
            got, cache = L.layer_decode_step(pr["hidden"], pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"],
                                             q_len, pr["w"], input_norm=input_norm, residual=residual)
            ref, bcache = _brute_layer(pr, input_norm, residual)
            assert np.max(np.abs(got - ref)) < 1e-7, (seed, input_norm, residual, np.max(np.abs(got - ref)))
            for s in pr["slots"]:
                blk, off = divmod(int(s), pr["dims"][6])
                assert np.max(np.abs(cache[blk, off, 0] - np.array(bcache[(blk, off)]))) <= 1e-6


def test_layer_naive_equals_absorbed():
    for seed, dims in ((3, {}), (4, dict(H=3, D=16, dc=8, dr=4, dn=4, dv=5, bs=4, ctxs=(9, 17, 4), q_len=2))):
        pr = _tiny(seed=seed, **dims)
        args = (pr["hidden"], pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"], pr["q_len"], pr["w"])
        a, _ = L.layer_decode_step(*args, attention="absorbed")
        n, _ = L.layer_decode_step(*args, attention="naive")
        assert np.max(np.abs(a - n)) < 1e-10


def test_folded_projections_equal_unfolded():
    """q_lat = x . (Wq_nope^T W_uk) per head, and out = sum_h o_lat[h] . (W_uv[h]^T Wo_h^T): the layer
    computed through the folded matrices equals the layer step."""
    pr = _tiny(seed=5, H=3, D=16, dc=8, dr=4, dn=4, dv=5, bs=4, ctxs=(9, 17, 4), q_len=2)
    w = pr["w"]
    H, D, dc, dr, dn, dv, bs = pr["dims"]
    ref, cache = L.layer_decode_step(pr["hidden"], pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"],
                                     pr["q_len"], w)
    Wqk = L.folded_query_weights(w)          # [H, D, dc]
    Wvo = L.folded_output_weights(w)         # [H, dc, D]
    Wq = np.asarray(w["q_proj"]).reshape(H, dn + dr, D)
    x = O.rms_norm(pr["hidden"], w["input_norm_gamma"], w["eps"])
    out = np.array(pr["hidden"], dtype=np.float64, copy=True)
    for b, ctx in enumerate(pr["seq_lens"]):
        C, R = O.gather_sequence(cache, pr["bt"][b], int(ctx), dc)
        for i in range(pr["q_len"]):
            n = b * pr["q_len"] + i
            p = int(ctx) - pr["q_len"] + i
            for hh in range(H):
                q_lat = x[n] @ Wqk[hh]
                q_pe = O.rope(Wq[hh, dn:, :] @ x[n], p, w["theta"])
                s = w["scale"] * (C[:p + 1] @ q_lat + R[:p + 1] @ q_pe)
                o_lat = O.softmax(s) @ C[:p + 1]
                out[n] += o_lat @ Wvo[hh]
    assert np.max(np.abs(out - ref)) < 1e-10


def test_zero_o_proj_keeps_the_residual_stream():
    pr = _tiny(seed=6)
    pr["w"]["o_proj"] = np.zeros_like(pr["w"]["o_proj"])
    out, _ = L.layer_decode_step(pr["hidden"], pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"],
                                 pr["q_len"], pr["w"])
    assert np.array_equal(out, pr["hidden"])


def test_kv_a_split_order():
    """kv_a_proj = identity (D = dc + dr) and no input norm: the new cache row is
    [kv_a_layernorm(h[:dc]) | RoPE(h[dc:])], i.e. compressed_kv first, k_pe after ([P-mini] 版本 1)."""
    pr = _tiny(seed=7, D=6, dc=4, dr=2)
    pr["w"]["kv_a_proj"] = np.eye(6)
    _, cache = L.layer_decode_step(pr["hidden"], pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"],
                                   pr["q_len"], pr["w"], input_norm=False)
    for j, s in enumerate(pr["slots"]):
        h = pr["hidden"][j]
        want = np.concatenate([O.rms_norm(h[:4], pr["w"]["kv_norm_gamma"], 1e-6), O.rope(h[4:], pr["pos"][j], 1e4)])
        blk, off = divmod(int(s), 2)
        assert np.array_equal(cache[blk, off, 0], O.round_to_f32(want))


def test_input_norm_scale_invariance():
    pr = _tiny(seed=8)
    pr["w"]["eps"] = 0.0
    args = (pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"], pr["q_len"], pr["w"])
    a, _ = L.layer_decode_step(pr["hidden"], *args, residual=False)
    b, _ = L.layer_decode_step(3.7 * pr["hidden"], *args, residual=False)
    assert np.max(np.abs(a - b)) < 1e-12
    c, _ = L.layer_decode_step(3.7 * pr["hidden"], *args, residual=False, input_norm=False)
    assert np.max(np.abs(a - c)) > 1e-3   # without the norm the scale matters


def test_missing_kv_norm_changes_the_output():
    """[P-mini] 坑 3: leaving out kv_a_layernorm gives a visibly different result (the page measured a
    max diff of 0.165 on real weights).  Here the un-normed latent has RMS about 4."""
    pr = _tiny(seed=9, H=2, D=16, dc=8, dr=4, dn=4, dv=4, bs=4, ctxs=(12, 7))
    pr["w"]["kv_a_proj"] = 4.0 * np.asarray(pr["w"]["kv_a_proj"])
    pr["w"]["kv_norm_gamma"] = np.ones(8)
    # a history written the same way (un-normed) as the new rows would be
    args = (pr["hidden"], pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"], pr["q_len"], pr["w"])
    good, _ = L.layer_decode_step(*args, residual=False)
    bad, _ = L.layer_decode_step(*args, residual=False, kv_norm=False)
    assert np.max(np.abs(good - bad)) > 0.1


def test_model_step_stack():
    pr = _tiny(seed=10)
    w2 = _tiny(seed=11)["w"]
    args = (pr["pos"], pr["slots"], [pr["cache"], pr["cache"]], pr["bt"], pr["seq_lens"], pr["q_len"])
    # one layer is the layer step
    one, c1 = L.model_decode_step(pr["hidden"], args[0], args[1], [pr["cache"]], *args[3:], [pr["w"]])
    ref, rc = L.layer_decode_step(pr["hidden"], pr["pos"], pr["slots"], pr["cache"], pr["bt"], pr["seq_lens"],
                                  pr["q_len"], pr["w"])
    assert np.array_equal(one, ref) and np.array_equal(c1[0], rc, equal_nan=True)
    # two layers against the brute force applied twice (layer 2 on layer 1's output, its own cache)
    two, caches = L.model_decode_step(pr["hidden"], *args, [pr["w"], w2])
    b1, _ = _brute_layer(pr)
    pr2 = dict(pr, w=w2, hidden=b1)
    b2, _ = _brute_layer(pr2)
    assert np.max(np.abs(two - b2)) < 1e-7
    # zero o_proj everywhere: the stack passes the hidden states through; every layer wrote its rows
    z1, z2 = dict(pr["w"], o_proj=np.zeros_like(pr["w"]["o_proj"])), dict(w2, o_proj=np.zeros_like(w2["o_proj"]))
    same, caches = L.model_decode_step(pr["hidden"], *args, [z1, z2])
    assert np.array_equal(same, pr["hidden"])
    for c in caches:
        for s in pr["slots"]:
            assert np.all(np.isfinite(c[int(s) // 2, int(s) % 2, 0]))
