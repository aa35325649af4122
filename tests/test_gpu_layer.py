"""GPU parity of one attention layer's decode step from hidden states (mla_layer_decode_step, through
the C ABI) against the fp64 layer oracle (oracle/mla_layer.py) on seeded inputs.

Small cases compare every output element and every new cache row: the decoder-layer form (input
RMSNorm, residual) and the bare module, 16 and 32 heads, q_len 1 and 2 (the 16-row and 32-row decode
kernels), input and kv_a_layernorm gammas other than one, an FP8 cache, and two steps in a row (the
second reads the rows the first wrote).  The single-sequence shapes of the pages' latency table
(batch 1, 1 / 256 / 1,024 cached tokens) and the batch-64 x 4,096-token shape run in full; at that
size the oracle takes every sequence on its own blocks of the GPU's history cache.

Tolerances: the output as the decode's bf16 contract (max abs <= 2e-2, relative L2 <= 5e-3), plus half
a bf16 spacing of each value where the residual is added (the output's own rounding); the new cache
rows within two bf16 spacings plus 2^-7 of the row's RMS (they come from an fp32 projection of bf16
operands, whose error scales with the row) and relative L2 <= 5e-3.
"""

import numpy as np
import pytest

from oracle import mla_fp8 as F
from oracle import mla_layer as L
from oracle import mla_oracle as O
from workloads import mla_inputs as W

from ._harness import compare, dev, dev_i32

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_latent_kv_paged_amd import load
    load()


def _say(*a):
    print("[case]", *a, flush=True)


def _weights(w, lw):
    return dict(lw, num_heads=w.num_heads, eps=w.eps, theta=w.theta, scale=w.scale, storage="bf16")


class LayerRun:
    """A layer attached to a context on the GPU; its pool holds the oracle's history rows of every sequence
    (bf16 rows, or FP8 bytes), every other slot NaN (0xFF bytes).  history: the oracle's bf16 history cache,
    if the caller already holds it."""

    def __init__(self, w, lw, input_norm=True, residual=True, cache="bf16", extra_ctx=0, history=None):
        from mla_latent_kv_paged_amd import MLAContext
        self.w = w
        mx = int(w.seq_lens.max()) + extra_ctx
        self.max_ctx = mx
        self.ctx = MLAContext(dev(lw["kv_b_proj"], "bf16"), dev(lw["kv_norm_gamma"], "bf16") if w.gamma_noise else None,
                              num_heads=w.num_heads, dtype="fp8" if cache == "fp8" else "bf16", rms_eps=w.eps,
                              rope_theta=w.theta, max_q_tokens=w.n_q, max_batch=w.batch, max_position=mx + 16,
                              max_seq_len=mx + 16)
        self.ctx.layer_weights(dev(lw["q_proj"], "bf16"), dev(lw["kv_a_proj"], "bf16"), dev(lw["o_proj"], "bf16"),
                               dev(lw["input_norm_gamma"], "bf16"), input_norm=input_norm, residual=residual)
        if cache == "fp8":
            # the oracle's FP8 rows of the history (every other byte 0xFF)
            hist = w.all_tokens(history_only=True)
            self.pool8 = F.cache_write_fp8(np.full((w.n_blocks, 16, 1, 656), 0xFF, np.uint8), hist["c_kv"],
                                           hist["k_pe"], hist["positions"], hist["slot_mapping"],
                                           np.asarray(lw["kv_norm_gamma"], np.float64), w.eps, w.theta)
            self.pool = torch.from_numpy(self.pool8).to("cuda")
        else:
            self.hist = _oracle_history(w, lw) if history is None else history
            self.pool = dev(self.hist, "bf16")  # the oracle rounded every row to bf16: exact
        new = w.all_tokens(new_only=True)
        self.pos, self.slots = new["positions"], new["slot_mapping"]
        self.bt, self.sl = dev_i32(w.block_table), dev_i32(w.seq_lens)

    def step(self, hidden, pos=None, slots=None, seq_lens=None):
        pos = self.pos if pos is None else pos
        slots = self.slots if slots is None else slots
        sl = self.sl if seq_lens is None else dev_i32(seq_lens)
        out = self.ctx.layer_decode_step(dev(hidden, "bf16"), dev_i32(pos), dev_i32(slots), self.pool, self.bt, sl,
                                         self.max_ctx, q_len=self.w.q_len)
        torch.cuda.synchronize()
        return out.to(torch.float32).cpu().numpy().astype(np.float64)

    def free(self):
        self.ctx.free()


def _oracle_history(w, lw):
    hist = w.all_tokens(history_only=True)
    pool = np.full((w.n_blocks, 16, 1, 576), np.nan)
    return O.cache_write(pool, hist["c_kv"], hist["k_pe"], hist["positions"], hist["slot_mapping"],
                         np.asarray(lw["kv_norm_gamma"], np.float64), w.eps, w.theta, "bf16")


def _spacing(x):
    """bf16 spacing at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    m = np.abs(x)
    e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def _compare_out(got, ref, residual, label):
    """Without the residual: the decode's bf16 contract (max abs <= 2e-2, rel L2 <= 5e-3).  With it, the
    output adds the hidden state (|values| up to about 5) before its own rounding to bf16, which alone
    can move a value by half a bf16 spacing of it (2^-6 at [4, 8)): elementwise <= 2e-2 + half a spacing
    of the oracle's value, and rel L2 <= 5e-3."""
    if not residual:
        return compare(got, ref, "bf16", label)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = np.abs(got - ref)
    assert np.all(err <= 2e-2 + 0.5 * _spacing(ref)), f"{label}: max abs {err.max()}"
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert rel <= 5e-3, f"{label}: rel L2 {rel}"
    return float(err.max()), rel


def _check_rows(got_pool, ref_cache, slots, label):
    """The step's new cache rows (latent and rope parts apart).  They come from an fp32 projection of bf16
    operands, whose error is relative to the row's scale, not to each element: elementwise within two
    bf16 spacings of the oracle's value plus 2^-7 of the part's RMS; relative L2 <= 5e-3."""
    g = np.stack([got_pool[s // 16, s % 16, 0] for s in slots])
    r = np.stack([ref_cache[s // 16, s % 16, 0] for s in slots])
    assert np.all(np.isfinite(g)), f"{label}: non-finite new rows"
    for part in (slice(0, 512), slice(512, 576)):
        gp, rp = g[:, part], r[:, part]
        rms = np.sqrt(np.mean(rp * rp, axis=1, keepdims=True))
        assert np.all(np.abs(gp - rp) <= 2 * _spacing(rp) + 2.0 ** -7 * rms), f"{label}: new rows beyond the bound"
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    assert rel <= 5e-3, f"{label}: new rows rel L2 {rel}"


SMALL = [  # label, heads, q_len, seq_lens, input_norm, residual, gamma noise (kv_a, input)
    ("decoder_h16_q1", 16, 1, [300, 17, 1000, 65], True, True, (0.0, 0.0)),
    ("module_h16_q1", 16, 1, [300, 17, 1000, 65], False, False, (0.0, 0.0)),
    ("decoder_h16_q2_gammas", 16, 2, [129, 2, 700], True, True, (0.1, 0.1)),
    ("module_h32_q1", 32, 1, [64, 513, 40], False, False, (0.0, 0.2)),
    ("decoder_h32_q1_norm_only", 32, 1, [900, 33], True, False, (0.1, 0.0)),
]


@pytest.mark.parametrize("label,heads,q_len,seqs,input_norm,residual,noise", SMALL, ids=[c[0] for c in SMALL])
def test_layer_step_small(label, heads, q_len, seqs, input_norm, residual, noise):
    w = W.custom(f"layer_{label}", "bf16", heads, seqs, q_len=q_len, seed=401, gamma_noise=noise[0])
    _say("layer step", label)
    lw = w.layer_weights(0, input_gamma_noise=noise[1])
    hidden = w.hidden()
    run = LayerRun(w, lw, input_norm, residual)
    try:
        got = run.step(hidden)
        pool = run.pool.to(torch.float32).cpu().numpy().astype(np.float64)
    finally:
        run.free()
    ref, cache = L.layer_decode_step(hidden, run.pos, run.slots, run.hist, w.block_table, w.seq_lens,
                                     q_len, _weights(w, lw), input_norm=input_norm, residual=residual)
    max_abs, rel = _compare_out(got, ref, residual, label)
    _say(label, f"max abs {max_abs:.3e}, rel L2 {rel:.3e}")
    _check_rows(pool, cache, run.slots, label)


def test_layer_two_steps_in_a_row():
    """Step 1 writes the new tokens' rows at positions ctx-1; step 2 (new hidden states, one more token
    per sequence) reads them: both outputs and both sets of rows against the oracle chained."""
    w = W.custom("layer_two", "bf16", 16, [200, 31, 500], q_len=1, seed=402, pool_factor=1.5)
    _say("layer step twice")
    lw = w.layer_weights(0)
    wts = _weights(w, lw)
    run = LayerRun(w, lw, extra_ctx=1)
    try:
        h1, h2 = w.hidden(0), w.hidden(1)
        got1 = run.step(h1)
        # step 2: every context one token longer; the new token's slot in the same block table
        sl2 = w.seq_lens + 1
        need = (sl2 + 15) // 16
        bt2 = np.zeros((w.batch, int(need.max())), np.int32)
        free = sorted(set(range(w.n_blocks)) - set(w.block_table[w.block_table >= 0].ravel().tolist()))
        for b in range(w.batch):
            nb = (int(w.seq_lens[b]) + 15) // 16
            bt2[b, :nb] = w.block_table[b, :nb]
            if need[b] > nb:
                bt2[b, nb] = free.pop(0)
        pos2 = sl2 - 1
        slots2 = np.array([bt2[b, p // 16] * 16 + p % 16 for b, p in enumerate(pos2)], np.int32)
        run.bt = dev_i32(bt2)
        got2 = run.step(h2, pos2, slots2, sl2)
        pool = run.pool.to(torch.float32).cpu().numpy().astype(np.float64)
    finally:
        run.free()
    cache = run.hist
    ref1, cache = L.layer_decode_step(h1, run.pos, run.slots, cache, w.block_table, w.seq_lens, 1, wts)
    ref2, cache = L.layer_decode_step(h2, pos2, slots2, cache, bt2, sl2, 1, wts)
    _compare_out(got1, ref1, True, "step 1")
    _compare_out(got2, ref2, True, "step 2")
    _check_rows(pool, cache, list(run.slots) + list(slots2), "two steps")


def test_layer_step_fp8_cache():
    """One layer step over an FP8 cache whose history rows are the oracle's bytes.  The oracle writes
    the new tokens' rows from its own fp64 projection and decodes over the dequantised bytes; the
    GPU's new rows come from its own projection, so a code may sit one e4m3 step away (one row of
    each context).  The new rows the GPU wrote are checked against the oracle's to the e4m3 spacing."""
    w = W.custom("layer_fp8", "bf16", 16, [400, 90, 1200], q_len=1, seed=403)
    _say("layer step, fp8 cache")
    lw = w.layer_weights(0)
    hidden = w.hidden()
    run = LayerRun(w, lw, cache="fp8")
    try:
        got = run.step(hidden)
        got8 = run.pool.cpu().numpy()
    finally:
        run.free()
    x = O.rms_norm(hidden.astype(np.float64), lw["input_norm_gamma"], w.eps)
    q = (x @ lw["q_proj"].astype(np.float64).T).reshape(w.n_q, 16, 192)
    kv = x @ lw["kv_a_proj"].astype(np.float64).T
    pool8 = F.cache_write_fp8(run.pool8, kv[:, :512], kv[:, 512:], run.pos, run.slots,
                              np.asarray(lw["kv_norm_gamma"], np.float64), w.eps, w.theta)
    want = F.dequantize_cache(pool8)
    W_uk, W_uv = O.absorb(lw["kv_b_proj"].astype(np.float64), 16, 128, 128)
    a = O.decode_absorbed(q, want, w.block_table, w.seq_lens, 1, W_uk, W_uv, w.scale, w.theta)
    ref = a.reshape(w.n_q, -1) @ lw["o_proj"].astype(np.float64).T + hidden
    _compare_out(got, ref, True, "fp8 layer step")
    deq = F.dequantize_cache(got8)
    for s in run.slots:
        g, r = deq[s // 16, s % 16, 0], want[s // 16, s % 16, 0]
        assert np.linalg.norm(g - r) / np.linalg.norm(r) < 2 ** -4
    hist = np.ones(got8.shape[:2], bool)
    hist[run.slots // 16, run.slots % 16] = False
    assert np.array_equal(got8[hist], run.pool8[hist]), "the step changed bytes outside its new rows"


@pytest.mark.parametrize("seq_len", [1, 256, 1024])
def test_layer_step_batch1(seq_len):
    """The pages' latency-table shapes: one sequence, seq_len cached tokens + 1 new one, 16 heads."""
    w = W.lite_b1(seq_len)
    _say("layer step batch 1, seq_len", seq_len)
    lw = w.layer_weights(0)
    hidden = w.hidden()
    run = LayerRun(w, lw, residual=False)
    try:
        got = run.step(hidden)
        pool = run.pool.to(torch.float32).cpu().numpy().astype(np.float64)
    finally:
        run.free()
    ref, cache = L.layer_decode_step(hidden, run.pos, run.slots, run.hist, w.block_table, w.seq_lens, 1,
                                     _weights(w, lw), residual=False)
    compare(got, ref, "bf16", f"batch 1 seq {seq_len}")
    _check_rows(pool, cache, run.slots, f"batch 1 seq {seq_len}")


def test_layer_step_b64_s4096_every_sequence():
    """Batch 64 x 4,096 cached tokens (16 heads, D = 2,048), input RMSNorm without the residual (so that the
    comparison rests on the attention and its projections): every sequence against the oracle's layer step
    on that sequence's blocks of the oracle's history cache (the GPU's pool holds the same rows)."""
    w = W.lite_b64()
    _say("layer step lite_b64, every sequence")
    lw = w.layer_weights(0)
    wts = _weights(w, lw)
    hidden = w.hidden()
    run = LayerRun(w, lw, residual=False)
    try:
        got = run.step(hidden)
        # each sequence's blocks: the oracle's history, and the GPU's pool after the step
        locs, news = [], []
        for b in range(w.batch):
            nb = (int(w.seq_lens[b]) + 15) // 16
            locs.append(run.hist[w.block_table[b, :nb]])
            ids = torch.from_numpy(w.block_table[b, :nb].astype(np.int64)).cuda()
            news.append(run.pool[ids].to(torch.float32).cpu().numpy().astype(np.float64))
    finally:
        run.free()
    ref = np.empty_like(got)
    for b in range(w.batch):
        ctx = int(w.seq_lens[b])
        nb = (ctx + 15) // 16
        p = ctx - 1
        out_b, cache_b = L.layer_decode_step(hidden[b:b + 1], [p], [p], locs[b], np.arange(nb)[None, :],
                                             np.array([ctx]), 1, wts, residual=False)
        ref[b] = out_b[0]
        compare(got[b:b + 1], out_b, "bf16", f"lite_b64 sequence {b}")
        _check_rows(news[b], cache_b, [p], f"lite_b64 sequence {b}")
    compare(got, ref, "bf16", "lite_b64 whole output")


def test_layer_status_codes():
    from mla_latent_kv_paged_amd import MLAContext, MLAError
    w = W.custom("layer_abi", "bf16", 16, [20, 40], seed=404)
    lw = w.layer_weights(0)
    ctx = MLAContext(dev(lw["kv_b_proj"], "bf16"), None, num_heads=16, dtype="bf16", max_q_tokens=2, max_batch=2,
                     max_position=64, max_seq_len=64)
    try:
        pool = torch.zeros((8, 16, 1, 576), dtype=torch.bfloat16, device="cuda")
        h = torch.zeros((2, 2048), dtype=torch.bfloat16, device="cuda")
        i2 = torch.zeros((2,), dtype=torch.int32, device="cuda")
        bt = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
        sl = torch.full((2,), 40, dtype=torch.int32, device="cuda")
        ctx.hidden_dim = 2048
        with pytest.raises(MLAError) as e:          # no layer attached
            ctx.layer_decode_step(h, i2, i2, pool, bt, sl, 40)
        assert e.value.status == -1
        bad = torch.zeros((16 * 192, 1280), dtype=torch.bfloat16, device="cuda")
        p = bad.data_ptr()
        assert ctx.lib.mla_layer_weights(ctx.handle, 1280, p, p, p, None, 3, None) == -2  # D not a multiple of 512
        assert ctx.lib.mla_layer_weights(ctx.handle, 2048, p, p, p, None, 8, None) == -1  # unknown flag
        assert ctx.lib.mla_layer_weights(ctx.handle, 2048, None, p, p, None, 3, None) == -1  # null weights
    finally:
        ctx.free()
    ctx32 = MLAContext(torch.zeros((16 * 256, 512), dtype=torch.float32, device="cuda"), None, num_heads=16,
                       dtype="f32", max_q_tokens=2, max_batch=2, max_position=64, max_seq_len=64)
    try:
        z = torch.zeros((1,), dtype=torch.float32, device="cuda")
        assert ctx32.lib.mla_layer_weights(ctx32.handle, 2048, z.data_ptr(), z.data_ptr(), z.data_ptr(), None, 3,
                                           None) == -2  # fp32 context: unsupported
    finally:
        ctx32.free()


def test_model_step_27_layers_every_layer():
    """A decode step through 27 attention layers (one context, set of weights and cache per layer, layer l's
    output the input of layer l + 1), as bench.py --mode layer --layers 27 runs it, at 16 heads, three
    sequences.  End to end: the GPU's chained result against the oracle's 27-layer model step, within the
    bound the per-layer roundings allow.  Per layer: the oracle runs its own chain, rounding each layer's
    input to bf16 (the GPU's hidden states are bf16); each GPU layer is then stepped again on the oracle's
    rounded input to that layer, and its output and new cache rows are compared with the oracle's layer
    step on the same input."""
    L_ = 27
    w = W.custom("model27", "bf16", 16, [130, 37, 300], q_len=1, seed=405)
    _say("27-layer model step")
    lws = [w.layer_weights(li) for li in range(L_)]
    new = w.all_tokens(new_only=True)
    caches0 = []
    for li in range(L_):
        hist = {k: [] for k in ("c_kv", "k_pe", "positions", "slot_mapping")}
        for b in range(w.batch):
            c, k = w.history(b, li)
            n = int(w.seq_lens[b]) - 1
            hist["c_kv"].append(c[:n]); hist["k_pe"].append(k[:n])
            hist["positions"].append(np.arange(n)); hist["slot_mapping"].append(w.slots(b, 0, n))
        caches0.append(O.cache_write(np.full((w.n_blocks, 16, 1, 576), np.nan), np.concatenate(hist["c_kv"]),
                                     np.concatenate(hist["k_pe"]), np.concatenate(hist["positions"]),
                                     np.concatenate(hist["slot_mapping"]),
                                     lws[li]["kv_norm_gamma"].astype(np.float64), w.eps, w.theta, "bf16"))
    # the oracle's chain with bf16 inputs: the per-layer cases
    ins_o, refs, caches1 = [], [], []
    h = w.hidden().astype(np.float64)
    for li in range(L_):
        ins_o.append(O.round_to_bf16(h))
        h, cache_after = L.layer_decode_step(ins_o[li], new["positions"], new["slot_mapping"], caches0[li],
                                             w.block_table, w.seq_lens, 1, _weights(w, lws[li]))
        refs.append(h)
        caches1.append(cache_after)
    runs = []
    try:
        for li in range(L_):  # every layer its own history (the oracle's rows)
            runs.append(LayerRun(w, lws[li], history=caches0[li]))
        h = w.hidden()
        for run in runs:  # the chained step
            h = run.step(h)
        out_chain = h
        outs, pools = [], []
        for li, run in enumerate(runs):  # each layer again on the oracle's input (its new rows rewritten)
            outs.append(run.step(ins_o[li]))
            pools.append(run.pool.to(torch.float32).cpu().numpy().astype(np.float64))
    finally:
        for run in runs:
            run.free()
    for li in range(L_):
        _compare_out(outs[li], refs[li], True, f"layer {li}")
        _check_rows(pools[li], caches1[li], new["slot_mapping"], f"layer {li}")
    # end to end: the oracle's model step keeps the residual stream in fp64, the GPU stores it in bf16 after
    # every layer.  Each layer's error carries into the next through the residual, so elementwise the errors
    # add up to at most L times one layer's bound, and in relative L2 the output roundings (at most 2^-9 of a
    # value each, independent) grow like a random walk, sqrt(L) 2^-9 on top of the single-step bound
    ref27, _ = L.model_decode_step(w.hidden(), new["positions"], new["slot_mapping"], caches0, w.block_table,
                                   w.seq_lens, 1, [_weights(w, lw) for lw in lws])
    err = np.abs(out_chain - ref27)
    rel = float(np.linalg.norm(out_chain - ref27) / np.linalg.norm(ref27))
    _say(f"27 layers end to end: max abs {err.max():.3e}, rel L2 {rel:.3e}")
    assert np.all(err <= L_ * (2e-2 + 0.5 * _spacing(ref27)))
    assert rel <= 5e-3 + np.sqrt(L_) * 2.0 ** -9
