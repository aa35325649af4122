"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on seeded inputs.

Small cases compare every element; the full-size workloads compare every row of every sequence,
computed sequence by sequence by the oracle, in the launch configuration the benchmark uses.  Tolerances: fp32 storage -> cache bit-exact and decode max abs <= 1e-4;
bf16 storage -> cache within 1 bf16 ulp, decode max abs <= 2e-2 and relative L2 <= 5e-3."""

import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import mla_inputs as W

from ._harness import (DeviceRun, bf16_ulp_distance, compare, dev, dev_i32, oracle_all_sequences, oracle_full,
                       oracle_weights)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_latent_kv_paged_amd import load
    load()  # the HIP library must load: no fallback


def _say(*a):
    print("[case]", *a, flush=True)


def _check_cache(run, cache_ref, storage):
    got = run.pool_f64()
    live = np.isfinite(cache_ref)
    assert np.array_equal(np.isnan(got), ~live), "slots outside the written set changed"
    if storage == "f32":
        assert np.array_equal(got[live], cache_ref[live]), "fp32 cache not bit-exact"
    else:
        d = bf16_ulp_distance(got[live], cache_ref[live])
        assert np.max(d) <= 1.0
        assert np.mean(d > 0) <= 1e-4


# ------------------------------------------------------------------------------- small, elementwise

SMALL = [
    ("tiny_f32", lambda: W.tiny()),
    ("lite_b1_s1", lambda: W.lite_b1(1)),
    ("lite_b1_s256", lambda: W.lite_b1(256)),
    ("lite_b1_s1024", lambda: W.lite_b1(1024)),
    ("lite_b4_s300", lambda: W.lite_b64(batch=4, seq_len=300, n_blocks=200)),
    ("wide_h128_b2", lambda: W.wide(batch=2, lo=100, hi=700)),
    ("ragged_b8_q4", lambda: W.ragged(batch=8, median=200, hi=900)),
    ("ragged_b6_q4_f32", lambda: W.custom("r_f32", "f32", 16, [4, 5, 21, 64, 300, 17], q_len=4, seed=5)),
    ("wide_f32", lambda: W.custom("w_f32", "f32", 32, [33, 80], q_len=1, seed=6)),
    ("gamma_bf16", lambda: W.custom("g_bf16", "bf16", 16, [70, 129], q_len=2, seed=7, gamma_noise=0.1)),
    ("gamma_f32", lambda: W.custom("g_f32", "f32", 16, [70, 129], q_len=2, seed=8, gamma_noise=0.1)),
    ("ctx_eq_qlen", lambda: W.custom("edge", "bf16", 16, [1, 2, 3, 4, 16, 17], q_len=1, seed=9)),
    ("ctx_eq_qlen4", lambda: W.custom("edge4", "bf16", 16, [4, 16, 17, 20], q_len=4, seed=10)),
    ("h48_q2_bf16", lambda: W.custom("h48", "bf16", 48, [40, 300, 77], q_len=2, seed=11)),
    ("h32_q1_bf16", lambda: W.custom("h32", "bf16", 32, [33, 200, 517], q_len=1, seed=12)),
    # enough (head, 64-row) tiles to fill the device: the 64-row combine, by piece and by split, with a
    # ragged last tile (130 and 1,000 rows)
    ("rows64_h128_q2", lambda: W.custom("r64", "bf16", 128, [2 + (37 * i) % 400 for i in range(65)], q_len=2,
                                        seed=13)),
    ("rows64_h16_b1000", lambda: W.custom("r64s", "bf16", 16, [1 + (53 * i) % 150 for i in range(1000)], q_len=1,
                                          seed=14)),
    # other head counts: 64 (two 32-row tiles per query), 96 (three, with two queries per sequence, and
    # the 64-row combine)
    ("h64_q1", lambda: W.custom("h64", "bf16", 64, [40, 300, 77, 1000], q_len=1, seed=15)),
    ("h96_q2_rows64", lambda: W.custom("h96", "bf16", 96, [2 + (29 * i) % 200 for i in range(96)], q_len=2,
                                       seed=16)),
]


@pytest.mark.parametrize("name,make", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(name, make):
    w = make()
    _say(name, w.storage, "H", w.num_heads, "B", w.batch, "q_len", w.q_len, "ctx", list(w.seq_lens[:8]))
    cache_ref, out_ref = oracle_full(w)
    run = DeviceRun(w)
    try:
        _check_cache(run, cache_ref, w.storage)
        out = run.decode()
        compare(out, out_ref, w.storage, name)
    finally:
        run.free()


def test_decode_only_from_generator_pool():
    """Decode alone on a pool filled directly by the generator (isolates decode error)."""
    w = W.ragged(batch=6, median=150, hi=600, seed=21)
    _say("decode-only ragged", list(w.seq_lens))
    pool = w.random_pool()
    W_uk, W_uv = oracle_weights(w)
    ref = O.decode_absorbed(w.queries(), pool.astype(np.float64), w.block_table, w.seq_lens, w.q_len, W_uk, W_uv,
                            w.scale, w.theta)
    run = DeviceRun(w)
    try:
        out = run.decode(pool=dev(pool, w.storage))
        compare(out, ref, w.storage, "decode-only")
    finally:
        run.free()


@pytest.mark.parametrize("heads,q_len", [(16, 1), (32, 1), (16, 4)])
def test_latent_beyond_fp16_range(heads, q_len):
    """Latent cache entries far beyond fp16's range (the c part scaled by 2^17 > 65504, exact in
    bf16) with W_uk scaled by 2^-17, so that every score is unchanged and the output scales by
    exactly 2^17.  The bf16 kernels keep their split / piece partials in fp16; a partial row that
    would not fit must be stored scaled, not overflow.  One case per bf16 decode kernel shape (16
    rows; 32 rows with one and with two tiles per workgroup); compared after dividing by 2^17."""
    from mla_latent_kv_paged_amd import MLAContext
    w = W.custom("big", "bf16", heads, [40, 300, 77, 1000], q_len=q_len, seed=71)
    _say("latent beyond fp16", "H", heads, "q_len", q_len)
    big = 2.0 ** 17
    pool = w.random_pool()
    pool[..., :512] *= big
    kvb = w.kv_b_proj().reshape(heads, 256, 512).copy()
    kvb[:, :128, :] /= big  # W_uk rows
    kvb = kvb.reshape(heads * 256, 512)
    W_uk, W_uv = O.absorb(kvb.astype(np.float64), heads, 128, 128)
    ref = O.decode_absorbed(w.queries(), pool.astype(np.float64), w.block_table, w.seq_lens, w.q_len, W_uk, W_uv,
                            w.scale, w.theta)
    mx = int(w.seq_lens.max())
    ctx = MLAContext(dev(kvb, "bf16"), None, num_heads=heads, dtype="bf16", rms_eps=w.eps, rope_theta=w.theta,
                     max_q_tokens=w.n_q, max_batch=w.batch, max_position=mx + 16, max_seq_len=mx + 16)
    try:
        for sb in (0, 5):  # the library's split, and short splits (many partials per row)
            ctx.set_decode_tuning(sb, 0)
            out = ctx.decode(dev(w.queries(), "bf16"), dev(pool, "bf16"), dev_i32(w.block_table),
                             dev_i32(w.seq_lens), mx, q_len=w.q_len)
            torch.cuda.synchronize()
            got = out.to(torch.float32).cpu().numpy().astype(np.float64) / big
            compare(got, ref / big, "bf16", f"latent x2^17 H={heads} q_len={q_len} split={sb}")
    finally:
        ctx.free()


@pytest.mark.parametrize("heads,q_len", [(16, 1), (16, 2), (128, 1)])
def test_large_score_jump(heads, q_len):
    """A score far above everything before it: the rope part of the token at position 200 is scaled
    by 2^8 (exact in bf16), which puts its score near +-300 (log2 units) for most rows, so the
    running max jumps by far more than any softmax headroom in the middle of a split.

    Such a key magnifies the bf16 rounding of q into its score (about 0.4 log2 units), so rows where
    the spike competes with the other tokens are ill-conditioned for any bf16 kernel; the test
    compares the rows where the fp64 oracle puts the spike at least 40 log2 units above (it
    dominates) or below (it vanishes) every other visible score, and requires both kinds, with
    jumps of more than 64 over the split's first steps, to be present."""
    w = W.custom("jump", "bf16", heads, [40, 260, 700], q_len=q_len, seed=61)
    _say("score jump", "H", heads, "q_len", q_len)
    spike = 200
    pool = w.random_pool()
    for b in range(w.batch):
        if int(w.seq_lens[b]) > spike:
            pool[w.block_table[b, spike // 16], spike % 16, 0, 512:] *= 256.0
    pool64 = pool.astype(np.float64)
    W_uk, W_uv = oracle_weights(w)
    ref = O.decode_absorbed(w.queries(), pool64, w.block_table, w.seq_lens, w.q_len, W_uk, W_uv, w.scale, w.theta)

    log2e = 1.0 / np.log(2.0)
    q = w.queries().astype(np.float64)
    keep = np.ones(ref.shape[:2], dtype=bool)
    n_dom = n_van = 0
    for b in range(w.batch):
        ctx = int(w.seq_lens[b])
        if ctx <= spike:
            continue
        C, R = O.gather_sequence(pool64, w.block_table[b], ctx, 512)
        for i in range(w.q_len):
            pos, row = ctx - w.q_len + i, b * w.q_len + i
            for h in range(heads):
                s2 = O._absorbed_scores(q[row, h], C, R, W_uk[h], pos, w.scale, w.theta)[:pos + 1] * log2e
                d = s2[spike] - np.max(np.delete(s2, spike))
                keep[row, h] = abs(d) >= 40.0
                if d >= 40.0 and s2[spike] - np.max(s2[:32]) > 64.0:
                    n_dom += 1
                n_van += d <= -40.0
    assert n_dom > 0 and n_van > 0 and keep.mean() > 0.75, (n_dom, n_van, keep.mean())

    run = DeviceRun(w)
    try:
        for sb in (64, 5):
            out = run.decode(pool=dev(pool, w.storage), split_blocks=sb)
            got = out.float().cpu().numpy().astype(np.float64)
            compare(got[keep], ref[keep], w.storage, f"score jump split_blocks={sb}")
    finally:
        run.free()


CLIMB_LOG2 = 72.0  # rise of every row's score over its sequence (log2 units)


def climb_case(heads, q_len, seed):
    """Inputs whose scores climb steadily along each sequence, by CLIMB_LOG2 in log2 units: latent
    channel 0 of token t holds A t / (ctx - 1) and every query reads it with weight kappa (q_nope
    component 0 is 1, W_uk row 0 is kappa e_0), on top of the usual random scores.  W_uv column 0
    is zero, so channel 0 steers the softmax but adds nothing to the output.

    A row's running max then rises past any fixed headroom above its first blocks while the terms
    just below it still carry most of the weight: a kernel may rescale what it has accumulated or
    drop it only where it is negligible.  Only one channel carries the climb, so the kernels' bf16
    rounding of the scaled query moves score differences by at most 2^-9 relative: the case is
    well conditioned.  Returns (workload, queries, kv_b_proj, pool) as float32 storage values."""
    w = W.custom("climb", "bf16", heads, [300, 1000, 2500], q_len=q_len, seed=seed)
    kappa = 4.0
    amp = CLIMB_LOG2 / (kappa * w.scale / np.log(2.0))
    q = w.queries().copy()
    q[:, :, 0] = 1.0
    kvb = w.kv_b_proj().reshape(heads, 256, 512).copy()
    kvb[:, 0, :] = 0.0
    kvb[:, 0, 0] = kappa
    kvb[:, 128:, 0] = 0.0
    kvb = kvb.reshape(heads * 256, 512)
    pool = w.random_pool()
    for b in range(w.batch):
        ctx = int(w.seq_lens[b])
        t = np.arange(ctx)
        vals = W.bf16_bits_to_f32(W.f32_to_bf16_bits((amp * t / (ctx - 1)).astype(np.float32)))
        pool[w.block_table[b, t // 16], t % 16, 0, 0] = vals
    return w, q, kvb, pool


def climb_rows(w, q, kvb, pool):
    """Rows whose score max rises by more than 64 log2 units above their first two blocks (the
    pattern the case is built for), from the fp64 oracle's scores."""
    W_uk, _ = O.absorb(kvb.astype(np.float64), w.num_heads, 128, 128)
    pool64 = pool.astype(np.float64)
    n = 0
    log2e = 1.0 / np.log(2.0)
    for b in range(w.batch):
        ctx = int(w.seq_lens[b])
        C, R = O.gather_sequence(pool64, w.block_table[b], ctx, 512)
        pos, row = ctx - 1, b * w.q_len + w.q_len - 1
        for h in range(w.num_heads):
            s2 = O._absorbed_scores(q[row, h].astype(np.float64), C, R, W_uk[h], pos, w.scale, w.theta)[:pos + 1]
            s2 = s2 * log2e
            n += np.max(s2) - np.max(s2[:32]) > 64.0
    return n


@pytest.mark.parametrize("heads,q_len", [(16, 1), (32, 1), (16, 2), (128, 1)])
def test_score_climb(heads, q_len):
    """Steadily climbing scores (climb_case): one case per bf16 decode kernel shape (16 rows; 32
    rows with one and with four tiles per workgroup), at the library's split and at the longest
    ranges the tuning allows, against the fp64 oracle on every row."""
    from mla_latent_kv_paged_amd import MLAContext
    w, q, kvb, pool = climb_case(heads, q_len, seed=81)
    _say("score climb", "H", heads, "q_len", q_len)
    assert climb_rows(w, q, kvb, pool) >= heads  # most rows of every sequence climb past 64
    W_uk, W_uv = O.absorb(kvb.astype(np.float64), heads, 128, 128)
    ref = O.decode_absorbed(q, pool.astype(np.float64), w.block_table, w.seq_lens, w.q_len, W_uk, W_uv, w.scale,
                            w.theta)
    mx = int(w.seq_lens.max())
    ctx = MLAContext(dev(kvb, "bf16"), None, num_heads=heads, dtype="bf16", rms_eps=w.eps, rope_theta=w.theta,
                     max_q_tokens=w.n_q, max_batch=w.batch, max_position=mx + 16, max_seq_len=mx + 16)
    try:
        # library choice; fewest 32-row workgroups; longest 16-row splits, at two and four waves
        for sb, waves in ((0, 0), (1, 0), (160, 0), (160, 4), (3, 4)):
            if waves and (heads * q_len) % 32 == 0:
                continue  # the wave count applies to the 16-row kernel
            ctx.set_decode_tuning(sb, waves)
            out = ctx.decode(dev(q, "bf16"), dev(pool, "bf16"), dev_i32(w.block_table), dev_i32(w.seq_lens), mx,
                             q_len=w.q_len)
            torch.cuda.synchronize()
            compare(out, ref, "bf16", f"score climb H={heads} q_len={q_len} tuning={sb} waves={waves}")
    finally:
        ctx.free()


@pytest.mark.parametrize("storage,heads,q_len", [("bf16", 16, 2), ("f32", 16, 2), ("bf16", 128, 1), ("bf16", 16, 4)])
def test_split_sweep_and_determinism(storage, heads, q_len):
    """Every split size from one block to the whole context (odd sizes end a two-block step past
    the split), run twice each: results within tolerance and bit-identical between runs."""
    w = W.custom("sweep", storage, heads, [4, 37, 200, 513], q_len=q_len, seed=31)
    _say("split sweep", storage, "H", heads, "q_len", q_len)
    _, ref = oracle_full(w)
    run = DeviceRun(w)
    try:
        for sb in (1, 2, 3, 5, 8, 13, 33, 0):
            out = run.decode(split_blocks=sb)
            compare(out, ref, storage, f"split_blocks={sb}")
            again = run.decode(split_blocks=sb)
            assert torch.equal(out, again), f"non-deterministic at split_blocks={sb}"
    finally:
        run.free()


@pytest.mark.parametrize("waves", [2, 4])
def test_16row_kernel_waves_split_sweep(waves):
    """The 16-row bf16 kernel (16 heads, one query token) at two and four waves per workgroup: split sizes
    from one block to past the longest context (a wave with no block, odd block counts per wave), each run
    twice (bitwise equal), against the oracle; contexts of 1 to 1,500 tokens."""
    w = W.custom("w16", "bf16", 16, [1, 15, 16, 17, 200, 513, 1000, 1500], q_len=1, seed=33)
    _say("16-row kernel", "waves", waves)
    _, ref = oracle_full(w)
    run = DeviceRun(w)
    try:
        for sb in (1, 2, 3, 5, 8, 13, 33, 96, 0):
            out = run.decode(split_blocks=sb, waves=waves)
            shape = run.ctx.last_decode_shape()
            assert shape["waves"] == waves, shape
            compare(out, ref, "bf16", f"waves={waves} split_blocks={sb}")
            again = run.decode(split_blocks=sb, waves=waves)
            assert torch.equal(out, again), f"non-deterministic at waves={waves} split_blocks={sb}"
    finally:
        run.free()


def test_block_table_relabel_invariance():
    w = W.custom("relabel", "bf16", 16, [45, 130], q_len=1, seed=41)
    _say("relabel")
    run = DeviceRun(w)
    try:
        base = run.decode()
        perm = np.random.default_rng(3).permutation(w.n_blocks)
        pool2 = torch.empty_like(run.pool)
        pool2[torch.from_numpy(perm).cuda()] = run.pool
        bt2 = dev_i32(perm[w.block_table])
        out = run.ctx.decode(run.q, pool2, bt2, run.sl, run.max_ctx, q_len=w.q_len)
        torch.cuda.synchronize()
        assert torch.equal(out, base)
    finally:
        run.free()


# ------------------------------------------------------------------------------- full size, every sequence

FULL = [
    ("lite_b64_s4096", lambda: W.lite_b64()),
    ("wide_h128_b128", lambda: W.wide()),
    ("ragged_b256_q4", lambda: W.ragged()),
]


@pytest.mark.parametrize("name,make", FULL, ids=[f[0] for f in FULL])
def test_full_size_every_sequence(name, make):
    """The three full-size workloads in the launch configuration the benchmark uses (the library's
    own split or partition): every row of every sequence against the oracle.  The oracle computes
    each sequence on an identity-paged local pool (paging relabel invariance), in worker processes.
    Both tolerances are applied per sequence and to the whole output."""
    w = make()
    _say(name, "B", w.batch, "sum ctx", w.total_ctx, "every sequence")
    run = DeviceRun(w, per_sequence_upload=True)
    try:
        out = run.decode()
        shape = run.ctx.last_decode_shape()
        got = out.to(torch.float32).cpu().numpy().astype(np.float64)
    finally:
        run.free()
    _say(name, "launch", shape, "oracle on every sequence")
    ref = oracle_all_sequences(w)
    for b in range(w.batch):
        rows = slice(b * w.q_len, (b + 1) * w.q_len)
        compare(got[rows], ref[rows], w.storage, f"{name} seq {b} (ctx {w.seq_lens[b]})")
    max_abs, rel = compare(got, ref, w.storage, f"{name} whole output")
    _say(name, f"max abs {max_abs:.3e}, rel L2 {rel:.3e}")


def test_f32_long_context_split_within_workspace():
    """fp32 storage with a context bound above 65,536 tokens: the split count must stay within the
    partial workspace sized at mla_absorb_weights (32 splits), so a split holds more than 128 blocks
    here (the fp32 kernel reads its block ids as it goes).  A 70,000-token sequence beside a short one,
    every row against the oracle."""
    w = W.custom("f32_long", "f32", 16, [40, 70000], q_len=1, seed=61)
    _say("fp32 long context", list(w.seq_lens))
    run = DeviceRun(w)
    try:
        out = run.decode()
        shape = run.ctx.last_decode_shape()
        assert shape["n_split"] <= 32, shape
        assert shape["split_blocks"] * shape["n_split"] >= (70000 + 15) // 16, shape
        got = out.to(torch.float32).cpu().numpy().astype(np.float64)
    finally:
        run.free()
    ref = oracle_all_sequences(w)
    compare(got, ref, "f32", "fp32 long context")


# ------------------------------------------------------------------------------- ABI on the GPU

def test_abi_status_codes_on_device():
    from mla_latent_kv_paged_amd import MLAContext, MLAError
    w = W.custom("abi", "bf16", 16, [20, 40], seed=51)
    run = DeviceRun(w)
    try:
        with pytest.raises(MLAError) as e:      # batch above the cap
            bt = dev_i32(np.zeros((3, 8)))
            run.ctx.decode(dev(np.zeros((3, 16, 192), np.float32), "bf16"), run.pool, bt,
                           dev_i32([5, 5, 5]), 40)
        assert e.value.status == -5
        with pytest.raises(MLAError) as e:      # max_seq_len above the cap
            run.ctx.decode(run.q, run.pool, run.bt, run.sl, 10 ** 6)
        assert e.value.status == -5
        with pytest.raises(MLAError) as e:      # block table narrower than max_seq_len needs
            run.ctx.decode(run.q, run.pool, run.bt[:, :1].contiguous(), run.sl, 40)
        assert e.value.status == -1
        with pytest.raises(MLAError) as e:      # unsupported head count
            MLAContext(dev(np.zeros((24 * 256, 512), np.float32), "bf16"), num_heads=24, dtype="bf16")
        assert e.value.status == -2
    finally:
        run.free()


def test_profiling_helpers_on_device():
    """The inspection helpers the benchmark reads, through the binding: per-kernel event totals and
    samples after profiled decodes, and the last launch shape."""
    from mla_latent_kv_paged_amd import K_CACHE_WRITE, K_COMBINE, K_DECODE, K_Q_ABSORB
    w = W.custom("prof", "bf16", 16, [300, 40], seed=52)
    run = DeviceRun(w)
    try:
        run.ctx.profile_enable(True)
        for _ in range(3):
            run.decode()
        for kid in (K_Q_ABSORB, K_DECODE, K_COMBINE):
            ms, n = run.ctx.profile_read(kid)
            assert n == 3 and ms > 0.0, (kid, ms, n)
            samples = run.ctx.profile_samples(kid)
            assert len(samples) == 3 and all(x > 0.0 for x in samples), (kid, samples)
        assert run.ctx.profile_read(K_CACHE_WRITE)[1] == 0
        run.ctx.profile_enable(False)
        shape = run.ctx.last_decode_shape()
        assert shape["n_split"] >= 1 and shape["waves"] >= 1, shape
    finally:
        run.free()
