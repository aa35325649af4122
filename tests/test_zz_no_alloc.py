"""mla_decode_noalloc (the decode on the library's static scratch region, no allocation) against
mla_decode (the context's workspace) through the C ABI: the same kernels and launch shape, so the
outputs must be equal bit for bit; also against the fp64 oracle at the contract's tolerance.  Two
calls in a row, the second with a smaller input, for each decode kernel family (16-row bf16, 32-row
bf16, FP8 rows, fp32); a decode too large for the region is refused with MLA_ECAP."""

import numpy as np
import pytest

from oracle import mla_fp8 as F
from oracle import mla_oracle as O
from workloads import mla_inputs as W

from ._harness import DeviceRun, compare, dev, dev_i32, oracle_full, oracle_weights

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


def _both(run, w, q, bt, sl, max_ctx):
    """(mla_decode output, mla_decode_noalloc output) for the same arguments."""
    ref = run.ctx.decode(q, run.pool, bt, sl, max_ctx, q_len=w.q_len)
    out = torch.full_like(ref, float("nan"))
    run.ctx.decode_noalloc(q, run.pool, bt, sl, max_ctx, out, q_len=w.q_len)
    torch.cuda.synchronize()
    return ref, out


CASES = [  # (label, storage, heads, q_len, first seq_lens, second (smaller) seq_lens)
    ("bf16_16row", "bf16", 16, 1, [300, 1000, 37, 4097, 17, 640, 2048, 129], [40, 513, 16]),
    ("bf16_32row", "bf16", 32, 1, [900, 77, 1500, 2000, 33], [300, 40]),
    ("bf16_32row_q4", "bf16", 16, 4, [700, 21, 1200, 4, 333], [64, 9]),
    ("f32", "f32", 16, 2, [129, 70, 400], [33, 5]),
]


@pytest.mark.parametrize("label,storage,heads,q_len,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_decode(label, storage, heads, q_len, first, second):
    w = W.custom(f"na_{label}", storage, heads, first, q_len=q_len, seed=301)
    _say("noalloc", label, "first", first, "second", second)
    cache_oracle, ref_oracle = oracle_full(w)
    run = DeviceRun(w)
    try:
        a, b = _both(run, w, run.q, run.bt, run.sl, run.max_ctx)
        assert torch.equal(a, b), f"{label}: first call differs from mla_decode"
        compare(b, ref_oracle, storage, f"{label} first call vs oracle")
        # second call: the first sequences only, a shorter bound, on the same context and pool
        nb = len(second)
        sl2 = dev_i32(np.minimum(w.seq_lens[:nb], second))
        mx2 = int(max(second))
        q2 = run.q[:nb * q_len].contiguous()
        bt2 = run.bt[:nb].contiguous()
        a2, b2 = _both(run, w, q2, bt2, sl2, mx2)
        assert torch.equal(a2, b2), f"{label}: second call differs from mla_decode"
        # oracle for the second call: the oracle's cache, shorter contexts (the last q_len tokens of
        # each shortened context are the queries' positions)
        W_uk, W_uv = oracle_weights(w)
        ref2 = O.decode_absorbed(w.queries()[:nb * q_len], cache_oracle, w.block_table[:nb],
                                 np.minimum(w.seq_lens[:nb], second), q_len, W_uk, W_uv, w.scale, w.theta)
        compare(b2, ref2, storage, f"{label} second call vs oracle")
    finally:
        run.free()


def test_noalloc_fp8_matches_decode():
    from mla_latent_kv_paged_amd import MLAContext
    w = W.custom("na_fp8", "bf16", 16, [500, 1300, 64, 2000], q_len=1, seed=302)
    _say("noalloc fp8")
    mx = int(w.seq_lens.max())
    ctx = MLAContext(dev(w.kv_b_proj(), "bf16"), None, num_heads=16, dtype="fp8", rms_eps=w.eps,
                     rope_theta=w.theta, max_q_tokens=w.n_q, max_batch=w.batch, max_position=mx + 16,
                     max_seq_len=mx + 16)
    try:
        # the oracle's FP8 rows (every other byte 0xFF: NaN codes, rope values and scales)
        tok = w.all_tokens()
        pool8 = F.cache_write_fp8(np.full((w.n_blocks, 16, 1, 656), 0xFF, np.uint8), tok["c_kv"], tok["k_pe"],
                                  tok["positions"], tok["slot_mapping"], w.gamma().astype(np.float64), w.eps,
                                  w.theta)
        deq = F.dequantize_cache(pool8)
        pool = torch.from_numpy(pool8).to("cuda")
        q, bt, sl = dev(w.queries(), "bf16"), dev_i32(w.block_table), dev_i32(w.seq_lens)
        for nb, mxx in ((4, mx), (2, 700)):
            sl_n = dev_i32(np.minimum(w.seq_lens[:nb], mxx))
            a = ctx.decode(q[:nb].contiguous(), pool, bt[:nb].contiguous(), sl_n, mxx)
            b = torch.full_like(a, float("nan"))
            ctx.decode_noalloc(q[:nb].contiguous(), pool, bt[:nb].contiguous(), sl_n, mxx, b)
            torch.cuda.synchronize()
            assert torch.equal(a, b), f"fp8: batch {nb} differs from mla_decode"
            W_uk, W_uv = oracle_weights(w)
            ref = O.decode_absorbed(w.queries()[:nb], deq, w.block_table[:nb], np.minimum(w.seq_lens[:nb], mxx), 1,
                                    W_uk, W_uv, w.scale, w.theta)
            compare(b, ref, "bf16", f"fp8 batch {nb} vs oracle")
    finally:
        ctx.free()


def test_noalloc_refuses_beyond_region():
    """128 heads x 128 sequences of up to 8,192 tokens need about 70 MB of scratch: MLA_ECAP, and the
    output is left untouched.  The arguments are refused before anything is launched."""
    from mla_latent_kv_paged_amd import MLAContext, MLAError
    H, B, S = 128, 128, 8192
    _say("noalloc over the region: H", H, "B", B, "S", S)
    kvb = torch.zeros((H * 256, 512), dtype=torch.bfloat16, device="cuda")
    ctx = MLAContext(kvb, None, num_heads=H, dtype="bf16", max_q_tokens=B, max_batch=B, max_position=S,
                     max_seq_len=S)
    try:
        q = torch.zeros((B, H, 192), dtype=torch.bfloat16, device="cuda")
        pool = torch.zeros((8, 16, 1, 576), dtype=torch.bfloat16, device="cuda")
        bt = torch.zeros((B, S // 16), dtype=torch.int32, device="cuda")
        sl = torch.full((B,), S, dtype=torch.int32, device="cuda")
        out = torch.full((B, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(MLAError) as e:
            ctx.decode_noalloc(q, pool, bt, sl, S, out)
        assert e.value.status == -5
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    finally:
        ctx.free()
