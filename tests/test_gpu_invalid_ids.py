"""Out-of-range block ids through the C ABI: the library reads such a block as 16 rows of zeros (every
kernel checks an id against num_blocks before it reads, negative ids included).  Each case runs with a
block table that has a negative id and an id past the pool in the middle of a context, and compares
with the fp64 oracle over the same cache with one block of zeros appended and those entries pointing
at it (the oracle's own gather, unchanged).  Cases: the 16-row and the 32-row bf16 decode, the FP8
decode, and the chunked prefill over bf16 and over FP8 rows (whose rows are dequantised first)."""

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


def _cu(chunks):
    return np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)


def _bad_table(w):
    """The workload's table with entry (0, 2) negative and entry (1, 5) past the pool (both blocks of
    history tokens), and the oracle's table with both pointing at an appended block index n_blocks."""
    bad = w.block_table.copy()
    assert int(w.seq_lens[0]) > 3 * 16 and int(w.seq_lens[1]) > 6 * 16
    bad[0, 2] = -3
    bad[1, 5] = w.n_blocks + 7
    ref = bad.copy()
    ref[0, 2] = w.n_blocks
    ref[1, 5] = w.n_blocks
    return bad, ref


def _with_zero_block(cache):
    return np.concatenate([cache, np.zeros((1,) + cache.shape[1:], cache.dtype)], axis=0)


@pytest.mark.parametrize("heads", [16, 32], ids=["16row", "32row"])
def test_decode_out_of_range_ids(heads):
    w = W.custom("badids", "bf16", heads, [100, 300, 64], q_len=1, seed=301 + heads)
    _say("decode out-of-range ids", "H", heads)
    bad, ref_bt = _bad_table(w)
    cache, _ = oracle_full(w)
    W_uk, W_uv = oracle_weights(w)
    ref = O.decode_absorbed(w.queries(), _with_zero_block(cache), ref_bt, w.seq_lens, w.q_len, W_uk, W_uv, w.scale,
                            w.theta)
    run = DeviceRun(w)
    try:
        out = run.ctx.decode(run.q, run.pool, dev_i32(bad), run.sl, run.max_ctx, q_len=w.q_len)
        torch.cuda.synchronize()
        compare(out, ref, "bf16", f"decode out-of-range ids H={heads}")
    finally:
        run.free()


def _fp8_pool(w):
    tok = w.all_tokens()
    pool8 = F.cache_write_fp8(np.full((w.n_blocks, 16, 1, F.ROW_BYTES), 0xFF, np.uint8), tok["c_kv"], tok["k_pe"],
                              tok["positions"], tok["slot_mapping"], w.gamma().astype(np.float64), w.eps, w.theta)
    return pool8, F.dequantize_cache(pool8)


def _fp8_ctx(w):
    from mla_latent_kv_paged_amd import MLAContext
    max_ctx = int(w.seq_lens.max())
    return MLAContext(dev(w.kv_b_proj(), "bf16"), None, num_heads=w.num_heads, dtype="fp8", rms_eps=w.eps,
                      rope_theta=w.theta, max_q_tokens=w.n_q, max_batch=w.batch, max_position=max_ctx + 16,
                      max_seq_len=max_ctx + 16)


def test_fp8_decode_out_of_range_ids():
    w = W.custom("badids8", "bf16", 16, [100, 300, 64], q_len=1, seed=311)
    _say("fp8 decode out-of-range ids")
    bad, ref_bt = _bad_table(w)
    pool8, deq = _fp8_pool(w)
    W_uk, W_uv = oracle_weights(w)
    ref = O.decode_absorbed(w.queries(), _with_zero_block(deq), ref_bt, w.seq_lens, w.q_len, W_uk, W_uv, w.scale,
                            w.theta)
    ctx = _fp8_ctx(w)
    try:
        out = ctx.decode(dev(w.queries(), "bf16"), torch.from_numpy(pool8).to("cuda"), dev_i32(bad),
                         dev_i32(w.seq_lens), int(w.seq_lens.max()), q_len=w.q_len)
        torch.cuda.synchronize()
        compare(out, ref, "bf16", "fp8 decode out-of-range ids")
    finally:
        ctx.free()


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_prefill_out_of_range_ids(fp8):
    w = W.custom("badids_pf", "bf16", 16, [300, 140], q_len=1, seed=321)
    chunks = [64, 140]
    _say("prefill out-of-range ids", "fp8" if fp8 else "bf16", "chunks", chunks)
    bad, ref_bt = _bad_table(w)
    W_uk, W_uv = oracle_weights(w)
    q = w.chunk_queries(chunks)
    if fp8:
        pool8, cache = _fp8_pool(w)
    else:
        cache, _ = oracle_full(w)
    ref = O.prefill_naive(q, _cu(chunks), _with_zero_block(cache), ref_bt, w.seq_lens, W_uk, W_uv, w.scale, w.theta)
    if fp8:
        ctx, pool = _fp8_ctx(w), torch.from_numpy(pool8).to("cuda")
    else:
        run = DeviceRun(w)
        ctx, pool = run.ctx, run.pool
    try:
        out = ctx.prefill(dev(q, "bf16"), dev_i32(_cu(chunks)), pool, dev_i32(bad), dev_i32(w.seq_lens),
                          int(w.seq_lens.max()), max(chunks))
        torch.cuda.synchronize()
        compare(out, ref, "bf16", f"prefill out-of-range ids {'fp8' if fp8 else 'bf16'}")
    finally:
        ctx.free()
