"""GPU parity of the chunked prefill (mla_prefill) through the C ABI against the fp64 oracle's
prefill_naive (oracle/mla_oracle.py), to the bf16 tolerance (max abs 2e-2, relative L2 5e-3), over
bf16 rows and over FP8 rows (the oracle's bytes, dequantised by oracle/mla_fp8.py for the oracle).

Each case writes every context token with mla_cache_write (the chunk's tokens included, as a serving
engine does before attention), then runs one prefill whose chunk of sequence b is its last n_b
tokens.  The oracle reads its own cache (oracle cache_write of the same seeded tokens).  The queries
are the seeded workload's chunk queries (one row per chunk token, in sequence order).
Unused pool slots are NaN, so a read of a token the kernels should not see poisons the output."""

import numpy as np
import pytest

from oracle import mla_fp8 as F
from oracle import mla_oracle as O
from workloads import mla_inputs as W

from ._harness import DeviceRun, compare, dev, dev_i32, oracle_weights

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


def _oracle_prefill(w, chunks):
    W_uk, W_uv = oracle_weights(w)
    tok = w.all_tokens()
    cache = O.cache_write(np.full((w.n_blocks, 16, 1, 576), np.nan), tok["c_kv"], tok["k_pe"], tok["positions"],
                          tok["slot_mapping"], w.gamma().astype(np.float64), w.eps, w.theta, w.storage)
    return O.prefill_naive(w.chunk_queries(chunks), _cu(chunks), cache, w.block_table, w.seq_lens, W_uk, W_uv,
                           w.scale, w.theta)


def _run_prefill(run, chunks, max_q_len=None):
    w = run.w
    q = dev(w.chunk_queries(chunks), w.storage)
    mq = int(max_q_len or max(max(chunks), 1))
    out = run.ctx.prefill(q, dev_i32(_cu(chunks)), run.pool, run.bt, run.sl, run.max_ctx, mq)
    torch.cuda.synchronize()
    return out


PREFILL_CASES = [
    # name, heads, context lengths, chunk lengths (the last n_b tokens of each context)
    ("mixed_h16", 16, [300, 77, 129], [64, 77, 1]),        # a fresh prefill, a one-token chunk
    ("h128", 128, [150, 90], [100, 90]),
    ("ragged_h16", 16, [513, 1000, 40], [257, 333, 0]),   # tails off every tile size, an empty chunk
    ("h32_q", 32, [200, 65], [130, 64]),
]


@pytest.mark.parametrize("name,heads,ctxs,chunks", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_parity(name, heads, ctxs, chunks):
    w = W.custom("pf_" + name, "bf16", heads, ctxs, q_len=1, seed=90 + heads)
    _say("prefill", name, "H", heads, "ctx", ctxs, "chunks", chunks)
    ref = _oracle_prefill(w, chunks)
    run = DeviceRun(w)
    try:
        out = _run_prefill(run, chunks)
        compare(out, ref, "bf16", f"prefill {name}")
        out2 = _run_prefill(run, chunks, max_q_len=max(chunks) + 37)  # a looser launch bound
        assert torch.equal(out, out2), "prefill result depends on the launch bound"
        assert torch.equal(out, _run_prefill(run, chunks)), "prefill is not deterministic"
    finally:
        run.free()


def test_prefill_gamma_and_long_fresh_chunk():
    """A 2,048-token chunk that is the whole context (every query tile, the longest first, and the
    diagonal tiles), with gamma != 1 in the cache write."""
    w = W.custom("pf_long", "bf16", 16, [2048], q_len=1, seed=95, gamma_noise=0.1)
    _say("prefill long fresh chunk 2048, gamma noise")
    ref = _oracle_prefill(w, [2048])
    run = DeviceRun(w)
    try:
        compare(_run_prefill(run, [2048]), ref, "bf16", "prefill 2048 fresh")
    finally:
        run.free()


def test_prefill_one_token_chunks_match_decode():
    """Chunks of one token are a decode: the prefill (expanded K/V, MHA-style) and mla_decode (the
    absorbed form) reach the same result by different arithmetic; both against the oracle, and
    against each other to twice the tolerance."""
    w = W.custom("pf_dec", "bf16", 16, [700, 33, 258], q_len=1, seed=96)
    _say("prefill one-token chunks vs decode")
    ref = _oracle_prefill(w, [1, 1, 1])
    run = DeviceRun(w)
    try:
        pf = _run_prefill(run, [1, 1, 1])
        dc = run.ctx.decode(dev(w.chunk_queries([1, 1, 1]), "bf16"), run.pool, run.bt, run.sl, run.max_ctx, q_len=1)
        torch.cuda.synchronize()
        compare(pf, ref, "bf16", "prefill one-token chunks")
        compare(dc, ref, "bf16", "decode")
        d = (pf.float() - dc.float()).abs().max().item()
        assert d <= 4e-2, d
    finally:
        run.free()


class Fp8Prefill:
    """An FP8-cache context whose pool holds the oracle's FP8 rows of every token (other bytes 0xFF:
    NaN codes, rope values and scales), and the oracle's dequantised values of the same bytes."""

    def __init__(self, w):
        from mla_latent_kv_paged_amd import MLAContext
        self.w = w
        self.max_ctx = int(w.seq_lens.max())
        self.ctx = MLAContext(dev(w.kv_b_proj(), "bf16"), dev(w.gamma(), "bf16") if w.gamma_noise else None,
                              num_heads=w.num_heads, dtype="fp8", rms_eps=w.eps, rope_theta=w.theta,
                              max_q_tokens=w.n_q, max_batch=w.batch, max_position=self.max_ctx + 16,
                              max_seq_len=self.max_ctx + 16)
        tok = w.all_tokens()
        pool8 = F.cache_write_fp8(np.full((w.n_blocks, 16, 1, F.ROW_BYTES), 0xFF, np.uint8), tok["c_kv"],
                                  tok["k_pe"], tok["positions"], tok["slot_mapping"], w.gamma().astype(np.float64),
                                  w.eps, w.theta)
        self.deq = F.dequantize_cache(pool8)
        self.pool = torch.from_numpy(pool8).to("cuda")
        self.bt, self.sl = dev_i32(w.block_table), dev_i32(w.seq_lens)

    def oracle(self, chunks):
        W_uk, W_uv = oracle_weights(self.w)
        return O.prefill_naive(self.w.chunk_queries(chunks), _cu(chunks), self.deq, self.w.block_table,
                               self.w.seq_lens, W_uk, W_uv, self.w.scale, self.w.theta)

    def free(self):
        self.ctx.free()


FP8_PREFILL_CASES = [
    ("mixed_h16", 16, [300, 77, 129], [64, 77, 1], 0.0),
    ("ragged_h16", 16, [513, 1000, 40], [257, 333, 0], 0.0),
    ("h128", 128, [150, 90], [100, 90], 0.0),
    ("fresh_2048_gamma", 16, [2048], [2048], 0.1),
]


@pytest.mark.parametrize("name,heads,ctxs,chunks,gamma_noise", FP8_PREFILL_CASES,
                         ids=[c[0] for c in FP8_PREFILL_CASES])
def test_prefill_fp8_cache(name, heads, ctxs, chunks, gamma_noise):
    """Chunked prefill over FP8 rows (dequantised to bf16 rows, code x group scale, before the expansion)
    against the oracle's prefill_naive over the same bytes dequantised by the oracle's format decoder."""
    w = W.custom("pf8_" + name, "bf16", heads, ctxs, q_len=1, seed=190 + heads, gamma_noise=gamma_noise)
    _say("fp8 prefill", name, "H", heads, "ctx", ctxs, "chunks", chunks)
    run = Fp8Prefill(w)
    try:
        ref = run.oracle(chunks)
        q = dev(w.chunk_queries(chunks), "bf16")
        out = run.ctx.prefill(q, dev_i32(_cu(chunks)), run.pool, run.bt, run.sl, run.max_ctx, max(max(chunks), 1))
        torch.cuda.synchronize()
        compare(out, ref, "bf16", f"fp8 prefill {name}")
    finally:
        run.free()


def test_prefill_fp8_one_token_chunks_match_decode():
    """One-token chunks over FP8 rows: the prefill (expanded K/V) and mla_decode (absorbed, FP8 rows
    read in the decode kernel) against the oracle and against each other."""
    w = W.custom("pf8_dec", "bf16", 16, [700, 33, 258], q_len=1, seed=196)
    _say("fp8 prefill one-token chunks vs decode")
    run = Fp8Prefill(w)
    try:
        ref = run.oracle([1, 1, 1])
        q = dev(w.chunk_queries([1, 1, 1]), "bf16")
        pf = run.ctx.prefill(q, dev_i32(_cu([1, 1, 1])), run.pool, run.bt, run.sl, run.max_ctx, 1)
        dc = run.ctx.decode(q, run.pool, run.bt, run.sl, run.max_ctx, q_len=1)
        torch.cuda.synchronize()
        compare(pf, ref, "bf16", "fp8 prefill one-token chunks")
        compare(dc, ref, "bf16", "fp8 decode")
        assert (pf.float() - dc.float()).abs().max().item() <= 4e-2
    finally:
        run.free()


def test_prefill_status_codes():
    """Host-side validation through the C ABI: a workspace one byte short, a chunk bound above the
    context bound, and an fp32 context (unsupported) are refused before any launch."""
    from mla_latent_kv_paged_amd import MLAError, MLAContext
    w = W.custom("pf_err", "bf16", 16, [40], q_len=1, seed=97)
    run = DeviceRun(w)
    cu = _cu([8])
    q = dev(w.chunk_queries([8]), "bf16")
    try:
        need = run.ctx.prefill_workspace_size(1, 8, run.max_ctx)
        ws = torch.empty((need - 1,), dtype=torch.uint8, device="cuda")
        with pytest.raises(MLAError):
            run.ctx.prefill(q, dev_i32(cu), run.pool, run.bt, run.sl, run.max_ctx, 8, workspace=ws)
        with pytest.raises(MLAError):
            run.ctx.prefill(q, dev_i32(cu), run.pool, run.bt, run.sl, 4, 8)
    finally:
        run.free()
    ctx32 = MLAContext(dev(w.kv_b_proj(), "f32"), None, num_heads=16, dtype="f32", max_q_tokens=8, max_batch=1,
                       max_position=64, max_seq_len=64)
    try:
        pool32 = torch.zeros((w.n_blocks, 16, 1, 576), dtype=torch.float32, device="cuda")
        q32 = dev(w.chunk_queries([8]), "f32")
        with pytest.raises(MLAError):
            ctx32.prefill(q32, dev_i32(cu), pool32, dev_i32(w.block_table), dev_i32(w.seq_lens), 48, 8)
    finally:
        ctx32.free()


def test_prefill_full_size_sampled():
    """The benchmark's configuration and launch (4 sequences, each a fresh chunk of 4,096 tokens, 16
    heads, the same seed): sampled rows against the oracle.  A causal row depends only on the tokens
    up to its own position, so the last 8 rows of each sequence are the oracle's prefill of an
    8-token chunk over the whole context, and the first 8 rows its prefill of an 8-token context (the
    first 8 tokens, the same cache rows)."""
    B, S, R = 4, 4096, 8
    w = W.custom(f"prefill_b{B}_s{S}", "bf16", 16, [S] * B, q_len=1, seed=1240)
    _say("prefill full size", B, "x", S, "sampled rows", R, "first and last per sequence")
    W_uk, W_uv = oracle_weights(w)
    tok = w.all_tokens()
    cache = O.cache_write(np.full((w.n_blocks, 16, 1, 576), np.nan), tok["c_kv"], tok["k_pe"], tok["positions"],
                          tok["slot_mapping"], w.gamma().astype(np.float64), w.eps, w.theta, w.storage)
    q = w.chunk_queries([S] * B)
    cu_r = _cu([R] * B)
    last_rows = np.concatenate([np.arange(b * S + S - R, b * S + S) for b in range(B)])
    first_rows = np.concatenate([np.arange(b * S, b * S + R) for b in range(B)])
    ref_last = O.prefill_naive(q[last_rows], cu_r, cache, w.block_table, w.seq_lens, W_uk, W_uv, w.scale, w.theta)
    ref_first = O.prefill_naive(q[first_rows], cu_r, cache, w.block_table, np.full(B, R), W_uk, W_uv, w.scale,
                                w.theta)
    run = DeviceRun(w)
    try:
        out = _run_prefill(run, [S] * B)
        compare(out[torch.from_numpy(last_rows).cuda()], ref_last, "bf16", "prefill full size, last rows")
        compare(out[torch.from_numpy(first_rows).cuda()], ref_first, "bf16", "prefill full size, first rows")
    finally:
        run.free()
