"""GPU: mla_decode_step (the step's cache write and the decode in one call) through the C ABI.

Each case starts from a pool that holds only the history tokens (NaN-poisoned elsewhere for bf16 and
fp32 rows, zero bytes for FP8 rows), then runs the step on the new tokens two ways on two copies of
that pool:
  * mla_cache_write followed by mla_decode (the two calls the step stands for);
  * mla_decode_step.
The written pools and the outputs must match bit for bit (with bf16 storage the cache write runs in
the query absorption's launch; with fp32 storage the step launches it on its own first).  The step's
output is also checked against the fp64 oracle (oracle_full: every context token written, then the
absorbed decode) to the contract's tolerance.  Argument errors of either half are refused before
anything runs: the pool is left as it was."""

import numpy as np
import pytest

from workloads import mla_inputs as W

from ._harness import compare, dev, dev_i32, oracle_full

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


def _bits(t):
    """Tensor -> integer view of its bytes (NaN payloads compare exactly)."""
    return t.contiguous().view(torch.uint8).cpu().numpy()


class StepRun:
    def __init__(self, w, mode):
        from mla_latent_kv_paged_amd import MLAContext
        self.w, self.mode = w, mode
        st = "bf16" if mode == "fp8" else w.storage
        self.st = st
        self.max_ctx = int(w.seq_lens.max())
        self.ctx = MLAContext(dev(w.kv_b_proj(), st), dev(w.gamma(), st) if w.gamma_noise else None,
                              num_heads=w.num_heads, dtype=mode, rms_eps=w.eps, rope_theta=w.theta,
                              max_q_tokens=w.n_q, max_batch=w.batch, max_position=self.max_ctx + 16,
                              max_seq_len=self.max_ctx + 16)
        if mode == "fp8":
            self.pool = torch.zeros((w.n_blocks, 16, 1, 656), dtype=torch.uint8, device="cuda")
        else:
            self.pool = torch.full((w.n_blocks, 16, 1, 576), float("nan"),
                                   dtype=torch.bfloat16 if st == "bf16" else torch.float32, device="cuda")
        h = w.all_tokens(history_only=True)
        if len(h["positions"]):
            self.ctx.cache_write(dev(h["c_kv"], st), dev(h["k_pe"], st), dev_i32(h["positions"]),
                                 dev_i32(h["slot_mapping"]), self.pool)
        n = w.all_tokens(new_only=True)
        self.new = (dev(n["c_kv"], st), dev(n["k_pe"], st), dev_i32(n["positions"]), dev_i32(n["slot_mapping"]))
        self.q = dev(w.queries(), st)
        self.bt = dev_i32(w.block_table)
        self.sl = dev_i32(w.seq_lens)
        torch.cuda.synchronize()

    def two_calls(self, pool):
        self.ctx.cache_write(*self.new, pool)
        out = self.ctx.decode(self.q, pool, self.bt, self.sl, self.max_ctx, q_len=self.w.q_len)
        torch.cuda.synchronize()
        return out

    def step(self, pool):
        out = self.ctx.decode_step(*self.new, self.q, pool, self.bt, self.sl, self.max_ctx, q_len=self.w.q_len)
        torch.cuda.synchronize()
        return out


STEP_CASES = [
    # name, cache mode, heads, context lengths, q_len
    ("bf16_h16", "bf16", 16, [700, 33, 258, 1025], 1),     # 16-row decode kernel
    ("bf16_h32_q2", "bf16", 32, [300, 2, 129], 2),        # 32-row kernel, two new tokens per sequence
    ("fp8_h16", "fp8", 16, [517, 64, 1000], 1),
    ("f32_h16", "f32", 16, [90, 17, 300], 1),             # separate launches
]


@pytest.mark.parametrize("name,mode,heads,ctxs,q_len", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_matches_two_calls(name, mode, heads, ctxs, q_len):
    storage = "f32" if mode == "f32" else "bf16"
    w = W.custom("step_" + name, storage, heads, ctxs, q_len=q_len, seed=170 + heads + q_len)
    _say("decode_step", name, "H", heads, "ctx", ctxs, "q_len", q_len)
    run = StepRun(w, mode)
    try:
        p1, p2 = run.pool.clone(), run.pool.clone()
        o1 = run.two_calls(p1)
        o2 = run.step(p2)
        assert np.array_equal(_bits(p1), _bits(p2)), "cache rows differ"
        assert np.array_equal(_bits(o1), _bits(o2)), "outputs differ"
        if mode != "fp8":  # the FP8 rows are checked against the oracle's format in test_gpu_fp8.py
            _, ref = oracle_full(w)
            compare(o2, ref, storage, f"decode_step {name}")
        # a second step on the written pool (the write is idempotent) gives the same output
        assert np.array_equal(_bits(o2), _bits(run.step(p2)))
    finally:
        run.ctx.free()


def test_decode_step_refuses_bad_arguments_before_writing():
    from mla_latent_kv_paged_amd import MLAError
    w = W.custom("step_err", "bf16", 16, [40, 20], q_len=1, seed=181)
    run = StepRun(w, "bf16")
    try:
        before = _bits(run.pool)
        # decode half invalid (max_seq_len below q_len): nothing may be written
        with pytest.raises(MLAError):
            run.ctx.decode_step(*run.new, run.q, run.pool, run.bt, run.sl, 0, q_len=1)
        # decode half over the context's caps
        with pytest.raises(MLAError):
            run.ctx.decode_step(*run.new, run.q, run.pool, run.bt, run.sl, run.max_ctx + 1000, q_len=1)
        torch.cuda.synchronize()
        assert np.array_equal(before, _bits(run.pool)), "a refused step wrote the cache"
        # no new tokens: the step is the decode alone
        empty = (torch.empty((0, 512), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((0,), dtype=torch.int32, device="cuda"), torch.empty((0,), dtype=torch.int32, device="cuda"))
        p1, p2 = run.pool.clone(), run.pool.clone()
        run.ctx.cache_write(*run.new, p1)
        run.ctx.cache_write(*run.new, p2)
        o1 = run.ctx.decode(run.q, p1, run.bt, run.sl, run.max_ctx, q_len=1)
        o2 = run.ctx.decode_step(*empty, run.q, p2, run.bt, run.sl, run.max_ctx, q_len=1)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o1), _bits(o2))
        assert np.array_equal(_bits(p1), _bits(p2))
    finally:
        run.ctx.free()


def test_decode_step_full_size_matches_two_calls():
    """The benchmark's step at full size (lite_b64: 64 sequences x 4,096 cached + 1 new token, 16 heads,
    bf16 pool of 20,000 blocks, the library's own launch): mla_decode_step against mla_cache_write +
    mla_decode on copies of the pool, bit for bit.  (The decode itself is checked against the oracle at
    this size in test_gpu_parity.py.)"""
    w = W.lite_b64()
    _say("decode_step full size: lite_b64")
    run = StepRun(w, "bf16")
    try:
        p1, p2 = run.pool.clone(), run.pool.clone()
        o1 = run.two_calls(p1)
        o2 = run.step(p2)
        assert torch.equal(p1.view(torch.int16), p2.view(torch.int16)), "cache rows differ"
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "outputs differ"
    finally:
        run.ctx.free()
