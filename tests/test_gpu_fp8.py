"""GPU parity of the FP8 cache mode (MLA_BF16_FP8): the HIP library through the C ABI against the
fp64 oracle (oracle/mla_fp8.py for the cache format, oracle/mla_oracle.py for attention).

* Cache write: every row's bytes against the oracle's.  The codes are integers decided by fp64
  arithmetic on both sides; the sum of squares inside RMSNorm is reduced in a different order
  (NumPy pairwise vs the kernel's lane tree), which moves a normed value by an ulp or so.  So a
  code may differ by one step where the oracle's quotient lies within 1e-9 (relative) of the tie
  between the two codes, a scale by one fp32 step where amax / 448 lies that close to an fp32
  midpoint, and a rope value by one bf16 ulp; anything else fails.
* Decode: the oracle's bytes are copied into the GPU's pool, and the kernel's output over them is
  compared with the oracle's absorbed decode over the same bytes decoded by the oracle's format
  decoder, to the bf16 tolerance (max abs 2e-2, relative L2 5e-3)."""

import numpy as np
import pytest

from oracle import mla_fp8 as F
from oracle import mla_oracle as O
from workloads import mla_inputs as W

from ._harness import bf16_ulp_distance, compare, dev, dev_i32, oracle_all_sequences, oracle_weights

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


class Fp8Run:
    """Context in FP8-cache mode, a zeroed byte pool, every context token written by the kernel."""

    def __init__(self, w, fill=0):
        from mla_latent_kv_paged_amd import MLAContext
        self.w = w
        self.max_ctx = int(w.seq_lens.max())
        self.ctx = MLAContext(dev(w.kv_b_proj(), "bf16"), dev(w.gamma(), "bf16") if w.gamma_noise else None,
                              num_heads=w.num_heads, dtype="fp8", rms_eps=w.eps, rope_theta=w.theta,
                              max_q_tokens=w.n_q, max_batch=w.batch, max_position=self.max_ctx + 16,
                              max_seq_len=self.max_ctx + 16)
        self.pool = torch.full((w.n_blocks, 16, 1, F.ROW_BYTES), fill, dtype=torch.uint8, device="cuda")
        self.tok = w.all_tokens()
        t = self.tok
        self.ctx.cache_write(dev(t["c_kv"], "bf16"), dev(t["k_pe"], "bf16"), dev_i32(t["positions"]),
                             dev_i32(t["slot_mapping"]), self.pool)
        self.q = dev(w.queries(), "bf16")
        self.bt = dev_i32(w.block_table)
        self.sl = dev_i32(w.seq_lens)

    def decode(self, split_blocks=None, waves=0):
        if split_blocks is not None or waves:
            self.ctx.set_decode_tuning(split_blocks or 0, waves)
        out = self.ctx.decode(self.q, self.pool, self.bt, self.sl, self.max_ctx, q_len=self.w.q_len)
        torch.cuda.synchronize()
        if split_blocks is not None or waves:
            self.ctx.set_decode_tuning(0, 0)
        return out

    def pool_bytes(self):
        return self.pool.cpu().numpy()

    def load_pool(self, pool8):
        """Replace the pool's bytes by the given ones (the oracle's)."""
        self.pool.copy_(torch.from_numpy(np.ascontiguousarray(pool8)))
        torch.cuda.synchronize()

    def free(self):
        self.ctx.free()


def _oracle_cache(w):
    t = w.all_tokens()
    pool = np.zeros((w.n_blocks, 16, 1, F.ROW_BYTES), dtype=np.uint8)
    return F.cache_write_fp8(pool, t["c_kv"], t["k_pe"], t["positions"], t["slot_mapping"],
                             w.gamma().astype(np.float64), w.eps, w.theta)


def _check_fp8_cache(got, ref, w):
    """Compare byte pools row by row (see the module docstring for the allowances)."""
    t = w.all_tokens()
    slots = t["slot_mapping"]
    written = np.zeros(got.shape[:2], dtype=bool)
    written[slots // 16, slots % 16] = True
    assert np.array_equal(got[~written], ref[~written]), "bytes outside the written slots changed"
    g = got[written].reshape(-1, F.ROW_BYTES)
    r = ref[written].reshape(-1, F.ROW_BYTES)
    # scales
    gs = g[:, 640:].copy().view("<f4").astype(np.float64)
    rs = r[:, 640:].copy().view("<f4").astype(np.float64)
    diff_s = gs != rs
    assert np.mean(diff_s) <= 1e-3, f"scales differ in {np.sum(diff_s)} groups"
    for i, k in zip(*np.where(diff_s)):
        assert abs(np.float32(gs[i, k]).view(np.int32) - np.float32(rs[i, k]).view(np.int32)) == 1
    # rope values (bf16)
    gr = (g[:, 512:640].copy().view("<u2").astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rr = (r[:, 512:640].copy().view("<u2").astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = bf16_ulp_distance(gr, rr)
    assert np.max(d) <= 1.0 and np.mean(d > 0) <= 1e-4
    # codes, in groups whose scale matches: one step apart at most, and only next to a tie
    gc, rc = g[:, :512], r[:, :512]
    same_scale = ~np.repeat(diff_s, 128, axis=1)
    bad = (gc != rc) & same_scale
    assert np.mean(bad) <= 1e-4, f"{np.sum(bad)} codes differ"
    if np.any(bad):
        vals = F.e4m3_values()
        gamma = w.gamma().astype(np.float64)
        order = np.argsort(slots)  # written rows come out in slot order: row i is token order[i]
        for i, k in zip(*np.where(bad)):
            a, b = vals[gc[i, k]], vals[rc[i, k]]
            assert abs(int(gc[i, k]) - int(rc[i, k])) == 1, (i, k, a, b)
            j = order[i]
            c = O.rms_norm(t["c_kv"][j].astype(np.float64), gamma, w.eps)
            qv = c[k] / rs[i, k // 128]
            tie = (abs(a) + abs(b)) / 2
            assert abs(abs(qv) - tie) <= 1e-9 * abs(qv), (i, k, qv, tie)


FP8_CASES = [
    ("lite_b4_s300", lambda: W.lite_b64(batch=4, seq_len=300, n_blocks=200)),
    ("h128_b2", lambda: W.wide(batch=2, lo=100, hi=700)),
    ("ragged_b6_q4", lambda: W.ragged(batch=6, median=200, hi=900)),
    ("edges_q1", lambda: W.custom("fp8e", "bf16", 16, [1, 2, 16, 17, 33], q_len=1, seed=41)),
    ("gamma_q2", lambda: W.custom("fp8g", "bf16", 32, [70, 129], q_len=2, seed=42, gamma_noise=0.1)),
]


@pytest.mark.parametrize("name,make", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_cache_and_decode(name, make):
    w = make()
    _say("fp8", name, "H", w.num_heads, "q_len", w.q_len, list(w.seq_lens)[:6])
    ref_pool = _oracle_cache(w)
    run = Fp8Run(w)
    try:
        _check_fp8_cache(run.pool_bytes(), ref_pool, w)
        run.load_pool(ref_pool)
        W_uk, W_uv = oracle_weights(w)
        deq = F.dequantize_cache(ref_pool)
        ref = O.decode_absorbed(w.queries(), deq, w.block_table, w.seq_lens, w.q_len, W_uk, W_uv, w.scale, w.theta)
        out = run.decode()
        compare(out, ref, "bf16", f"fp8 {name}")
        for sb in (1, 3, 5):  # short splits: many partials per row, the empty-split markers
            for waves in (2, 4):  # waves sharing a query tile (4 is the default)
                compare(run.decode(split_blocks=sb, waves=waves), ref, "bf16", f"fp8 {name} split {sb} waves {waves}")
        compare(run.decode(waves=2), ref, "bf16", f"fp8 {name} waves 2")
        out2 = run.decode()
        assert torch.equal(out, out2), "fp8 decode is not deterministic"
    finally:
        run.free()


def test_fp8_quantisation_error_is_bounded():
    """The FP8 cache costs accuracy against the bf16 cache; on N(0,1) data the output's relative L2
    distance to the unquantised fp64 result stays within the e4m3 spacing (2^-4 relative)."""
    w = W.lite_b64(batch=4, seq_len=300, n_blocks=200)
    run = Fp8Run(w)
    try:
        out = run.decode().to(torch.float32).cpu().numpy().astype(np.float64)
        W_uk, W_uv = oracle_weights(w)
        t = w.all_tokens()
        exact = O.cache_write(np.full((w.n_blocks, 16, 1, 576), np.nan), t["c_kv"], t["k_pe"], t["positions"],
                              t["slot_mapping"], w.gamma().astype(np.float64), w.eps, w.theta, "f32")
        ref = O.decode_absorbed(w.queries(), exact, w.block_table, w.seq_lens, w.q_len, W_uk, W_uv, w.scale,
                                w.theta)
        rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
        _say("fp8 vs unquantised: rel L2", rel)
        assert rel <= 2.0 ** -4
    finally:
        run.free()


def _fp8_pool_from_values(w, pool):
    """FP8 byte pool holding the live rows of a float32 value pool (quantised by the oracle's
    format code); every other row is 0xFF bytes (NaN codes, NaN rope values, NaN scales), so a
    kernel that reads a row it should not see yields NaN."""
    out = np.full((w.n_blocks, 16, 1, F.ROW_BYTES), 0xFF, dtype=np.uint8)
    for b in range(w.batch):
        for t in range(int(w.seq_lens[b])):
            blk, off = int(w.block_table[b, t // 16]), t % 16
            v = pool[blk, off, 0].astype(np.float64)
            codes, scales = F.quantize_latent(v[:512])
            out[blk, off, 0] = F.pack_row(codes, v[512:], scales)
    return out


@pytest.mark.parametrize("heads,q_len", [(16, 1), (16, 2)])
def test_fp8_score_climb(heads, q_len):
    """The steadily climbing scores of the bf16 test (test_gpu_parity.climb_case) over an FP8
    cache, with both wave counts and the longest splits, against the oracle on the dequantised
    bytes; the rows past each sequence's end are NaN bytes."""
    from mla_latent_kv_paged_amd import MLAContext
    from .test_gpu_parity import climb_case, climb_rows
    w, q, kvb, pool = climb_case(heads, q_len, seed=82)
    _say("fp8 score climb", "H", heads, "q_len", q_len)
    pool8 = _fp8_pool_from_values(w, pool)
    deq = F.dequantize_cache(pool8)
    assert climb_rows(w, q, kvb, deq.astype(np.float32)) >= heads
    W_uk, W_uv = O.absorb(kvb.astype(np.float64), heads, 128, 128)
    ref = O.decode_absorbed(q, deq, w.block_table, w.seq_lens, w.q_len, W_uk, W_uv, w.scale, w.theta)
    mx = int(w.seq_lens.max())
    ctx = MLAContext(dev(kvb, "bf16"), None, num_heads=heads, dtype="fp8", rms_eps=w.eps, rope_theta=w.theta,
                     max_q_tokens=w.n_q, max_batch=w.batch, max_position=mx + 16, max_seq_len=mx + 16)
    try:
        dpool = torch.from_numpy(pool8).to("cuda")
        for sb, waves in ((0, 0), (160, 4), (160, 2), (3, 4)):
            ctx.set_decode_tuning(sb, waves)
            out = ctx.decode(dev(q, "bf16"), dpool, dev_i32(w.block_table), dev_i32(w.seq_lens), mx, q_len=w.q_len)
            torch.cuda.synchronize()
            compare(out, ref, "bf16", f"fp8 score climb H={heads} q_len={q_len} split={sb} waves={waves}")
    finally:
        ctx.free()


def test_fp8_full_size_every_sequence():
    """The benchmark's FP8 configuration and launch (lite_b64: 64 sequences x 4,097 tokens, 16 heads,
    FP8 rows, the library's own split).  The kernel's cache write of every token against the oracle's
    bytes; then, over the oracle's bytes, every sequence against the oracle's absorbed decode (each
    computed on an identity-paged local pool of that sequence's blocks)."""
    w = W.lite_b64()
    _say("fp8 full size: lite_b64, every sequence")
    ref, ref_pool = oracle_all_sequences(w, fp8=True)
    run = Fp8Run(w, fill=0xFF)
    try:
        _check_fp8_cache(run.pool_bytes(), ref_pool, w)
        run.load_pool(ref_pool)
        res = run.decode().to(torch.float32).cpu().numpy().astype(np.float64)
    finally:
        run.free()
    for b in range(w.batch):
        rows = slice(b * w.q_len, (b + 1) * w.q_len)
        compare(res[rows], ref[rows], "bf16", f"fp8 full size, sequence {b}")
    max_abs, rel = compare(res, ref, "bf16", "fp8 full size, whole output")
    _say(f"fp8 full size: max abs {max_abs:.3e}, rel L2 {rel:.3e}")
