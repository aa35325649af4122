"""Shared test plumbing: run a seeded workload through the HIP library (via the binding) and
through the fp64 oracle.  The two sides share only the seeded inputs from workloads/."""

from __future__ import annotations

import math

import numpy as np

from oracle import mla_oracle as O
from workloads import mla_inputs as W

# tolerances of the contract
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_MAX_ABS = 1e-4


def torch_dtype(storage):
    import torch
    return torch.bfloat16 if storage == "bf16" else torch.float32


def dev(x, storage):
    """float32 numpy values (exactly representable in the storage dtype) -> device tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch_dtype(storage))


def dev_i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


class DeviceRun:
    """A workload resident on the GPU: context, NaN-poisoned pool, written cache."""

    def __init__(self, w: W.Workload, max_ctx=None, per_sequence_upload=False, extra_caps=0):
        import torch
        from mla_latent_kv_paged_amd import MLAContext
        self.w = w
        self.storage = w.storage
        self.max_ctx = int(max_ctx or w.seq_lens.max())
        self.ctx = MLAContext(dev(w.kv_b_proj(), w.storage),
                              dev(w.gamma(), w.storage) if w.gamma_noise else None,
                              num_heads=w.num_heads, dtype=w.storage, rms_eps=w.eps, rope_theta=w.theta,
                              max_q_tokens=w.n_q + extra_caps, max_batch=w.batch + extra_caps,
                              max_position=self.max_ctx + 16, max_seq_len=self.max_ctx + 16)
        self.pool = torch.full((w.n_blocks, 16, 1, 576), float("nan"), dtype=torch_dtype(w.storage), device="cuda")
        if per_sequence_upload:
            for b in range(w.batch):
                c, k = w.history(b)
                ctxb = int(w.seq_lens[b])
                self.ctx.cache_write(dev(c, w.storage), dev(k, w.storage), dev_i32(np.arange(ctxb)),
                                     dev_i32(w.slots(b, 0, ctxb)), self.pool)
        else:
            tok = w.all_tokens()
            self.ctx.cache_write(dev(tok["c_kv"], w.storage), dev(tok["k_pe"], w.storage),
                                 dev_i32(tok["positions"]), dev_i32(tok["slot_mapping"]), self.pool)
        self.q = dev(w.queries(), w.storage)
        self.bt = dev_i32(w.block_table)
        self.sl = dev_i32(w.seq_lens)

    def decode(self, pool=None, split_blocks=None, waves=0):
        import torch
        if split_blocks is not None or waves:
            self.ctx.set_decode_tuning(split_blocks or 0, waves)
        out = self.ctx.decode(self.q, self.pool if pool is None else pool, self.bt, self.sl, self.max_ctx,
                              q_len=self.w.q_len)
        torch.cuda.synchronize()
        if split_blocks is not None or waves:
            self.ctx.set_decode_tuning(0, 0)
        return out

    def pool_f64(self):
        import torch
        return self.pool.to(torch.float32).cpu().numpy().astype(np.float64)

    def free(self):
        self.ctx.free()


def oracle_weights(w):
    kvb = w.kv_b_proj().astype(np.float64)
    return O.absorb(kvb, w.num_heads, w.qk_nope_head_dim, w.v_head_dim)


def oracle_full(w):
    """Oracle cache (NaN pool, every context token written) and absorbed decode output."""
    W_uk, W_uv = oracle_weights(w)
    tok = w.all_tokens()
    pool = np.full((w.n_blocks, 16, 1, 576), np.nan)
    cache = O.cache_write(pool, tok["c_kv"], tok["k_pe"], tok["positions"], tok["slot_mapping"],
                          w.gamma().astype(np.float64), w.eps, w.theta, w.storage)
    out = O.decode_absorbed(w.queries(), cache, w.block_table, w.seq_lens, w.q_len, W_uk, W_uv, w.scale, w.theta)
    return cache, out


def oracle_sequence(w, b, W_uk=None, W_uv=None, q=None, fp8=False):
    """Oracle output rows of sequence b alone, computed on an identity-paged local pool
    (paging relabel invariance makes the physical placement irrelevant).  q: w.queries(), if the
    caller already holds it.  fp8: the cache holds the oracle's FP8 rows (oracle/mla_fp8.py) and the
    decode reads their dequantised values; returns (rows, the local pool's bytes [nb, 16, 1, 656],
    rows past the context 0xFF)."""
    from oracle import mla_fp8 as F
    if W_uk is None:
        W_uk, W_uv = oracle_weights(w)
    if q is None:
        q = w.queries()
    ctx = int(w.seq_lens[b])
    nb = (ctx + 15) // 16
    c, k = w.history(b)
    gamma = w.gamma().astype(np.float64)
    if fp8:
        local = F.cache_write_fp8(np.full((nb, 16, 1, F.ROW_BYTES), 0xFF, np.uint8), c, k, np.arange(ctx),
                                  np.arange(ctx), gamma, w.eps, w.theta)
        cache = F.dequantize_cache(local)
    else:
        cache = O.cache_write(np.full((nb, 16, 1, 576), np.nan), c, k, np.arange(ctx), np.arange(ctx), gamma,
                              w.eps, w.theta, w.storage)
    rows = O.decode_absorbed(q[b * w.q_len:(b + 1) * w.q_len], cache, np.arange(nb)[None, :], np.array([ctx]),
                             w.q_len, W_uk, W_uv, w.scale, w.theta)
    return (rows, local) if fp8 else rows


def _oracle_rows_task(args):
    """Worker of oracle_all_sequences: the oracle rows of a list of sequences (one BLAS thread)."""
    w, seqs, fp8 = args
    try:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(1)
    except Exception:  # pragma: no cover
        lim = None
    W_uk, W_uv = oracle_weights(w)
    q = w.queries()
    res = [(b, oracle_sequence(w, b, W_uk, W_uv, q, fp8)) for b in seqs]
    if lim is not None:
        lim.unregister()
    return res


def oracle_all_sequences(w, seqs=None, workers=None, fp8=False):
    """oracle_sequence for every sequence (or those in seqs), spread over worker processes started
    fresh (spawn: they import NumPy and the oracle only, never the GPU).  Returns [B*q_len, H, dv]
    float64 rows; rows of sequences not asked for are NaN.  fp8: returns (rows, the FP8 byte pool
    [n_blocks, 16, 1, 656] with each sequence's oracle rows at its block table's blocks, every other
    byte 0xFF)."""
    import concurrent.futures
    import multiprocessing
    import os
    seqs = list(range(w.batch) if seqs is None else seqs)
    n = max(1, min(workers or 16, len(os.sched_getaffinity(0)), len(seqs)))
    # longest first, dealt round robin, so that the workers finish together
    order = sorted(seqs, key=lambda b: -int(w.seq_lens[b]))
    parts = [order[i::n] for i in range(n)]
    out = np.full((w.n_q, w.num_heads, w.v_head_dim), np.nan)
    pool = np.full((w.n_blocks, 16, 1, 656), 0xFF, np.uint8) if fp8 else None
    with concurrent.futures.ProcessPoolExecutor(n, mp_context=multiprocessing.get_context("spawn")) as ex:
        for res in ex.map(_oracle_rows_task, [(w, p, fp8) for p in parts]):
            for b, r in res:
                if fp8:
                    r, local = r
                    pool[w.block_table[b, :len(local)]] = local
                out[b * w.q_len:(b + 1) * w.q_len] = r
    return (out, pool) if fp8 else out


def compare(out_gpu, ref, storage, label=""):
    """Assert the contract tolerance; returns (max_abs, rel_l2)."""
    import torch
    got = out_gpu.to(torch.float32).cpu().numpy().astype(np.float64) if hasattr(out_gpu, "cpu") else out_gpu
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = got - ref
    max_abs = float(np.max(np.abs(err)))
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    if storage == "bf16":
        assert max_abs <= BF16_MAX_ABS, f"{label}: max abs {max_abs}"
        assert rel <= BF16_REL_L2, f"{label}: rel L2 {rel}"
    else:
        assert max_abs <= F32_MAX_ABS, f"{label}: max abs {max_abs}"
    return max_abs, rel


def bf16_ulp_distance(a, b):
    """|a - b| in units of bf16 spacing at max(|a|,|b|) (both arrays of bf16 values)."""
    m = np.maximum(np.abs(a), np.abs(b))
    e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    ulp = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.abs(a - b) / ulp


def sample_rows_of(w, b):
    return slice(b * w.q_len, (b + 1) * w.q_len)


def isclose_scale():
    return 1.0 / math.sqrt(192.0)
