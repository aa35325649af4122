#!/usr/bin/env python3
"""Benchmark of one MLA decode step over the paged latent cache on one MI355X.

A step is one pass of the whole per-token hot path on one batch: mla_cache_write of the
batch's new tokens (RMSNorm + RoPE + scatter) followed by mla_decode (query absorption, split-KV
attention over the latent cache, log-sum-exp combine fused with W_uv).  The weight split
(mla_absorb_weights) runs once per layer at load time; its time is reported separately.

Default workload: DeepSeek-V2-Lite shapes (16 heads, kv_lora_rank 512, rope 64), batch 64,
4096 cached tokens + 1 new token per sequence, bf16 cache of 20,000 blocks x 16 slots, blocks
shuffled over the pool.  Inputs are seeded synthetic data.  Three copies of the cache pool are
rotated between steps so that consecutive steps never re-read the same 302 MB (the 256 MB
Infinity Cache cannot serve a step from the previous one); each layer of a real model reads
its own cache once per step in the same way.

Prints ONE JSON line.  `value` = algorithmic latent-cache bytes per step / step time (GB/s).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/step + achieved latent-cache GB/s, V2-Lite b=64 s=4096"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mla_latent_kv_paged_amd", "csrc")
# committed rocprofv3 FETCH/WRITE summaries per default workload, and the kernel source they were taken on
TRAFFIC = {"lite_b64": ("decode_bf16_lite_b64_s4096_traffic.json", "decode_bf16.hip"),
           "wide": ("decode_bf16_mt32_wide_h128_b128_traffic.json", "decode_bf16_mt32.hip"),
           "ragged": ("decode_bf16_mt32_ragged_b256_q4_traffic.json", "decode_bf16_mt32.hip")}
TRAFFIC_FP8 = {"lite_b64": ("decode_fp8_lite_b64_s4096_traffic.json", "decode_fp8.hip")}
# the chunked prefill's attention kernel at the default prefill sizes (4 sequences x 4,096 tokens)
TRAFFIC_PF = ("prefill_attn_b4_s4096_traffic.json", "prefill_attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="lite_b64", choices=["lite_b64", "wide", "ragged", "lite_b1"])
    ap.add_argument("--seq-len", type=int, default=0, help="cached tokens per sequence (lite_b1: default 1024; "
                    "lite_b64: default 4096)")
    ap.add_argument("--batch", type=int, default=0, help="batch for lite_b64 (default 64)")
    ap.add_argument("--rotate", type=int, default=3, help="cache pool copies rotated between steps")
    ap.add_argument("--cache", default="native", choices=["native", "fp8"],
                    help="native: the workload's storage dtype (bf16 for the benchmark workloads); fp8: "
                         "FP8 E4M3 latent rows of 656 bytes (MLA_BF16_FP8), bf16 everything else")
    ap.add_argument("--split-blocks", type=int, default=0, help="force the split size (0 = library choice)")
    ap.add_argument("--waves", type=int, default=0, help="force waves per decode workgroup (0 = library choice)")
    ap.add_argument("--separate-write", action="store_true",
                    help="step as mla_cache_write + mla_decode (two calls) instead of mla_decode_step, which "
                         "runs the cache write in the query absorption's launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unflushed", action="store_true",
                    help="also time steps that all read the same pool (pass D: the pool may sit in the Infinity Cache)")
    ap.add_argument("--cpu-sample", type=int, default=256, help="sequences in the oracle's timed sample (capped at "
                    "the batch)")
    ap.add_argument("--pf-batch", type=int, default=4, help="prefill mode: sequences")
    ap.add_argument("--pf-len", type=int, default=4096, help="prefill mode: tokens per sequence, all new (fresh "
                    "prefill: the chunk is the whole context)")
    ap.add_argument("--layers", type=int, default=1, help="layer mode: attention layers in the model step (each "
                    "with its own weights and cache)")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy-calibration", "decode-only", "prefill",
                                                        "prefill-only", "layer", "layer-only", "ceiling",
                                                        "mfma-calibration"],
                    help="copy-calibration: run a plain 256 MiB device copy (for counter scaling); "
                         "decode-only: run just the decode loop (for profilers); ceiling: the decode kernel "
                         "beside a plain streaming read of the same byte count and the decode's block gather "
                         "alone (no math); mfma-calibration: the matrix cores' issue rate (mla_ceiling_mfma), "
                         "the reference for the MFMA-busy counter")
    return ap.parse_args()


def make_workload(args):
    from workloads import mla_inputs as W
    if args.workload == "lite_b64":
        if args.seq_len or args.batch:
            S, B = args.seq_len or 4096, args.batch or 64
            nb = B * ((S + 1 + 15) // 16)
            return W.lite_b64(batch=B, seq_len=S, n_blocks=max(20000, int(nb * 1.25)))
        return W.lite_b64()
    if args.workload == "wide":
        return W.wide()
    if args.workload == "ragged":
        return W.ragged()
    return W.lite_b1(args.seq_len or 1024)


def describe(w):
    return {
        "workload": f"{w.name}: MLA decode, {w.num_heads} heads, kv_lora_rank 512 + rope 64, batch {w.batch}, "
                    f"q_len {w.q_len}, context {int(w.seq_lens.min())}..{int(w.seq_lens.max())} tokens "
                    f"(sum {w.total_ctx}), {w.storage} paged cache [{w.n_blocks},16,1,576], shuffled block table",
        "batch": w.batch, "q_len": w.q_len, "num_heads": w.num_heads,
        "max_ctx": int(w.seq_lens.max()), "sum_ctx": w.total_ctx, "pool_blocks": w.n_blocks,
    }


def copy_calibration():
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy-calibration", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": 5}), flush=True)


def mfma_calibration(args):
    """mla_ceiling_mfma for both shapes (independent chains of v_mfma_f32_16x16x32_bf16, or of
    v_mfma_f32_32x32x16_bf16, four waves per SIMD, 1,000 rounds per launch), each launch timed by events;
    their MFMA-busy and GPU-active counters (taken in a profiler pass of this mode) define a fully
    issued matrix pipe for each shape."""
    import numpy as np
    import torch
    from mla_latent_kv_paged_amd import _lib as L
    L.load()
    sink = torch.empty((1 << 20) // 4, dtype=torch.int32, device="cuda")
    iters = 1000
    res = {"mode": "mfma-calibration", "iterations": iters}
    for shape, name in ((0, "16x16x32_bf16"), (1, "32x32x16_bf16")):
        for _ in range(max(1, args.warmup)):
            L.ceiling_mfma(shape, iters, sink)
        n = max(1, args.steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        flops = 0.0
        for i in range(n):
            ev[i][0].record()
            flops = L.ceiling_mfma(shape, iters, sink)
            ev[i][1].record()
        torch.cuda.synchronize()
        med = float(np.median(np.array([a_.elapsed_time(b_) for a_, b_ in ev]) * 1e3))
        res[name] = {"launches": n, "flops_per_launch": flops, "us_median": round(med, 2),
                     "tflops_median": round(flops / (med * 1e-6) / 1e12, 1),
                     "fraction_of_bf16_peak": round(flops / (med * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    print(json.dumps(res), flush=True)


def kernel_source_sha(src):
    """sha256 of a kernel's source followed by the internal headers it includes (the prefill kernels'
    shared header, then mla_internal.h)."""
    h = hashlib.sha256()
    for f in (src,) + (("prefill_common.h",) if src.startswith("prefill") else ()) + ("mla_internal.h",):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def prefill_traffic(args):
    """HBM traffic of the prefill attention kernel from its committed rocprofv3 --pmc summary (default
    sizes only), if it was taken on the current kernel source; else None."""
    if args.pf_batch != 4 or args.pf_len != 4096:
        return None
    fname, src = TRAFFIC_PF
    path = os.path.join(PROFILES, fname)
    try:
        rec = json.load(open(path))
        if rec.get("kernel_source_sha256") != kernel_source_sha(src):
            return None
        return rec.get("traffic_bytes_per_launch")
    except Exception:
        return None


def traffic_entry(args):
    """HBM traffic of the decode kernel from the committed rocprofv3 --pmc summary of this workload
    (default sizes only), if it was taken on the current kernel source; else None."""
    table = TRAFFIC_FP8 if getattr(args, "cache", "native") == "fp8" else TRAFFIC
    if args.workload not in table or args.seq_len or args.batch:
        return None
    fname, src = table[args.workload]
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("kernel_source_sha256") != kernel_source_sha(src):
            return None
        return rec.get("traffic_bytes_per_launch")
    except Exception:
        return None


def cpu_baseline(w, n_seq, fp8=False):
    """Time the fp64 oracle (absorbed form) on a bounded sample of the same workload: the step's
    cache write of each sampled sequence's new tokens plus its full decode."""
    import numpy as np
    from oracle import mla_oracle as O
    from oracle import mla_fp8 as F
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctxmgr = threadpool_limits(cores) if threadpool_limits else None
    rng = np.random.default_rng(0)
    seqs = sorted(rng.choice(w.batch, size=min(n_seq, w.batch), replace=False).tolist())
    kvb = w.kv_b_proj().astype(np.float64)
    W_uk, W_uv = O.absorb(kvb, w.num_heads, w.qk_nope_head_dim, w.v_head_dim)
    gamma = w.gamma().astype(np.float64)
    qall = w.queries()
    prepared = []
    for b in seqs:   # history (not timed): identity-paged local pool per sequence
        ctx = int(w.seq_lens[b])
        nb = (ctx + 15) // 16
        c, k = w.history(b)
        hist = ctx - w.q_len
        if fp8:
            pool = F.cache_write_fp8(np.zeros((nb, 16, 1, F.ROW_BYTES), np.uint8), c[:hist], k[:hist],
                                     np.arange(hist), np.arange(hist), gamma, w.eps, w.theta)
        else:
            pool = O.cache_write(np.full((nb, 16, 1, 576), np.nan), c[:hist], k[:hist], np.arange(hist),
                                 np.arange(hist), gamma, w.eps, w.theta, w.storage)
        prepared.append((b, ctx, nb, c[hist:], k[hist:], pool))
    # repeat the sampled step until about 10 s of CPU work has been timed (at least 3 runs, at most
    # 30 s), and report the median run
    times = []
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 200):
        t0 = time.perf_counter()
        for b, ctx, nb, cn, kn, pool in prepared:
            if fp8:  # the FP8 write, then the values the decode sees
                cache = F.dequantize_cache(F.cache_write_fp8(pool, cn, kn, np.arange(ctx - w.q_len, ctx),
                                                             np.arange(ctx - w.q_len, ctx), gamma, w.eps, w.theta))
            else:
                cache = O.cache_write(pool, cn, kn, np.arange(ctx - w.q_len, ctx), np.arange(ctx - w.q_len, ctx),
                                      gamma, w.eps, w.theta, w.storage)
            O.decode_absorbed(qall[b * w.q_len:(b + 1) * w.q_len], cache, np.arange(nb)[None, :],
                              np.array([ctx]), w.q_len, W_uk, W_uv, w.scale, w.theta)
        times.append(time.perf_counter() - t0)
        if sum(times) > 30:
            break
    t = float(np.median(times))
    blas_threads = cores
    if threadpool_limits:
        try:
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [cores])
        except Exception:
            pass
    if ctxmgr is not None:
        ctxmgr.unregister() if hasattr(ctxmgr, "unregister") else None
    bytes_sample = sum(int(w.seq_lens[b]) for b in seqs) * (F.ROW_BYTES if fp8 else 576 * w.elem_bytes)
    return {"value": bytes_sample / t / 1e9, "unit": "GB/s", "cores": int(min(cores, blas_threads)),
            "kind": "oracle",
            "sample": f"{len(seqs)} of {w.batch} sequences (full context each); one step = cache write of the "
                      f"new token(s) + absorbed fp64 decode; median of {len(times)} runs ({sum(times):.1f} s of "
                      f"CPU work), {t:.3f} s per run; host threads available {cores}",
            "seconds_per_sample_step": t}


def prefill_flops(ctxs, chunks, H):
    """Algorithmic flops of a chunked prefill in the naive form: attention 2 (192 + 128) per (row,
    visible token) and head, expansion 2 * 512 * 256 per context token and head."""
    att = 0
    for ctx, n in zip(ctxs, chunks):
        p0 = ctx - n  # visible tokens of chunk row i: p0 + i + 1
        att += n * p0 + n * (n + 1) // 2
    return att * H * 2 * (192 + 128), sum(ctxs) * H * 2 * 512 * 256


def prefill_cpu_baseline(w, tokens=1024):
    """The fp64 oracle's prefill_naive on a bounded sample: sequence 0's first `tokens` tokens as a
    fresh chunk (identity-paged local cache, written by the oracle, not timed)."""
    import numpy as np
    from oracle import mla_oracle as O
    cores = len(os.sched_getaffinity(0))
    kvb = w.kv_b_proj().astype(np.float64)
    W_uk, W_uv = O.absorb(kvb, w.num_heads, w.qk_nope_head_dim, w.v_head_dim)
    c, k = w.history(0)
    n = min(tokens, int(w.seq_lens[0]))
    nb = (n + 15) // 16
    cache = O.cache_write(np.full((nb, 16, 1, 576), np.nan), c[:n], k[:n], np.arange(n), np.arange(n),
                          w.gamma().astype(np.float64), w.eps, w.theta, w.storage)
    q = w.chunk_queries([n] + [0] * (w.batch - 1))[:n]
    times = []
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 100):
        t0 = time.perf_counter()
        O.prefill_naive(q, np.array([0, n]), cache, np.arange(nb)[None, :], np.array([n]), W_uk, W_uv, w.scale,
                        w.theta)
        times.append(time.perf_counter() - t0)
        if sum(times) > 30:
            break
    t = float(np.median(times))
    fa, fe = prefill_flops([n], [n], w.num_heads)
    return {"value": (fa + fe) / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"sequence 0, first {n} tokens as a fresh chunk (oracle prefill_naive, fp64); median of "
                      f"{len(times)} runs, {t:.3f} s per run; host threads available {cores}"}


def prefill_main(args):
    """Chunked prefill measurement: `--pf-batch` sequences, each a fresh chunk of `--pf-len` tokens
    (16 heads, V2-Lite shapes), after a cache write of all their tokens."""
    import numpy as np
    import torch
    from mla_latent_kv_paged_amd import MLAContext, K_PF_EXPAND, K_PF_ATTN
    from workloads import mla_inputs as W
    B, S = args.pf_batch, args.pf_len
    fp8 = args.cache == "fp8"
    w = W.custom(f"prefill_b{B}_s{S}", "bf16", 16, [S] * B, q_len=1, seed=1240)
    chunks = [S] * B

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)

    def dev_i(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()

    ctx = MLAContext(dev(w.kv_b_proj()), None, num_heads=16, dtype="fp8" if fp8 else "bf16", rms_eps=w.eps,
                     rope_theta=w.theta, max_q_tokens=B, max_batch=B, max_position=S, max_seq_len=S)
    if fp8:  # e4m3 rows of 656 bytes (mla_cache_write quantises)
        pool = torch.zeros((w.n_blocks, 16, 1, 656), dtype=torch.uint8, device="cuda")
    else:
        pool = torch.full((w.n_blocks, 16, 1, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        c, k = w.history(b)
        ctx.cache_write(dev(c), dev(k), dev_i(np.arange(S)), dev_i(w.slots(b, 0, S)), pool)
    q = dev(w.chunk_queries(chunks))
    cu = dev_i(np.concatenate([[0], np.cumsum(chunks)]))
    bt, sl = dev_i(w.block_table), dev_i(w.seq_lens)
    ws = torch.empty((ctx.prefill_workspace_size(B, B * S, S),), dtype=torch.uint8, device="cuda")
    out = torch.empty((B * S, 16, 128), dtype=torch.bfloat16, device="cuda")

    def run():
        ctx.prefill(q, cu, pool, bt, sl, S, S, workspace=ws, out=out)

    if args.mode == "prefill-only":
        for _ in range(args.warmup + args.steps):
            run()
        torch.cuda.synchronize()
        print(json.dumps({"mode": "prefill-only", "launches": args.warmup + args.steps, "workload": w.name}),
              flush=True)
        return
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ctx.profile_enable(True)
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    kus = {}
    for name, kid in (("expand", K_PF_EXPAND), ("attn", K_PF_ATTN)):
        t, n = ctx.profile_read(kid)
        kus[name] = round(1e3 * t / max(n, 1), 2)
    ctx.profile_enable(False)
    fa, fe = prefill_flops([S] * B, chunks, 16)
    res = {"metric": f"MLA chunked prefill TFLOP/s, V2-Lite b={B} chunk={S} (fresh)", "value": round((fa + fe) / ms / 1e9, 2),
           "unit": "TFLOP/s", "mode": "prefill", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_prefill": round(ms, 4), "higher_is_better": True, "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) activations, N(0,1/512) kv_b_proj)",
           "config": {"workload": f"prefill_b{B}_s{S}: {B} sequences, each a fresh chunk of {S} tokens, 16 heads, "
                                  "kv_lora_rank 512 + rope 64, naive form (K/V expanded once per chunk)",
                      "batch": B, "chunk": S, "num_heads": 16,
                      "cache": "fp8 e4m3, 656 B per token (MLA_BF16_FP8)" if fp8 else "bf16"},
           "flops": {"attention": fa, "expansion": fe}, "kernels_us": kus,
           "roofline": {"bound": "mfma", "achieved": round(fa / (kus["attn"] * 1e-6) / 1e12, 2),
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(fa / (kus["attn"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                        "traffic": prefill_traffic(args),
                        "kernel": "prefill_attn32_kernel (with the q_pe rotation before it)",
                        "expand_tflops": round(fe / (kus["expand"] * 1e-6) / 1e12, 2)}}
    if not args.no_cpu_baseline and not fp8:  # the oracle's sample is of the bf16 rows
        res["cpu_baseline"] = prefill_cpu_baseline(w)
    ctx.free()
    print(json.dumps(res), flush=True)


def ceiling_main(args, w, ctx, pools, q, bt, sl, max_ctx, out):
    """The decode kernel beside two ceilings for its latent-cache stream, each launch on its own events
    over rotated pools (every launch reads bytes the previous one did not): a plain streaming read of the
    same number of bytes, and the decode's HBM -> LDS block gather with no math."""
    import numpy as np
    import torch
    from mla_latent_kv_paged_amd import _lib as L, K_DECODE
    latent = w.latent_bytes()
    sink = torch.empty((1 << 20) // 4, dtype=torch.int32, device="cuda")
    flat = [p.view(-1).view(torch.uint8)[:latent] for p in pools]

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return np.array([a_.elapsed_time(b_) for a_, b_ in ev]) * 1e3

    def read(i):
        L.ceiling_read(flat[i % len(flat)], sink)

    def gather(i):
        ctx.ceiling_gather(pools[i % len(pools)], bt, sl, max_ctx, sink, q_len=w.q_len)

    def decode(i):
        ctx.decode(q, pools[i % len(pools)], bt, sl, max_ctx, q_len=w.q_len, out=out)

    for fn in (read, gather, decode):
        timed(fn, args.warmup)
    res = {"mode": "ceiling", "workload": w.name, "latent_bytes": latent, "launches": args.steps,
           "rotated_pools": len(pools)}
    for name, fn in (("stream_read", read), ("gather_dma", gather), ("decode_events", decode)):
        t = timed(fn, args.steps)
        res[name] = {"us_p10": round(float(np.percentile(t, 10)), 2), "us_median": round(float(np.median(t)), 2),
                     "us_p90": round(float(np.percentile(t, 90)), 2),
                     "tbps_median": round(latent / (float(np.median(t)) * 1e-6) / 1e12, 3)}
    # the decode kernel alone, with the library's events around it (as the benchmark's roofline)
    ctx.profile_enable(True)
    for i in range(args.steps):
        decode(i)
    torch.cuda.synchronize()
    d = np.array(ctx.profile_samples(K_DECODE)) * 1e3
    ctx.profile_enable(False)
    res["decode_kernel"] = {"us_median": round(float(np.median(d)), 2),
                            "tbps_median": round(latent / (float(np.median(d)) * 1e-6) / 1e12, 3)}
    res["decode_kernel_vs_gather"] = round(res["gather_dma"]["us_median"] / res["decode_kernel"]["us_median"], 4)
    res["hbm_peak_tbps"] = HBM_PEAK_GBPS / 1e3
    ctx.free()
    print(json.dumps(res), flush=True)


def layer_main(args):
    """Decode step from hidden states through `--layers` attention layers (mla_layer_decode_step: input
    RMSNorm, q_proj and kv_a_proj, the cache write of the new tokens, the absorbed attention, o_proj and
    the residual), each layer with its own seeded weights and its own cache.  Layer 0's history rows
    come from the workload's generator; the other layers' from a seeded device generator, written
    through mla_cache_write (the values only need to be realistic rows: parity is the tests')."""
    import numpy as np
    import torch
    from mla_latent_kv_paged_amd import (MLAContext, K_LAYER_QKV, K_PREP, K_DECODE, K_COMBINE, K_LAYER_O)
    w = make_workload(args)
    if w.storage != "bf16":
        raise SystemExit("layer mode needs a bf16 workload")
    L = args.layers

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)

    def dev_i(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()

    max_ctx = int(w.seq_lens.max())
    hist_pos, hist_slot = [], []
    for b in range(w.batch):
        hist = int(w.seq_lens[b]) - w.q_len
        hist_pos.append(np.arange(hist))
        hist_slot.append(w.slots(b, 0, hist))
    hpos, hslot = dev_i(np.concatenate(hist_pos)), dev_i(np.concatenate(hist_slot))
    new = w.all_tokens(new_only=True)
    npos, nslot = dev_i(new["positions"]), dev_i(new["slot_mapping"])
    bt, sl = dev_i(w.block_table), dev_i(w.seq_lens)
    t0 = time.perf_counter()
    layers = []
    weight_bytes = 0
    for li in range(L):
        lw = w.layer_weights(li)
        ctx = MLAContext(dev(lw["kv_b_proj"]), None, num_heads=w.num_heads, dtype="bf16", rms_eps=w.eps,
                         rope_theta=w.theta, max_q_tokens=w.n_q, max_batch=w.batch, max_position=max_ctx,
                         max_seq_len=max_ctx)
        ctx.layer_weights(dev(lw["q_proj"]), dev(lw["kv_a_proj"]), dev(lw["o_proj"]), dev(lw["input_norm_gamma"]))
        weight_bytes += 2 * sum(int(np.prod(lw[k].shape)) for k in ("q_proj", "kv_a_proj", "o_proj", "kv_b_proj"))
        pool = torch.full((w.n_blocks, 16, 1, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
        if li == 0:
            hist = w.all_tokens(history_only=True)
            ctx.cache_write(dev(hist["c_kv"]), dev(hist["k_pe"]), hpos, hslot, pool)
        else:
            g = torch.Generator(device="cuda")
            g.manual_seed(1240 + li)
            T = int(hpos.shape[0])
            c = torch.randn((T, 512), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
            k = torch.randn((T, 64), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
            ctx.cache_write(c, k, hpos, hslot, pool)
            del c, k
        layers.append((ctx, pool))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    # one layer: three copies of its pool rotate between steps (no step re-reads the previous one's cache
    # out of the Infinity Cache); several layers: each reads its own cache once per step anyway
    pools1 = [layers[0][1]] + ([layers[0][1].clone() for _ in range(max(0, args.rotate - 1))] if L == 1 else [])
    hidden0 = dev(w.hidden())
    bufs = [torch.empty_like(hidden0), torch.empty_like(hidden0)]

    def step(i):
        h = hidden0
        for li, (ctx, pool) in enumerate(layers):
            p = pools1[i % len(pools1)] if L == 1 else pool
            ctx.layer_decode_step(h, npos, nslot, p, bt, sl, max_ctx, q_len=w.q_len, out=bufs[li % 2])
            h = bufs[li % 2]

    if args.mode == "layer-only":
        for i in range(args.warmup + args.steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "layer-only", "layers": L, "launches": args.warmup + args.steps,
                          "workload": w.name}), flush=True)
        return
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    for ctx, _ in layers:
        ctx.profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kus = {}
    for name, kid in (("qkv_proj", K_LAYER_QKV), ("prep", K_PREP), ("decode", K_DECODE), ("combine", K_COMBINE),
                      ("o_proj", K_LAYER_O)):
        tot = n = 0
        for ctx, _ in layers:
            t_, n_ = ctx.profile_read(kid)
            tot += t_
            n += n_
        kus[name] = round(1e3 * tot / max(n, 1), 2)
    for ctx, _ in layers:
        ctx.profile_enable(False)
    latent = w.latent_bytes() * L
    res = {"metric": f"MLA decode step from hidden states, {L} attention layer(s), µs/step + GB/s (latent cache + "
                     f"weights), V2-Lite {w.name}",
           "value": round(ms * 1e3, 2), "unit": "µs/step", "mode": "layer", "layers": L, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": False,
           "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) hidden states and activations, N(0,1/fan_in) weights)",
           "config": dict(describe(w), hidden_dim=2048, layers=L),
           "kernels_us_per_layer": kus,
           "us_per_layer": round(ms * 1e3 / L, 2),
           "latent_gbps": round(latent / (ms * 1e-3) / 1e9, 1),
           "latent_plus_weights_gbps": round((latent + weight_bytes) / (ms * 1e-3) / 1e9, 1),
           "weight_bytes_per_step": weight_bytes, "latent_bytes_per_step": latent,
           "setup_s": round(setup_s, 1)}
    for ctx, _ in layers:
        ctx.free()
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU sharding is a design "
                                   "note only (the library has no cross-GPU step)",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)
    import numpy as np
    import torch
    if args.mode == "copy-calibration":
        copy_calibration()
        return
    if args.mode == "mfma-calibration":
        mfma_calibration(args)
        return
    if args.mode in ("prefill", "prefill-only"):
        prefill_main(args)
        return
    if args.mode in ("layer", "layer-only"):
        layer_main(args)
        return
    from mla_latent_kv_paged_amd import MLAContext, K_CACHE_WRITE, K_Q_ABSORB, K_DECODE, K_COMBINE, K_PREP

    w = make_workload(args)
    dt = torch.bfloat16 if w.storage == "bf16" else torch.float32
    fp8 = args.cache == "fp8"
    if fp8 and w.storage != "bf16":
        raise SystemExit("--cache fp8 needs a bf16 workload")

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(dt)

    def dev_i(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()

    max_ctx = int(w.seq_lens.max())
    t0 = time.perf_counter()
    kvb = dev(w.kv_b_proj())
    torch.cuda.synchronize()
    ta = time.perf_counter()
    ctx = MLAContext(kvb, None, num_heads=w.num_heads, dtype="fp8" if fp8 else w.storage, rms_eps=w.eps,
                     rope_theta=w.theta,
                     max_q_tokens=w.n_q, max_batch=w.batch, max_position=max_ctx, max_seq_len=max_ctx)
    absorb_ms = (time.perf_counter() - ta) * 1e3
    if args.split_blocks or args.waves:
        ctx.set_decode_tuning(args.split_blocks, args.waves)
    if fp8:
        pool = torch.zeros((w.n_blocks, 16, 1, 656), dtype=torch.uint8, device="cuda")
    else:
        pool = torch.full((w.n_blocks, 16, 1, 576), float("nan"), dtype=dt, device="cuda")
    new_c, new_k, new_pos, new_slot = [], [], [], []
    for b in range(w.batch):       # history fill through the library, one sequence at a time
        c, k = w.history(b)
        ctxb = int(w.seq_lens[b])
        hist = ctxb - w.q_len
        if hist > 0:
            ctx.cache_write(dev(c[:hist]), dev(k[:hist]), dev_i(np.arange(hist)), dev_i(w.slots(b, 0, hist)), pool)
        new_c.append(c[hist:]); new_k.append(k[hist:])
        new_pos.append(np.arange(hist, ctxb)); new_slot.append(w.slots(b, hist, ctxb))
    nc, nk = dev(np.concatenate(new_c)), dev(np.concatenate(new_k))
    npos, nslot = dev_i(np.concatenate(new_pos)), dev_i(np.concatenate(new_slot))
    q = dev(w.queries())
    bt = dev_i(w.block_table)
    sl = dev_i(w.seq_lens)
    pools = [pool] + [pool.clone() for _ in range(max(0, args.rotate - 1))]
    out = torch.empty((w.n_q, w.num_heads, 128), dtype=dt, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0

    def step(i, p=None):
        p = pools[i % len(pools)] if p is None else p
        if args.separate_write:
            ctx.cache_write(nc, nk, npos, nslot, p)
            ctx.decode(q, p, bt, sl, max_ctx, q_len=w.q_len, out=out)
        else:
            ctx.decode_step(nc, nk, npos, nslot, q, p, bt, sl, max_ctx, q_len=w.q_len, out=out)

    if args.mode == "ceiling":
        ceiling_main(args, w, ctx, pools, q, bt, sl, max_ctx, out)
        return

    if args.mode == "decode-only":
        for i in range(args.warmup + args.steps):
            ctx.decode(q, pools[i % len(pools)], bt, sl, max_ctx, q_len=w.q_len, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "decode-only", "launches": args.warmup + args.steps, "workload": w.name}),
              flush=True)
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # pass A: the step as a whole (no per-kernel events)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    # pass B: per-kernel HIP events recorded by the library on the launch stream
    ctx.profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern = {}
    # the step's first launch: cache write + query absorption (mla_decode_step), or the two apart
    first = (("prep", K_PREP),) if not args.separate_write else (("cache_write", K_CACHE_WRITE),
                                                                   ("q_absorb", K_Q_ABSORB))
    for name, kid in first + (("decode", K_DECODE), ("combine", K_COMBINE)):
        tot, n = ctx.profile_read(kid)
        kern[name] = {"avg_us": 1e3 * tot / max(n, 1), "launches": n}
    dec_samples = np.array(ctx.profile_samples(K_DECODE)) * 1e3
    ctx.profile_enable(False)
    shape = ctx.last_decode_shape()
    # pass C: each step bracketed by its own events (distribution of the step time)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    step_samples = np.array([a_.elapsed_time(b_) for a_, b_ in ev]) * 1e3
    # pass D (--unflushed only): every step on the same pool, so the previous step's cache may still sit
    # in the 256 MB Infinity Cache.  Off by default, so that every decode launch of a default run (and of
    # its profiler trace) reads a pool the previous steps did not
    unflushed_us = None
    if args.unflushed:
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            step(i, pools[0])
        e1.record()
        torch.cuda.synchronize()
        unflushed_us = e0.elapsed_time(e1) / args.steps * 1e3

    def pct(x):
        return {"p10": round(float(np.percentile(x, 10)), 2), "median": round(float(np.median(x)), 2),
                "p90": round(float(np.percentile(x, 90)), 2)}

    latent_bytes = w.total_ctx * 656 if fp8 else w.latent_bytes()
    decode_us = kern["decode"]["avg_us"]
    flops_attn = w.total_ctx * w.num_heads * w.q_len * 2 * (576 + 512)
    flops_gemm = 2 * w.n_q * w.num_heads * 131072  # q_nope . W_uk and o_lat . W_uv^T
    # (with mla_decode_step the first launch also writes the new tokens' rows)
    mla_decode_us = kern["prep" if "prep" in kern else "q_absorb"]["avg_us"] + decode_us + kern["combine"]["avg_us"]
    achieved = latent_bytes / (decode_us * 1e-6) / 1e9
    traffic = traffic_entry(args)
    rows32 = (w.num_heads * w.q_len) % 32 == 0
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "decode_fp8_kernel" if fp8 else
                ("decode_bf16_mt32_kernel" if rows32 else "decode_bf16_kernel") if w.storage == "bf16"
                else "decode_f32_kernel",
                "algorithmic_bytes_per_launch": latent_bytes,
                "mfma_tflops": round(flops_attn / (decode_us * 1e-6) / 1e12, 2),
                "mfma_frac": round(flops_attn / (decode_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "mfma_frac_mla_decode": round((flops_attn + flops_gemm) / (mla_decode_us * 1e-6) / 1e12
                                              / BF16_PEAK_TFLOPS, 4)}
    step_us = ms_per_step * 1e3
    res = {
        "metric": METRIC,
        "value": round(latent_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(step_us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.storage == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/512) kv_b_proj)",
        "config": dict(describe(w), cache="fp8 e4m3, 656 B per token (MLA_BF16_FP8)" if fp8 else "native"),
        "decode_us": round(decode_us, 2),
        "decode_us_dist": pct(dec_samples),
        "step_us_dist": pct(step_samples),
        "unflushed_us_per_step": None if unflushed_us is None else round(unflushed_us, 2),
        "decode_latent_gbps": round(achieved, 1),
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
        "step_calls": "mla_cache_write + mla_decode" if args.separate_write else "mla_decode_step",
        "split": shape,
        "absorb_weights_ms_once": round(absorb_ms, 2),
        "rotated_pools": len(pools),
        "setup_s": round(setup_s, 1),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample if not fp8 else min(args.cpu_sample, 8), fp8)
    ctx.free()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
