"""Seeded synthetic inputs for MLA decode over a paged latent cache.

This module only draws random numbers, rounds them to the storage dtype and lays out
the paging structure (seq_lens, block_table, slot_mapping).  It holds none of the
method's arithmetic (no RMSNorm, no RoPE, no attention), so that both the fp64 oracle
and the HIP library can consume the same values without sharing any compute code.

Workloads (shapes follow DeepSeek-V2-Lite as given on the mini-infer 17 page, "MLA 的数学结构":
kv_lora_rank 512, qk_rope_head_dim 64; per-head nope 128 and v 128; 16 heads):

  tiny      fp32, B=1, 64 cached + 1 new token (ctx 65), pool of 5 blocks, identity table.
  lite_b1   bf16, B=1, seq_len S in {1, 256, 1024} (ctx S+1), pool of 256 blocks,
            block table = first ceil(ctx/16) entries of a random permutation.
  lite_b64  bf16, B=64, S=4096 (ctx 4097), pool of 20,000 blocks, block table drawn
            from one random permutation of the pool.  Headline bandwidth workload.
  wide      bf16, 128 heads, B=128, S ~ U{1024..8192}, ctx S+1, pool = ceil(1.25 * blocks needed).
  ragged    bf16, B=256, S = clip(round(exp(N(ln 2048, 1))), 16, 32768), q_len 4, ctx S+4.

Values: activations (raw latent c_kv, raw k_pe, queries) ~ N(0, 1); kv_b_proj ~ N(0, 1/512);
gamma = 1 unless asked otherwise; eps 1e-6; theta 10000; scale 1/sqrt(192).
The hidden state -> projection step sits outside the library boundary: h ~ N(0,1) through a
weight ~ N(0, 1/fan_in) gives N(0,1) activations, so activations are drawn directly.
Every tensor is rounded to the storage dtype once, here (bf16: round-to-nearest-even).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64
QK_NOPE_HEAD_DIM = 128
V_HEAD_DIM = 128
BLOCK_SIZE = 16
ROW = KV_LORA_RANK + QK_ROPE_HEAD_DIM

# tags for independent seed streams
_T_WEIGHT, _T_GAMMA, _T_Q, _T_STRUCT, _T_HIST, _T_POOL, _T_QCHUNK, _T_LAYER, _T_HIDDEN = range(9)
HIDDEN_DIM = 2048  # DeepSeek-V2-Lite hidden size


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even. No NaN handling needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed, tag, *sub):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(tag,) + sub)))


@dataclasses.dataclass
class Workload:
    name: str
    storage: str                 # "f32" or "bf16"
    num_heads: int
    batch: int
    q_len: int
    seq_lens: np.ndarray         # int32 [B], context length incl. the q_len new tokens
    n_blocks: int                # pool size
    block_table: np.ndarray      # int32 [B, max_blocks]
    seed: int
    gamma_noise: float = 0.0     # 0 -> gamma = 1
    eps: float = 1e-6
    theta: float = 10000.0
    kv_lora_rank: int = KV_LORA_RANK
    qk_rope_head_dim: int = QK_ROPE_HEAD_DIM
    qk_nope_head_dim: int = QK_NOPE_HEAD_DIM
    v_head_dim: int = V_HEAD_DIM
    block_size: int = BLOCK_SIZE
    hidden_dim: int = HIDDEN_DIM

    # ---------------------------------------------------------------- derived sizes
    @property
    def scale(self):
        return 1.0 / math.sqrt(self.qk_nope_head_dim + self.qk_rope_head_dim)

    @property
    def n_q(self):
        return self.batch * self.q_len

    @property
    def total_ctx(self):
        return int(np.sum(self.seq_lens.astype(np.int64)))

    @property
    def elem_bytes(self):
        return 2 if self.storage == "bf16" else 4

    def latent_bytes(self):
        """Algorithmic latent-cache bytes one decode reads: every context row once."""
        return self.total_ctx * ROW * self.elem_bytes

    # ---------------------------------------------------------------- value storage
    def _store(self, x):
        """float32 draws -> storage dtype. Returns (values as float32, bits or None)."""
        if self.storage == "bf16":
            bits = f32_to_bf16_bits(x)
            return bf16_bits_to_f32(bits), bits
        return np.asarray(x, dtype=np.float32), None

    def kv_b_proj(self):
        """[H*(dn+dv), dc] float32 values (bf16-representable in bf16 mode)."""
        H = self.num_heads
        rows = H * (self.qk_nope_head_dim + self.v_head_dim)
        w = _rng(self.seed, _T_WEIGHT).standard_normal((rows, self.kv_lora_rank), dtype=np.float32)
        w *= np.float32(1.0 / math.sqrt(self.kv_lora_rank))
        return self._store(w)[0]

    def gamma(self):
        g = np.ones(self.kv_lora_rank, dtype=np.float32)
        if self.gamma_noise:
            g += np.float32(self.gamma_noise) * _rng(self.seed, _T_GAMMA).standard_normal(
                self.kv_lora_rank, dtype=np.float32)
        return self._store(g)[0]

    def queries(self):
        """[B*q_len, H, dn+dr] un-rotated queries ([nope | rope] per head)."""
        q = _rng(self.seed, _T_Q).standard_normal(
            (self.n_q, self.num_heads, self.qk_nope_head_dim + self.qk_rope_head_dim), dtype=np.float32)
        return self._store(q)[0]

    def chunk_queries(self, chunks):
        """[sum(chunks), H, dn+dr] un-rotated queries for a chunked prefill in which sequence b has
        chunks[b] new tokens (rows in sequence order), drawn from a stream of their own."""
        q = _rng(self.seed, _T_QCHUNK).standard_normal(
            (int(np.sum(chunks)), self.num_heads, self.qk_nope_head_dim + self.qk_rope_head_dim), dtype=np.float32)
        return self._store(q)[0]

    def hidden(self, layer=0):
        """[B*q_len, D] hidden states of the new tokens entering layer `layer` ~ N(0, 1)."""
        h = _rng(self.seed, _T_HIDDEN, layer).standard_normal((self.n_q, self.hidden_dim), dtype=np.float32)
        return self._store(h)[0]

    def layer_weights(self, layer=0, input_gamma_noise=0.0):
        """Projection weights of one attention layer, each ~ N(0, 1/fan_in) (float32 storage values):
        q_proj [H*(dn+dr), D], kv_a_proj [dc+dr, D], o_proj [D, H*dv]; input_norm_gamma [D] (1, or
        1 + noise * N(0,1)); kv_b_proj [H*(dn+dv), dc] (layer 0: the workload's kv_b_proj) and the
        kv_a_layernorm gamma [dc] (layer 0: the workload's gamma)."""
        H, D = self.num_heads, self.hidden_dim
        dq = self.qk_nope_head_dim + self.qk_rope_head_dim
        dkv = self.kv_lora_rank + self.qk_rope_head_dim

        def draw(k, shape, fan_in):
            w = _rng(self.seed, _T_LAYER, layer, k).standard_normal(shape, dtype=np.float32)
            return self._store(w * np.float32(1.0 / math.sqrt(fan_in)))[0]

        g = np.ones(D, dtype=np.float32)
        if input_gamma_noise:
            g += np.float32(input_gamma_noise) * _rng(self.seed, _T_LAYER, layer, 3).standard_normal(
                D, dtype=np.float32)
        if layer == 0:
            kvb, kvg = self.kv_b_proj(), self.gamma()
        else:
            kvb = draw(4, (H * (self.qk_nope_head_dim + self.v_head_dim), self.kv_lora_rank), self.kv_lora_rank)
            kvg = np.ones(self.kv_lora_rank, dtype=np.float32)
            if self.gamma_noise:
                kvg += np.float32(self.gamma_noise) * _rng(self.seed, _T_LAYER, layer, 5).standard_normal(
                    self.kv_lora_rank, dtype=np.float32)
            kvg = self._store(kvg)[0]
        return dict(q_proj=draw(0, (H * dq, D), D), kv_a_proj=draw(1, (dkv, D), D),
                    o_proj=draw(2, (D, H * self.v_head_dim), H * self.v_head_dim),
                    input_norm_gamma=self._store(g)[0], kv_b_proj=kvb, kv_norm_gamma=kvg)

    def history(self, b, layer=0):
        """Raw (un-normed c_kv, un-rotated k_pe) for every context token of sequence b,
        positions 0..ctx_b-1: ([ctx, dc], [ctx, dr]) float32 storage values (one stream per layer)."""
        ctx = int(self.seq_lens[b])
        g = _rng(self.seed, _T_HIST, b) if layer == 0 else _rng(self.seed, _T_HIST, b, layer)
        c = g.standard_normal((ctx, self.kv_lora_rank), dtype=np.float32)
        k = g.standard_normal((ctx, self.qk_rope_head_dim), dtype=np.float32)
        return self._store(c)[0], self._store(k)[0]

    def slots(self, b, t0, t1):
        """slot_mapping for tokens t0..t1-1 of sequence b: physical block * 16 + offset."""
        t = np.arange(t0, t1, dtype=np.int64)
        return (self.block_table[b, t // self.block_size].astype(np.int64) * self.block_size
                + t % self.block_size).astype(np.int32)

    def all_tokens(self, new_only=False, history_only=False):
        """Concatenate tokens of all sequences in order (b, t).

        Returns dict with c_kv [T, dc], k_pe [T, dr] (float32 values), positions [T] int32,
        slot_mapping [T] int32.  new_only -> the q_len new tokens per sequence;
        history_only -> the tokens before them.
        """
        cs, ks, ps, ss = [], [], [], []
        for b in range(self.batch):
            ctx = int(self.seq_lens[b])
            t0 = ctx - self.q_len if new_only else 0
            t1 = ctx - self.q_len if history_only else ctx
            c, k = self.history(b)
            cs.append(c[t0:t1])
            ks.append(k[t0:t1])
            ps.append(np.arange(t0, t1, dtype=np.int32))
            ss.append(self.slots(b, t0, t1))
        return dict(c_kv=np.concatenate(cs), k_pe=np.concatenate(ks),
                    positions=np.concatenate(ps), slot_mapping=np.concatenate(ss))

    def random_pool(self):
        """A cache pool whose live rows are random N(0,1) storage values and whose other
        slots are NaN: input for decode-only checks.  [n_blocks, 16, 1, 576] float32."""
        pool = np.full((self.n_blocks, self.block_size, 1, ROW), np.nan, dtype=np.float32)
        for b in range(self.batch):
            ctx = int(self.seq_lens[b])
            rows = _rng(self.seed, _T_POOL, b).standard_normal((ctx, ROW), dtype=np.float32)
            rows = self._store(rows)[0]
            t = np.arange(ctx)
            pool[self.block_table[b, t // self.block_size], t % self.block_size, 0, :] = rows
        return pool


# ------------------------------------------------------------------------------------ builders

def _blocks_needed(seq_lens):
    return [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in seq_lens]


def _table_from_pool(rng, seq_lens, n_blocks):
    need = _blocks_needed(seq_lens)
    perm = rng.permutation(n_blocks).astype(np.int32)
    width = max(need)
    table = np.zeros((len(seq_lens), width), dtype=np.int32)
    pos = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    return table


def custom(name, storage, num_heads, seq_lens, q_len=1, pool_factor=1.25, seed=1234,
           identity_table=False, gamma_noise=0.0):
    """Arbitrary workload: context lengths seq_lens (incl. q_len new tokens each)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if np.any(seq_lens < q_len):
        raise ValueError("every context must hold its q_len new tokens")
    need = sum(_blocks_needed(seq_lens))
    if identity_table:
        n_blocks = need
        table = np.zeros((len(seq_lens), max(_blocks_needed(seq_lens))), dtype=np.int32)
        pos = 0
        for b, nb in enumerate(_blocks_needed(seq_lens)):
            table[b, :nb] = np.arange(pos, pos + nb, dtype=np.int32)
            pos += nb
    else:
        n_blocks = int(math.ceil(pool_factor * need))
        table = _table_from_pool(_rng(seed, _T_STRUCT), seq_lens, n_blocks)
    return Workload(name=name, storage=storage, num_heads=num_heads, batch=len(seq_lens), q_len=q_len,
                    seq_lens=seq_lens, n_blocks=n_blocks, block_table=table, seed=seed,
                    gamma_noise=gamma_noise)


def tiny():
    """fp32, B=1, 64 cached + 1 new token, identity block table over 5 blocks."""
    return custom("tiny", "f32", 16, [65], q_len=1, seed=1234, identity_table=True)


def lite_b1(seq_len):
    """bf16, B=1, seq_len cached + 1 new, pool 256 blocks, randomly permuted table."""
    seed = 1235
    ctx = seq_len + 1
    rng = _rng(seed, _T_STRUCT)
    perm = rng.permutation(256).astype(np.int32)
    nb = (ctx + BLOCK_SIZE - 1) // BLOCK_SIZE
    table = perm[:nb].reshape(1, nb)
    return Workload(name=f"lite_b1_s{seq_len}", storage="bf16", num_heads=16, batch=1, q_len=1,
                    seq_lens=np.array([ctx], dtype=np.int32), n_blocks=256, block_table=table, seed=seed)


def lite_b64(batch=64, seq_len=4096, n_blocks=20000, seed=1236):
    """bf16, every sequence seq_len cached + 1 new token, blocks shuffled over a 20,000-block pool."""
    ctx = seq_len + 1
    nb = (ctx + BLOCK_SIZE - 1) // BLOCK_SIZE
    if batch * nb > n_blocks:
        raise ValueError("pool too small")
    perm = _rng(seed, _T_STRUCT).permutation(n_blocks).astype(np.int32)
    table = perm[:batch * nb].reshape(batch, nb)
    return Workload(name=f"lite_b{batch}_s{seq_len}", storage="bf16", num_heads=16, batch=batch, q_len=1,
                    seq_lens=np.full(batch, ctx, dtype=np.int32), n_blocks=n_blocks, block_table=table,
                    seed=seed)


def wide(batch=128, lo=1024, hi=8192, seed=1237):
    """bf16, 128 heads, seq_len ~ U{lo..hi} cached + 1 new token."""
    s = _rng(seed, _T_STRUCT, 1).integers(lo, hi + 1, size=batch)
    return custom(f"wide_h128_b{batch}", "bf16", 128, s + 1, q_len=1, seed=seed)


def ragged(batch=256, median=2048, sigma=1.0, lo=16, hi=32768, q_len=4, seed=1238):
    """bf16, lognormal seq_len (median 2048, sigma 1, clipped), 4 causal new tokens each."""
    z = _rng(seed, _T_STRUCT, 1).standard_normal(batch)
    s = np.clip(np.round(np.exp(np.log(median) + sigma * z)), lo, hi).astype(np.int64)
    return custom(f"ragged_b{batch}_q{q_len}", "bf16", 16, s + q_len, q_len=q_len, seed=seed)


def by_config(cfg_id, **kw):
    """The five contract workloads: 0 tiny, 1 lite_b1 (seq_len kw, default 1024), 2 lite_b64,
    3 wide, 4 ragged."""
    if cfg_id == 0:
        return tiny()
    if cfg_id == 1:
        return lite_b1(kw.get("seq_len", 1024))
    if cfg_id == 2:
        return lite_b64()
    if cfg_id == 3:
        return wide()
    if cfg_id == 4:
        return ragged()
    raise ValueError(cfg_id)
