"""FP8 (e4m3) latent cache for the MLA decode oracle.

TEST INFRASTRUCTURE ONLY, like mla_oracle.py: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; it depends on NumPy and mla_oracle.

What it follows.  The learning-book page on MLA in vLLM ([P-vllm] ch. 07 "模型架构特异：MLA / Mamba /
MoE 在 vLLM 源码层") lists an FP8 KV cache for MLA among the engine's options, and the same page
(§2.3) fixes the cache shape (n_blocks, block, 1, latent_d + rope_d); the pages give no scale
convention and no byte layout.  The reading taken here:

* Number format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  no infinities; S.1111.111 is NaN; the largest finite value is 1.75 * 2^8 = 448; exponent field 0
  holds the subnormals m * 2^-9.  Encoding rounds to the nearest value, ties to the even code.
* What is quantised: the RMS-normed latent c (512 channels) of each token, in 4 groups of 128
  channels.  Group g has scale s_g = the fp32 value nearest amax_g / 448 (stepped up to the next
  fp32 value if amax_g / s_g would exceed 448; s_g = 1 for an all-zero group), and codes
  e4m3(c / s_g), with the quotient c / s_g evaluated in fp64 (one IEEE rounding) before the
  e4m3 rounding.  The RoPE'd k_pe stays bf16 (round to nearest even), as in the bf16 cache.
* Row layout, 656 bytes per token: bytes 0..511 the latent codes (channel order), bytes 512..639
  the 64 bf16 rope values (little-endian), bytes 640..655 the 4 fp32 group scales.
* The value the decode sees for channel i of group g is decode(code_i) * s_g, exactly (a 4-bit
  significand times a 24-bit one fits fp64).

Pins: the test suite checks the value table against the format definition's landmarks, against
torch's float8_e4m3fn conversion, and the quantiser against its error bound.
"""

from __future__ import annotations

import numpy as np

from . import mla_oracle as O

ROW_BYTES = 656
DC, DR = 512, 64
GROUP = 128
E4M3_MAX = 448.0


def e4m3_values():
    """Value of each of the 256 codes (float64; NaN for the two NaN codes), from the format fields."""
    v = np.empty(256, dtype=np.float64)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            v[code] = np.nan
        elif e == 0:
            v[code] = m * 2.0 ** -9
        else:
            v[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        if s:
            v[code] = -v[code]
    return v


_VALUES = e4m3_values()
# the non-negative finite codes in increasing value order: codes 0x00..0x7E are already increasing
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _VALUES[:0x7F]


def e4m3_encode(x):
    """Round float64 values (|x| <= 448) to the nearest e4m3 code, ties to the even code.

    A table search: for |x| find the two neighbouring representable magnitudes and keep the
    nearer; on a tie keep the one with the even code (its last mantissa bit 0)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: values must be finite with |x| <= 448")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # first magnitude >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    exact = _POS_VALUES[hi] == a
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    neg = np.signbit(x) & (code != 0)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(codes):
    return _VALUES[np.asarray(codes, dtype=np.int64)]


def group_scale(amax):
    """fp32 scale of a group with largest magnitude amax (see the module docstring); amax may be an
    array of group maxima, one scale each."""
    amax = np.asarray(amax, dtype=np.float64)
    s = (amax / E4M3_MAX).astype(np.float32)
    up = amax > E4M3_MAX * s.astype(np.float64)          # 448 * s is exact in fp64
    s = np.where(up, np.nextafter(s, np.float32(np.inf)), s).astype(np.float64)
    s = np.where(amax == 0.0, 1.0, s)
    return float(s) if s.ndim == 0 else s


def quantize_latent(c):
    """c [..., 512] float64 -> (codes uint8 [..., 512], scales float64 [..., 4] (fp32 values)).
    Each row is quantised on its own: rows are independent."""
    c = np.asarray(c, dtype=np.float64)
    groups = c.reshape(c.shape[:-1] + (DC // GROUP, GROUP))
    scales = group_scale(np.max(np.abs(groups), axis=-1))
    codes = e4m3_encode(groups / np.asarray(scales)[..., None])
    return codes.reshape(c.shape), scales


def pack_row(codes, rope_bf16, scales):
    """656-byte cache row(s) [..., 656] from the latent codes [..., 512], the bf16 rope values [..., 64]
    and the scales [..., 4]."""
    codes = np.asarray(codes, dtype=np.uint8)
    row = np.zeros(codes.shape[:-1] + (ROW_BYTES,), dtype=np.uint8)
    row[..., :DC] = codes
    bits = np.ascontiguousarray(np.asarray(rope_bf16, dtype=np.float64).astype(np.float32)).view(np.uint32) >> 16
    row[..., DC:DC + 2 * DR] = np.ascontiguousarray(bits.astype("<u2")).view(np.uint8)
    row[..., DC + 2 * DR:] = np.ascontiguousarray(np.asarray(scales, dtype=np.float64).astype("<f4")).view(np.uint8)
    return row


def unpack_row(row):
    """656-byte row(s) [..., 656] -> (latent values [..., 512] float64, rope values [..., 64] float64)."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    scales = row[..., DC + 2 * DR:].copy().view("<f4").astype(np.float64)          # [..., 4]
    lat = e4m3_decode(row[..., :DC]) * np.repeat(scales, GROUP, axis=-1)
    rope = (row[..., DC:DC + 2 * DR].copy().view("<u2").astype(np.uint32) << 16).view(np.float32)
    return lat, rope.astype(np.float64)


def cache_write_fp8(cache, c_kv, k_pe, positions, slot_mapping, gamma, eps, theta):
    """Write new tokens into a copy of the byte cache [n_blocks, block, 1, 656] and return it.

    Per token: c = RMSNorm(c_kv) * gamma and k = RoPE(k_pe, pos) in fp64 (mla_oracle.rms_norm,
    mla_oracle.rope), then c is quantised by groups and k rounded to bf16.  Negative slots are
    skipped; untouched slots keep their bytes; a slot written twice keeps the later token.  Tokens
    are independent, so their rows are computed many at a time."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    n_blocks, block_size, _, width = out.shape
    if width != ROW_BYTES:
        raise ValueError("fp8 cache rows are 656 bytes")
    c_kv = np.asarray(c_kv, dtype=np.float64).reshape(-1, DC)
    k_pe = np.asarray(k_pe, dtype=np.float64).reshape(-1, DR)
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    keep = slots >= 0
    if np.any(slots[keep] // block_size >= n_blocks):
        raise IndexError("slot outside the cache pool")
    if not np.any(keep):
        return out
    idx = np.nonzero(keep)[0]
    # a slot written twice keeps the later token: store only each slot's last writer
    _, last = np.unique(slots[idx][::-1], return_index=True)
    idx = idx[len(idx) - 1 - last]
    pos = np.asarray(positions).reshape(-1)
    flat = out.reshape(-1, ROW_BYTES)
    for lo in range(0, len(idx), 8192):  # rows in batches, to bound the temporaries
        j = idx[lo:lo + 8192]
        codes, scales = quantize_latent(O.rms_norm(c_kv[j], gamma, eps))
        k = O.round_to_bf16(O.rope(k_pe[j], pos[j], theta))
        flat[slots[j]] = pack_row(codes, k, scales)
    return out


def dequantize_cache(cache):
    """Byte cache [n_blocks, block, 1, 656] -> float64 cache [n_blocks, block, 1, 576] of the values
    the decode sees (rows that were never written come out as whatever their bytes say)."""
    lat, rope = unpack_row(np.asarray(cache, dtype=np.uint8))
    return np.concatenate([lat, rope], axis=-1)
