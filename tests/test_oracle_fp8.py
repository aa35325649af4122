"""CPU pins of the FP8 (e4m3) cache oracle (oracle/mla_fp8.py).

The value table is checked against the landmarks of the OCP E4M3 definition and against torch's
independent float8_e4m3fn type (decoding all 256 codes, encoding random and tie values); the
quantiser against its error bound and scale rule; the row layout by round trip and against the
bf16 oracle cache (same RMSNorm and RoPE, only the storage differs)."""

import numpy as np
import pytest

from oracle import mla_fp8 as F
from oracle import mla_oracle as O

torch = pytest.importorskip("torch")


def test_e4m3_landmarks():
    v = F.e4m3_values()
    assert v[0x7E] == 448.0                      # largest finite: 1.75 * 2^8
    assert v[0x01] == 2.0 ** -9                  # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert v[0x08] == 2.0 ** -6                  # smallest normal (exponent field 1, bias 7)
    assert v[0x38] == 1.0
    assert v[0x3F] == 1.875
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.sum(np.isfinite(v)) == 254
    assert np.all(np.diff(v[:0x7F]) > 0)         # codes 0..0x7E increase with value
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])


def test_e4m3_table_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = F.e4m3_values()
    assert np.array_equal(np.isnan(t), np.isnan(v))
    ok = ~np.isnan(v)
    assert np.array_equal(t[ok], v[ok])


def test_e4m3_encode_ties_and_exact():
    enc = F.e4m3_encode
    assert enc(np.array([1.0625]))[0] == 0x38    # tie between 1.0 (0x38) and 1.125 (0x39): even
    assert enc(np.array([1.1875]))[0] == 0x3A    # tie between 1.125 and 1.25 (0x3A): even
    assert enc(np.array([2.0 ** -10]))[0] == 0x00
    assert enc(np.array([3 * 2.0 ** -10]))[0] == 0x02
    assert enc(np.array([-0.5]))[0] == 0xB0
    assert enc(np.array([448.0]))[0] == 0x7E
    assert enc(np.array([432.0]))[0] == 0x7E     # tie between 416 (0x7D) and 448 (0x7E): even
    assert enc(np.array([424.0]))[0] == 0x7D     # nearer 416
    v = F.e4m3_values()
    ok = np.where(~np.isnan(v))[0]
    ok = ok[ok != 0x80]                          # -0 encodes as +0
    assert np.array_equal(enc(v[ok]), ok.astype(np.uint8))
    with pytest.raises(ValueError):
        enc(np.array([449.0]))


def test_e4m3_encode_matches_torch_random():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-9, 6, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    # every midpoint between neighbouring values, in both signs
    v = F.e4m3_values()[:0x7F]
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    ref = np.where(ref == 0x80, 0, ref)          # torch keeps -0; the oracle encodes zero as +0
    assert np.array_equal(got, ref)


def test_quantize_scale_rule_and_error_bound():
    rng = np.random.default_rng(5)
    for trial in range(50):
        c = rng.standard_normal(512) * np.exp(rng.uniform(-20, 20, 4)).repeat(128)
        codes, scales = F.quantize_latent(c)
        assert codes.dtype == np.uint8 and scales.shape == (4,)
        deq = F.e4m3_decode(codes) * np.repeat(scales, 128)
        for g in range(4):
            part = c[g * 128:(g + 1) * 128]
            s, amax = scales[g], np.max(np.abs(part))
            assert s == float(np.float32(s))                 # an fp32 value
            assert amax <= 448 * s                           # never saturates
            assert amax > 448 * float(np.nextafter(np.float32(s), np.float32(0)))  # the smallest such
            k = int(np.argmax(np.abs(part)))
            assert abs(F.e4m3_decode(codes[g * 128 + k])) == 448.0  # the group max maps to 448
            err = np.abs(deq[g * 128:(g + 1) * 128] - part)
            # half a spacing: 2^-4 relative for normals, 2^-10 * s below the smallest normal
            bound = np.maximum(np.abs(part) * 2.0 ** -4, s * 2.0 ** -10)
            assert np.all(err <= bound * (1 + 1e-12))
    codes, scales = F.quantize_latent(np.zeros(512))
    assert np.all(codes == 0) and np.all(scales == 1.0)


def test_row_round_trip_and_bf16_consistency():
    rng = np.random.default_rng(7)
    T, theta, eps = 5, 10000.0, 1e-6
    c_kv = rng.standard_normal((T, 512))
    k_pe = rng.standard_normal((T, 64))
    pos = np.array([0, 3, 17, 250, 1024])
    slots = np.array([0, 5, 16, 31, -1])
    gamma = 1 + 0.1 * rng.standard_normal(512)
    pool8 = np.zeros((2, 16, 1, F.ROW_BYTES), dtype=np.uint8)
    out8 = F.cache_write_fp8(pool8, c_kv, k_pe, pos, slots, gamma, eps, theta)
    out16 = O.cache_write(np.full((2, 16, 1, 576), np.nan), c_kv, k_pe, pos, slots, gamma, eps, theta, "bf16")
    deq = F.dequantize_cache(out8)
    for j in range(T):
        if slots[j] < 0:
            continue
        b, o = divmod(int(slots[j]), 16)
        c = O.rms_norm(c_kv[j], gamma, eps)
        # rope part: the same bf16 values as the bf16 cache
        assert np.array_equal(deq[b, o, 0, 512:], out16[b, o, 0, 512:])
        # latent: within the quantiser's bound of the exact normed latent
        codes, scales = F.quantize_latent(c)
        assert np.array_equal(out8[b, o, 0, :512], codes)
        assert np.array_equal(deq[b, o, 0, :512], F.e4m3_decode(codes) * np.repeat(scales, 128))
        lat, rope = F.unpack_row(F.pack_row(codes, out16[b, o, 0, 512:], scales))
        assert np.array_equal(lat, deq[b, o, 0, :512]) and np.array_equal(rope, out16[b, o, 0, 512:])
    untouched = np.ones((2, 16), dtype=bool)
    for s in slots[slots >= 0]:
        untouched[s // 16, s % 16] = False
    assert np.all(out8[untouched] == 0)


def _hand_row():
    """A 656-byte row written byte by byte from the format fields and the row layout (latent codes at
    bytes 0..511, bf16 rope values little-endian at 512..639, fp32 group scales little-endian at
    640..655), with the values each byte stands for."""
    row = np.zeros(656, dtype=np.uint8)
    lat = np.zeros(512)
    # E4M3 codes: sign | exponent (bias 7) | mantissa
    row[0], lat[0] = 0x38, 1.0               # 0 0111 000: 2^0
    row[1], lat[1] = 0x7E, 448.0             # 0 1111 110: 1.75 * 2^8, the largest finite
    row[2], lat[2] = 0xC0, -2.0              # 1 1000 000
    row[127], lat[127] = 0x01, 2.0 ** -9     # 0 0000 001: the smallest subnormal
    row[128], lat[128] = 0x38, 1.0 * 0.5     # group 1, scale 0.5
    row[256], lat[256] = 0x7E, 448.0 * 2.0 ** -10   # group 2, scale 2^-10
    row[511], lat[511] = 0xB0, -0.5 * 3.0    # 1 0110 000 = -0.5; group 3, scale 3
    rope = np.zeros(64)
    row[512], row[513], rope[0] = 0x80, 0x3F, 1.0    # bf16 0x3F80
    row[514], row[515], rope[1] = 0x00, 0xC0, -2.0   # bf16 0xC000
    row[516], row[517], rope[2] = 0x00, 0x3F, 0.5    # bf16 0x3F00
    scales = np.array([1.0, 0.5, 2.0 ** -10, 3.0])
    row[640:644] = (0x00, 0x00, 0x80, 0x3F)   # fp32 0x3F800000
    row[644:648] = (0x00, 0x00, 0x00, 0x3F)   # fp32 0x3F000000
    row[648:652] = (0x00, 0x00, 0x80, 0x3A)   # fp32 0x3A800000
    row[652:656] = (0x00, 0x00, 0x40, 0x40)   # fp32 0x40400000
    return row, lat, rope, scales


def test_row_layout_against_hand_built_bytes():
    """pack_row and unpack_row against a row whose bytes are written out by hand (not by either
    function): a layout slip made in both (offsets, byte order, scale groups) fails here."""
    row, lat, rope, scales = _hand_row()
    codes = row[:512].copy()
    assert np.array_equal(F.pack_row(codes, rope, scales), row)
    got_lat, got_rope = F.unpack_row(row)
    assert np.array_equal(got_lat, lat)
    assert np.array_equal(got_rope, rope)
    # a cache of two such rows decodes to the same values in each slot
    cache = np.zeros((1, 16, 1, 656), dtype=np.uint8)
    cache[0, 3, 0] = row
    deq = F.dequantize_cache(cache)
    assert np.array_equal(deq[0, 3, 0, :512], lat) and np.array_equal(deq[0, 3, 0, 512:], rope)
    assert np.all(deq[0, 0, 0] == 0)


def test_quantiser_codes_by_hand():
    """quantize_latent on values whose codes and scales are worked out by hand from the format:
    exact values, ties to the even code (normal and subnormal), a zero group, and group scales of
    1, 1/2 and 3 (amax / 448 exact in fp32)."""
    c = np.zeros(512)
    expect = np.zeros(512, dtype=np.uint8)
    vals = [(448.0, 0x7E), (1.0625, 0x38), (1.1875, 0x3A), (2.5 * 2.0 ** -9, 0x02), (-0.5, 0xB0), (240.0, 0x77),
            (7 * 2.0 ** -9, 0x07), (2.0 ** -6, 0x08)]
    for i, (v, code) in enumerate(vals):          # group 0: amax 448 -> scale 1
        c[i], expect[i] = v, code
    c[128], expect[128] = 224.0, 0x7E              # group 1: amax 224 -> scale 0.5
    c[129], expect[129] = 0.5, 0x38
    c[130], expect[130] = -1.0, 0xC0
    # group 2 stays zero: scale 1, codes 0
    c[384], expect[384] = 1344.0, 0x7E             # group 3: amax 1344 -> scale 3
    c[385], expect[385] = -6.0, 0xC0
    codes, scales = F.quantize_latent(c)
    assert np.array_equal(codes, expect)
    assert np.array_equal(scales, [1.0, 0.5, 1.0, 3.0])
