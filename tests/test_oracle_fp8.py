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
