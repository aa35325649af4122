"""CPU-side checks of the C-ABI library: it loads, exports every function include/mla.h
declares, and rejects invalid host arguments before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from mla_latent_kv_paged_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libmla.so not built")
    return L, L.load()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    fns = _header_functions()
    for f in ("mla_absorb_weights", "mla_cache_write", "mla_decode", "mla_free"):
        assert f in fns


def test_library_exports_every_declared_function():
    L, lib = _lib()
    for f in _header_functions():
        assert hasattr(lib, f), f
    assert set(_header_functions()) == set(L.EXPORTS)


def test_status_strings():
    L, lib = _lib()
    for code, word in ((0, "MLA_OK"), (-1, "EINVAL"), (-2, "EUNSUPPORTED"), (-3, "ENOMEM"), (-4, "EHIP"),
                       (-5, "ECAP")):
        assert word in L.status_string(code)


def test_invalid_host_arguments_rejected_without_device():
    L, lib = _lib()
    host_checks(L, lib)


def host_checks(L, lib):
    """Host-side argument validation through the C ABI, with no device involved (also run against the
    host-AddressSanitizer build of the library by tests/test_host_asan.py)."""
    out = ctypes.c_void_p(123)
    # null config / weights
    assert lib.mla_absorb_weights(None, None, None, None, ctypes.byref(out)) == L.MLA_EINVAL
    assert out.value is None
    cfg = L.MLAConfig(16, 512, 128, 64, 128, 16, L.MLA_BF16, 0.0, 1e-6, 1e4, 64, 64, 4096, 4096)
    assert lib.mla_absorb_weights(ctypes.byref(cfg), None, None, None, ctypes.byref(out)) == L.MLA_EINVAL
    # unsupported dims are refused before any allocation
    fake = ctypes.c_void_p(0x1000)
    for field, val in (("kv_lora_rank", 256), ("qk_rope_head_dim", 32), ("block_size", 64), ("num_heads", 24),
                       ("dtype", 7)):
        bad = L.MLAConfig.from_buffer_copy(cfg)
        setattr(bad, field, val)
        assert lib.mla_absorb_weights(ctypes.byref(bad), fake, None, None, ctypes.byref(out)) == L.MLA_EUNSUPPORTED
    bad = L.MLAConfig.from_buffer_copy(cfg)
    bad.max_q_tokens = 0
    assert lib.mla_absorb_weights(ctypes.byref(bad), fake, None, None, ctypes.byref(out)) == L.MLA_EINVAL
    # null context
    assert lib.mla_cache_write(None, None, 512, None, 64, None, None, 1, None, 1, None) == L.MLA_EINVAL
    assert lib.mla_decode(None, None, 1, 1, None, 1, None, 1, None, 1, None, None) == L.MLA_EINVAL
    assert lib.mla_set_decode_tuning(None, 1, 0) == L.MLA_EINVAL
    n = ctypes.c_size_t(7)
    assert lib.mla_prefill_workspace_size(None, 1, 1, 64, ctypes.byref(n)) == L.MLA_EINVAL
    assert lib.mla_ceiling_read(None, 16, None, 1 << 20, None) == L.MLA_EINVAL
    assert lib.mla_ceiling_mfma(2, 10, fake, 1 << 20, None, None) == L.MLA_EINVAL
    assert lib.mla_ceiling_mfma(0, 0, fake, 1 << 20, None, None) == L.MLA_EINVAL
    for code in range(-6, 2):
        assert lib.mla_status_string(code)
    lib.mla_free(None)
