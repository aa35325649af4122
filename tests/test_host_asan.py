"""The library's host code under AddressSanitizer (CPU, no device).

libmla is built a second time with AddressSanitizer on its host code only (build.build_asan: every
sanitizer flag after -Xarch_host; the device code is unchanged), and a child process with the
sanitizer runtime preloaded runs the host-side ABI checks of tests/test_abi.py against it, plus a
context creation that fails for want of a device (its cleanup path).  Any sanitizer report fails the
test.  Leak detection is off: the Python interpreter itself does not free everything at exit."""

import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import ctypes, sys
    sys.path.insert(0, {root!r})
    from mla_latent_kv_paged_amd import _lib as L
    from tests.test_abi import host_checks
    lib = L.load({lib!r})
    host_checks(L, lib)
    # a well-formed context whose creation fails on a host without a device: the error path frees
    # what it had set up
    cfg = L.MLAConfig(16, 512, 128, 64, 128, 16, L.MLA_BF16, 0.0, 1e-6, 1e4, 64, 64, 4096, 4096)
    out = ctypes.c_void_p(123)
    st = lib.mla_absorb_weights(ctypes.byref(cfg), ctypes.c_void_p(0x1000), None, None, ctypes.byref(out))
    assert st != L.MLA_OK and out.value is None, (st, out.value)
    print("HOST-ASAN-CHILD-OK")
""")


def test_host_code_under_address_sanitizer():
    from mla_latent_kv_paged_amd import build as B
    try:
        rt = B.asan_runtime()
    except RuntimeError:
        rt = None
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = B.build_asan()
    env = dict(os.environ)
    # the sanitizer runtime goes first among the preloaded libraries; anything already preloaded stays
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # host code only
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib)], env=env, capture_output=True,
                       text=True, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and "HOST-ASAN-CHILD-OK" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
