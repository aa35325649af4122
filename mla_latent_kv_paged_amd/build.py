"""Build libmla.so in-tree with hipcc for gfx950.

    python -m mla_latent_kv_paged_amd.build          # compile every csrc/*.hip and link

The shared library lands next to this file (mla_latent_kv_paged_amd/libmla.so).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for all device code (-packed-fp32-ops); hipcc's host pass
# warns that it does not know the feature, which is harmless.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found")
    return h


# Per-source flags.  The decode kernels keep their MFMA accumulators in VGPRs so that the online
# softmax rescale runs on them in place (no AGPR<->VGPR copies); their block buffers then take the
# AGPR half of the register file.  The 32-row kernel uses the flag for its score MFMAs and pins its
# P.C accumulator to the AGPRs itself.  The prefill kernels build without it: the attention kernel's
# code is the same either way (two waves per SIMD leave no AGPRs), and the expansion kernel (one
# wave per SIMD) keeps its accumulators in AGPRs, which leaves VGPRs for reading ahead.
PER_FILE = {"decode_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
            "decode_bf16_mt32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
            "prefill_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src, extra, verbose, objdir=OBJDIR):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *PER_FILE.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose=False, extra_flags=(), objdir=OBJDIR, lib=LIB):
    """Compile every csrc/*.hip for gfx950 and link libmla.so. Returns the library path."""
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags), verbose, objdir), srcs))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


# AddressSanitizer on the host code only (every flag after -Xarch_host; the device code is built as
# usual).  The library leaves the sanitizer's symbols to the runtime, which the process preloads.
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
ASAN_OBJDIR = os.path.join(PKG, "_build_asan")
ASAN_LIB = os.path.join(ASAN_OBJDIR, "libmla_asan.so")


def build_asan(verbose=False):
    """libmla with host-side AddressSanitizer (for CPU tests of the host code). Returns its path."""
    return build(verbose, ASAN_HOST, ASAN_OBJDIR, ASAN_LIB)


def asan_runtime():
    """Path of the compiler's AddressSanitizer runtime for x86-64, or None."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
        return p
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
