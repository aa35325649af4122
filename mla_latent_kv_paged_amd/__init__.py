"""MI355X-native (gfx950) MLA decode over a paged latent KV cache with matrix absorption.

The compute path is the HIP library libmla.so (C ABI in include/mla.h); this package holds its
sources (csrc/), the in-tree build script (build.py) and a thin ctypes binding (_lib.py).
"""
from ._lib import (MLAContext, MLAError, MLAConfig, load, status_string, LIB_PATH, EXPORTS,  # noqa: F401
                   K_CACHE_WRITE, K_Q_ABSORB, K_DECODE, K_COMBINE, K_PF_EXPAND, K_PF_ATTN, K_PREP,
                   K_LAYER_QKV, K_LAYER_O)
