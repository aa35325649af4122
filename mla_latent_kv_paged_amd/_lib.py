"""ctypes binding of libmla (include/mla.h): argument marshalling only.

Every step of the path runs in the HIP library.  PyTorch supplies device memory and the
current stream; this module checks tensor shapes/dtypes on the host and forwards raw
pointers.  There is no fallback: if libmla.so is missing or fails to load, the calls raise.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")

MLA_F32, MLA_BF16, MLA_BF16_FP8 = 0, 1, 2
FP8_ROW_BYTES = 656  # FP8 cache row: 512 e4m3 codes | 64 bf16 rope values | 4 fp32 group scales
MLA_OK, MLA_EINVAL, MLA_EUNSUPPORTED, MLA_ENOMEM, MLA_EHIP, MLA_ECAP = 0, -1, -2, -3, -4, -5
K_CACHE_WRITE, K_Q_ABSORB, K_DECODE, K_COMBINE = 0, 1, 2, 3
K_PF_EXPAND, K_PF_ATTN, K_PREP = 4, 5, 6
K_LAYER_QKV, K_LAYER_O = 7, 8
LAYER_INPUT_NORM, LAYER_RESIDUAL = 1, 2

EXPORTS = ("mla_absorb_weights", "mla_cache_write", "mla_decode", "mla_decode_step", "mla_decode_noalloc",
           "mla_free", "mla_status_string",
           "mla_set_decode_tuning", "mla_last_decode_shape", "mla_profile_enable", "mla_profile_read",
           "mla_profile_samples", "mla_prefill", "mla_prefill_workspace_size", "mla_layer_weights",
           "mla_layer_decode_step", "mla_ceiling_read", "mla_ceiling_gather", "mla_ceiling_mfma")


class MLAConfig(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_nope_head_dim", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_q_tokens", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_position", ctypes.c_int32), ("max_seq_len", ctypes.c_int32)]


class MLAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def load(path=None):
    """Load libmla.so (once).  Raises OSError if it is missing or does not load."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"libmla.so not found at {p}: build it with `python -m mla_latent_kv_paged_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mla_absorb_weights.argtypes = [ctypes.POINTER(MLAConfig), vp, vp, vp, ctypes.POINTER(vp)]
    lib.mla_absorb_weights.restype = i32
    lib.mla_cache_write.argtypes = [vp, vp, i64, vp, i64, vp, vp, i32, vp, i32, vp]
    lib.mla_cache_write.restype = i32
    lib.mla_decode.argtypes = [vp, vp, i32, i32, vp, i32, vp, i32, vp, i32, vp, vp]
    lib.mla_decode.restype = i32
    lib.mla_decode_noalloc.argtypes = [vp, vp, i32, i32, vp, i32, vp, i32, vp, i32, vp, vp]
    lib.mla_decode_noalloc.restype = i32
    lib.mla_decode_step.argtypes = [vp, vp, i64, vp, i64, vp, vp, i32, vp, i32, i32, vp, i32, vp, i32, vp, i32, vp, vp]
    lib.mla_decode_step.restype = i32
    lib.mla_prefill.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, vp, i32, vp, i32, vp, ctypes.c_size_t, vp, vp]
    lib.mla_prefill.restype = i32
    lib.mla_prefill_workspace_size.argtypes = [vp, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_workspace_size.restype = i32
    lib.mla_layer_weights.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp]
    lib.mla_layer_weights.restype = i32
    lib.mla_layer_decode_step.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, vp, i32, vp, vp]
    lib.mla_layer_decode_step.restype = i32
    lib.mla_ceiling_read.argtypes = [vp, i64, vp, i64, vp]
    lib.mla_ceiling_read.restype = i32
    lib.mla_ceiling_gather.argtypes = [vp, i32, i32, vp, i32, vp, i32, vp, i32, vp, i64, vp]
    lib.mla_ceiling_gather.restype = i32
    lib.mla_ceiling_mfma.argtypes = [i32, i32, vp, i64, ctypes.POINTER(ctypes.c_double), vp]
    lib.mla_ceiling_mfma.restype = i32
    lib.mla_free.argtypes = [vp]
    lib.mla_free.restype = None
    lib.mla_status_string.argtypes = [i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_set_decode_tuning.argtypes = [vp, i32, i32]
    lib.mla_set_decode_tuning.restype = i32
    lib.mla_last_decode_shape.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.mla_last_decode_shape.restype = i32
    lib.mla_profile_enable.argtypes = [vp, i32]
    lib.mla_profile_enable.restype = i32
    lib.mla_profile_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.mla_profile_read.restype = i32
    lib.mla_profile_samples.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
    lib.mla_profile_samples.restype = i32
    if path is None:
        _lib = lib
    return lib


def ceiling_read(src, sink, stream=None):
    """mla_ceiling_read: a plain streaming read of every byte of the device tensor src."""
    nbytes = int(src.numel() * src.element_size())
    _check(load().mla_ceiling_read(_ptr(src), nbytes, _ptr(sink), int(sink.numel() * sink.element_size()),
                                   _stream_ptr(stream)), "mla_ceiling_read")


def ceiling_mfma(shape, iterations, sink, stream=None):
    """mla_ceiling_mfma: the matrix cores' issue rate for shape 0 (16x16x32 bf16) or 1 (32x32x16 bf16);
    returns the launch's flop count."""
    flops = ctypes.c_double()
    _check(load().mla_ceiling_mfma(int(shape), int(iterations), _ptr(sink), int(sink.numel() * sink.element_size()),
                                   ctypes.byref(flops), _stream_ptr(stream)), "mla_ceiling_mfma")
    return flops.value


def status_string(status):
    try:
        return load().mla_status_string(int(status)).decode()
    except OSError:
        return f"status {status}"


def _check(status, where):
    if status != MLA_OK:
        raise MLAError(status, where)


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype=None, device=True, contiguous=True, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class MLAContext:
    """Owns one mla_ctx (absorbed weights, RoPE table, decode workspace)."""

    def __init__(self, kv_b_proj, gamma=None, *, num_heads, dtype="bf16", softmax_scale=0.0, rms_eps=1e-6,
                 rope_theta=10000.0, max_q_tokens=1024, max_batch=1024, max_position=32768, max_seq_len=32768,
                 stream=None):
        torch = _torch()
        self.lib = load()
        if dtype not in ("bf16", "f32", "fp8"):
            raise ValueError("dtype must be 'bf16', 'f32' or 'fp8' (bf16 with an FP8 cache)")
        self.storage = dtype
        self.tdtype = torch.float32 if dtype == "f32" else torch.bfloat16
        # cache tensors: [n, 16, 1, 576] of the storage dtype, or [n, 16, 1, 656] bytes for fp8
        self.cache_dtype = torch.uint8 if dtype == "fp8" else self.tdtype
        self.cache_row = FP8_ROW_BYTES if dtype == "fp8" else 576
        self.num_heads = num_heads
        _need(kv_b_proj, "kv_b_proj", self.tdtype, shape=(num_heads * 256, 512))
        if gamma is not None:
            _need(gamma, "gamma", self.tdtype, shape=(512,))
        cfg = MLAConfig(num_heads, 512, 128, 64, 128, 16, {"bf16": MLA_BF16, "f32": MLA_F32, "fp8": MLA_BF16_FP8}[dtype],
                        softmax_scale, rms_eps, rope_theta, max_q_tokens, max_batch, max_position, max_seq_len)
        self.cfg = cfg
        h = ctypes.c_void_p()
        _check(self.lib.mla_absorb_weights(ctypes.byref(cfg), _ptr(kv_b_proj), _ptr(gamma), _stream_ptr(stream),
                                           ctypes.byref(h)), "mla_absorb_weights")
        self.handle = h

    # -- lifetime
    def free(self):
        if getattr(self, "handle", None) and self.handle.value:
            self.lib.mla_free(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    # -- the two per-step calls
    def cache_write(self, c_kv, k_pe, positions, slot_mapping, kv_cache, stream=None):
        w = self._write_args(c_kv, k_pe, positions, slot_mapping, kv_cache)
        st = self.lib.mla_cache_write(self.handle, *w, _ptr(kv_cache), int(kv_cache.shape[0]), _stream_ptr(stream))
        _check(st, "mla_cache_write")

    def _write_args(self, c_kv, k_pe, positions, slot_mapping, kv_cache):
        torch = _torch()
        T = int(positions.shape[0]) if positions is not None else 0
        _need(kv_cache, "kv_cache", self.cache_dtype)
        if kv_cache.dim() != 4 or tuple(kv_cache.shape[1:]) != (16, 1, self.cache_row):
            raise ValueError(f"kv_cache must be [n_blocks, 16, 1, {self.cache_row}]")
        if T:
            _need(c_kv, "c_kv", self.tdtype, contiguous=False)
            _need(k_pe, "k_pe", self.tdtype, contiguous=False)
            _need(positions, "positions", torch.int32, shape=(T,))
            _need(slot_mapping, "slot_mapping", torch.int32, shape=(T,))
            if c_kv.shape != (T, 512) or c_kv.stride(1) != 1 or k_pe.shape != (T, 64) or k_pe.stride(1) != 1:
                raise ValueError("c_kv must be [T, 512] and k_pe [T, 64] with unit inner stride")
        return (_ptr(c_kv), c_kv.stride(0) if T else 512, _ptr(k_pe), k_pe.stride(0) if T else 64, _ptr(positions),
                _ptr(slot_mapping), T)

    def decode_step(self, c_kv, k_pe, positions, slot_mapping, q, kv_cache, block_table, seq_lens, max_seq_len,
                    q_len=1, out=None, stream=None):
        """cache_write(c_kv, k_pe, positions, slot_mapping, kv_cache) then decode(q, kv_cache, ...), as one
        call (mla_decode_step): the same results, the cache write in the query absorption's launch."""
        torch = _torch()
        w = self._write_args(c_kv, k_pe, positions, slot_mapping, kv_cache)
        H = self.num_heads
        batch = int(seq_lens.shape[0])
        _need(q, "q", self.tdtype, shape=(batch * q_len, H, 192))
        _need(block_table, "block_table", torch.int32)
        _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
        if block_table.dim() != 2 or block_table.shape[0] != batch:
            raise ValueError("block_table must be [batch, stride]")
        if out is None:
            out = torch.empty((batch * q_len, H, 128), dtype=self.tdtype, device=q.device)
        _need(out, "out", self.tdtype, shape=(batch * q_len, H, 128))
        st = self.lib.mla_decode_step(self.handle, *w, _ptr(q), batch, q_len, _ptr(kv_cache), int(kv_cache.shape[0]),
                                      _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
                                      int(max_seq_len), _ptr(out), _stream_ptr(stream))
        _check(st, "mla_decode_step")
        return out

    def decode(self, q, kv_cache, block_table, seq_lens, max_seq_len, q_len=1, out=None, stream=None):
        torch = _torch()
        H = self.num_heads
        batch = int(seq_lens.shape[0])
        _need(q, "q", self.tdtype, shape=(batch * q_len, H, 192))
        _need(kv_cache, "kv_cache", self.cache_dtype)
        if kv_cache.dim() != 4 or tuple(kv_cache.shape[1:]) != (16, 1, self.cache_row):
            raise ValueError(f"kv_cache must be [n_blocks, 16, 1, {self.cache_row}]")
        _need(block_table, "block_table", torch.int32)
        _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
        if block_table.dim() != 2 or block_table.shape[0] != batch:
            raise ValueError("block_table must be [batch, stride]")
        if out is None:
            out = torch.empty((batch * q_len, H, 128), dtype=self.tdtype, device=q.device)
        _need(out, "out", self.tdtype, shape=(batch * q_len, H, 128))
        st = self.lib.mla_decode(self.handle, _ptr(q), batch, q_len, _ptr(kv_cache), int(kv_cache.shape[0]),
                                 _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(max_seq_len),
                                 _ptr(out), _stream_ptr(stream))
        _check(st, "mla_decode")
        return out

    def decode_noalloc(self, q, kv_cache, block_table, seq_lens, max_seq_len, out, q_len=1, stream=None):
        """mla_decode_noalloc: mla_decode on the library's static scratch region; allocates nothing, so
        `out` must be given (device [batch*q_len, H, 128] of the storage dtype)."""
        torch = _torch()
        H = self.num_heads
        batch = int(seq_lens.shape[0])
        _need(q, "q", self.tdtype, shape=(batch * q_len, H, 192))
        _need(kv_cache, "kv_cache", self.cache_dtype)
        if kv_cache.dim() != 4 or tuple(kv_cache.shape[1:]) != (16, 1, self.cache_row):
            raise ValueError(f"kv_cache must be [n_blocks, 16, 1, {self.cache_row}]")
        _need(block_table, "block_table", torch.int32)
        _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
        if block_table.dim() != 2 or block_table.shape[0] != batch:
            raise ValueError("block_table must be [batch, stride]")
        _need(out, "out", self.tdtype, shape=(batch * q_len, H, 128))
        st = self.lib.mla_decode_noalloc(self.handle, _ptr(q), batch, q_len, _ptr(kv_cache), int(kv_cache.shape[0]),
                                         _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
                                         int(max_seq_len), _ptr(out), _stream_ptr(stream))
        _check(st, "mla_decode_noalloc")
        return out

    def layer_weights(self, q_proj, kv_a_proj, o_proj, input_norm_gamma=None, *, input_norm=True, residual=True,
                      stream=None):
        """mla_layer_weights: attach one layer's projections (bf16 device tensors q_proj [H*192, D],
        kv_a_proj [576, D], o_proj [D, H*128], input_norm_gamma [D] or None)."""
        H = self.num_heads
        D = int(q_proj.shape[1]) if q_proj is not None and q_proj.dim() == 2 else 0
        _need(q_proj, "q_proj", self.tdtype, shape=(H * 192, D))
        _need(kv_a_proj, "kv_a_proj", self.tdtype, shape=(576, D))
        _need(o_proj, "o_proj", self.tdtype, shape=(D, H * 128))
        if input_norm_gamma is not None:
            _need(input_norm_gamma, "input_norm_gamma", self.tdtype, shape=(D,))
        flags = (LAYER_INPUT_NORM if input_norm else 0) | (LAYER_RESIDUAL if residual else 0)
        _check(self.lib.mla_layer_weights(self.handle, D, _ptr(q_proj), _ptr(kv_a_proj), _ptr(o_proj),
                                          _ptr(input_norm_gamma), flags, _stream_ptr(stream)), "mla_layer_weights")
        self.hidden_dim = D

    def layer_decode_step(self, hidden, positions, slot_mapping, kv_cache, block_table, seq_lens, max_seq_len,
                          q_len=1, out=None, stream=None):
        """mla_layer_decode_step: hidden [batch*q_len, D] -> out [batch*q_len, D] (out may be hidden)."""
        torch = _torch()
        batch = int(seq_lens.shape[0])
        n = batch * q_len
        D = getattr(self, "hidden_dim", 0)
        _need(hidden, "hidden", self.tdtype, shape=(n, D))
        _need(positions, "positions", torch.int32, shape=(n,))
        _need(slot_mapping, "slot_mapping", torch.int32, shape=(n,))
        _need(kv_cache, "kv_cache", self.cache_dtype)
        if kv_cache.dim() != 4 or tuple(kv_cache.shape[1:]) != (16, 1, self.cache_row):
            raise ValueError(f"kv_cache must be [n_blocks, 16, 1, {self.cache_row}]")
        _need(block_table, "block_table", torch.int32)
        _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
        if block_table.dim() != 2 or block_table.shape[0] != batch:
            raise ValueError("block_table must be [batch, stride]")
        if out is None:
            out = torch.empty((n, D), dtype=self.tdtype, device=hidden.device)
        _need(out, "out", self.tdtype, shape=(n, D))
        st = self.lib.mla_layer_decode_step(self.handle, _ptr(hidden), _ptr(positions), _ptr(slot_mapping), batch,
                                            q_len, _ptr(kv_cache), int(kv_cache.shape[0]), _ptr(block_table),
                                            int(block_table.shape[1]), _ptr(seq_lens), int(max_seq_len), _ptr(out),
                                            _stream_ptr(stream))
        _check(st, "mla_layer_decode_step")
        return out

    def prefill_workspace_size(self, batch, total_q, max_seq_len):
        n = ctypes.c_size_t()
        _check(self.lib.mla_prefill_workspace_size(self.handle, int(batch), int(total_q), int(max_seq_len),
                                                   ctypes.byref(n)), "mla_prefill_workspace_size")
        return n.value

    def prefill(self, q, cu_q_lens, kv_cache, block_table, seq_lens, max_seq_len, max_q_len, workspace=None,
                out=None, stream=None):
        """Chunked prefill (mla_prefill): q [total_q, H, 192]; cu_q_lens int32 [batch + 1] on the device.
        A workspace of mla_prefill_workspace_size bytes is allocated here when none is given."""
        torch = _torch()
        H = self.num_heads
        batch = int(seq_lens.shape[0])
        total_q = int(q.shape[0])
        _need(q, "q", self.tdtype, shape=(total_q, H, 192))
        _need(cu_q_lens, "cu_q_lens", torch.int32, shape=(batch + 1,))
        _need(kv_cache, "kv_cache", self.cache_dtype)
        if kv_cache.dim() != 4 or tuple(kv_cache.shape[1:]) != (16, 1, self.cache_row):
            raise ValueError(f"kv_cache must be [n_blocks, 16, 1, {self.cache_row}]")
        _need(block_table, "block_table", torch.int32)
        _need(seq_lens, "seq_lens", torch.int32, shape=(batch,))
        if block_table.dim() != 2 or block_table.shape[0] != batch:
            raise ValueError("block_table must be [batch, stride]")
        need = self.prefill_workspace_size(batch, total_q, max_seq_len)
        if workspace is None:
            workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
        _need(workspace, "workspace", torch.uint8)
        if out is None:
            out = torch.empty((total_q, H, 128), dtype=self.tdtype, device=q.device)
        _need(out, "out", self.tdtype, shape=(total_q, H, 128))
        st = self.lib.mla_prefill(self.handle, _ptr(q), _ptr(cu_q_lens), batch, total_q, int(max_q_len),
                                  _ptr(kv_cache), int(kv_cache.shape[0]), _ptr(block_table), int(block_table.shape[1]),
                                  _ptr(seq_lens), int(max_seq_len), _ptr(workspace), int(workspace.numel()),
                                  _ptr(out), _stream_ptr(stream))
        _check(st, "mla_prefill")
        return out

    # -- measurement kernels (not part of the compute path)
    def ceiling_gather(self, kv_cache, block_table, seq_lens, max_seq_len, sink, q_len=1, stream=None):
        """mla_ceiling_gather: the 16-row decode kernel's HBM->LDS block stream alone, for this decode."""
        batch = int(seq_lens.shape[0])
        _check(self.lib.mla_ceiling_gather(self.handle, batch, q_len, _ptr(kv_cache), int(kv_cache.shape[0]),
                                           _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
                                           int(max_seq_len), _ptr(sink), int(sink.numel() * sink.element_size()),
                                           _stream_ptr(stream)), "mla_ceiling_gather")

    # -- helpers
    def set_decode_tuning(self, split_blocks=0, waves=0):
        _check(self.lib.mla_set_decode_tuning(self.handle, int(split_blocks), int(waves)), "mla_set_decode_tuning")

    def last_decode_shape(self):
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self.lib.mla_last_decode_shape(self.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
               "mla_last_decode_shape")
        return dict(split_blocks=a.value, n_split=b.value, waves=c.value)

    def profile_enable(self, on=True):
        _check(self.lib.mla_profile_enable(self.handle, 1 if on else 0), "mla_profile_enable")

    def profile_read(self, kernel_id):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(self.lib.mla_profile_read(self.handle, int(kernel_id), ctypes.byref(ms), ctypes.byref(n)),
               "mla_profile_read")
        return ms.value, n.value

    def profile_samples(self, kernel_id, max_n=1024):
        """Durations (ms) of the most recent launches of a kernel, oldest first."""
        buf = (ctypes.c_float * max_n)()
        n = ctypes.c_int32()
        _check(self.lib.mla_profile_samples(self.handle, int(kernel_id), buf, int(max_n), ctypes.byref(n)),
               "mla_profile_samples")
        return list(buf[:n.value])

