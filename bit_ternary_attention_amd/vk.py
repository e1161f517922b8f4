"""Python binding of libvk.so: argument marshalling only.

Every step of the cache runs in the library's HIP kernels; torch is used for
device memory and streams.  Loading fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvk.so")

OK, ERR_ARG, ERR_OOM, ERR_CAPACITY, ERR_ALIGN, ERR_STATE, ERR_HIP = range(7)
DTYPE_F16, DTYPE_BF16 = 0, 1
FMT_TERNARY2, FMT_FP8E4M3, FMT_F16, FMT_LOSSLESS = 0, 1, 2, 3
N_FORMATS = 4
KERNELS = ("absmean", "finalize", "pack", "decode", "merge", "retier")
DECODE_DEFAULT, DECODE_VALU, DECODE_MFMA = 0, 1, 2

_c_i32, _c_i64, _c_f32, _c_u64, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint64, ctypes.c_void_p


class CacheConfig(ctypes.Structure):
    _fields_ = [("n_layers", _c_i32), ("n_kv_heads", _c_i32), ("n_q_heads", _c_i32), ("head_dim", _c_i32),
                ("block_size", _c_i32), ("max_seqs", _c_i32), ("max_tokens_per_seq", _c_i32),
                ("sink_tokens", _c_i32), ("sink_format", _c_i32), ("recent_tokens", _c_i32),
                ("recent_format", _c_i32), ("decode_kernel", _c_i32), ("fp8_dynamic", _c_i32), ("reserved0", _c_i32),
                ("pages_ternary", _c_i64), ("pages_fp8", _c_i64), ("pages_f16", _c_i64),
                ("eps", _c_f32), ("fp8_scale", _c_f32), ("page_shuffle_seed", _c_u64),
                ("pages_lossless", _c_i64)]


class Stats(ctypes.Structure):
    _fields_ = [("device_bytes", _c_i64), ("pool_pages", _c_i64 * 4), ("pages_used", _c_i64 * 4),
                ("tokens_stored", _c_i64 * 4), ("append_calls", _c_i64), ("decode_calls", _c_i64),
                ("last_decode_units", _c_i64 * 4), ("total_decode_units", _c_i64 * 4),
                ("last_decode_splits", _c_i32), ("last_decode_steal", _c_i32), ("retier_calls", _c_i64),
                ("pages_retiered", _c_i64), ("pages_evicted", _c_i64), ("last_decode_ordered", _c_i32),
                ("reserved", _c_i32)]

    def as_dict(self):
        out = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            out[name] = list(v) if hasattr(v, "__len__") else int(v)
        return out


EXPORTS = {
    "vk_config_defaults": (None, [ctypes.POINTER(CacheConfig)]),
    "vk_cache_device_bytes": (_c_i32, [ctypes.POINTER(CacheConfig), ctypes.POINTER(_c_i64)]),
    "vk_page_bytes": (_c_i64, [ctypes.POINTER(CacheConfig), _c_i32]),
    "vk_create_cache": (_c_i32, [ctypes.POINTER(CacheConfig), ctypes.POINTER(_c_vp)]),
    "vk_append": (_c_i32, [_c_vp, _c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_i32), _c_i32, _c_vp, _c_vp, _c_i32, _c_vp]),
    "vk_append_ragged": (_c_i32, [_c_vp, _c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32), _c_vp,
                                  _c_vp, _c_i32, _c_vp]),
    "vk_decode_attn": (_c_i32, [_c_vp, _c_i32, _c_i32, ctypes.POINTER(_c_i32), _c_vp, _c_i32, _c_i32, _c_f32,
                                _c_vp, _c_vp]),
    "vk_retier": (_c_i32, [_c_vp, _c_i32, ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i64), _c_vp]),
    "vk_evict": (_c_i32, [_c_vp, _c_i32, ctypes.POINTER(_c_i32), _c_i32, ctypes.POINTER(_c_i64), _c_vp]),
    "vk_reset_seqs": (_c_i32, [_c_vp, _c_i32, ctypes.POINTER(_c_i32), _c_vp]),
    "vk_seq_length": (_c_i32, [_c_vp, _c_i32, ctypes.POINTER(_c_i32)]),
    "vk_read_pages": (_c_i32, [_c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp, ctypes.POINTER(_c_i32),
                               ctypes.POINTER(_c_f32)]),
    "vk_get_stats": (_c_i32, [_c_vp, ctypes.POINTER(Stats)]),
    "vk_set_kernel_timing": (_c_i32, [_c_vp, _c_i32]),
    "vk_get_kernel_times": (_c_i32, [_c_vp, ctypes.POINTER(_c_i64), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double)]),
    "vk_release": (_c_i32, [_c_vp]),
    "vk_quantize_pack_workspace_bytes": (_c_i64, [_c_i64]),
    "vk_quantize_pack": (_c_i32, [_c_vp, _c_i64, _c_i32, _c_f32, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp]),
    "vk_quantize_pack_noalloc_max_elems": (_c_i64, []),
    "vk_quantize_pack_noalloc": (_c_i32, [_c_vp, _c_i64, _c_i32, _c_f32, _c_vp, _c_vp, _c_vp, _c_vp]),
    "vk_last_error": (ctypes.c_char_p, []),
    "vk_status_string": (ctypes.c_char_p, [_c_i32]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -m bit_ternary_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class VkError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{lib().vk_status_string(status).decode()}: {message}")


def _check(status: int) -> None:
    if status != OK:
        raise VkError(status, lib().vk_last_error().decode())


_id_arrays = {}  # recent sequence lists as int32 arrays (a decode loop passes the same list per layer)


def _ids(seq_ids: Sequence[int]):
    key = tuple(int(s) for s in seq_ids)
    arr = _id_arrays.get(key)
    if arr is None:
        if len(_id_arrays) >= 64:
            _id_arrays.clear()
        arr = _id_arrays[key] = (ctypes.c_int32 * len(key))(*key)
    return arr, len(key)


def _stream(stream, device_index=None):
    """The raw HIP stream handle: the given stream, else the current stream of the device."""
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None and device_index is not None:
            return raw(device_index)
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return DTYPE_F16
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError("tensor must be float16 or bfloat16")


def make_config(**kw) -> CacheConfig:
    cfg = CacheConfig()
    lib().vk_config_defaults(ctypes.byref(cfg))
    for k, v in kw.items():
        if not hasattr(cfg, k):
            raise TypeError(f"unknown config field {k}")
        setattr(cfg, k, v)
    return cfg


def device_bytes(cfg: CacheConfig) -> int:
    out = ctypes.c_int64()
    _check(lib().vk_cache_device_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def page_bytes(cfg: CacheConfig, fmt: int) -> int:
    return int(lib().vk_page_bytes(ctypes.byref(cfg), fmt))


class Cache:
    """A packed, tiered KV cache on the current HIP device."""

    def __init__(self, cfg: Optional[CacheConfig] = None, **kw):
        self.cfg = cfg if cfg is not None else make_config(**kw)
        h = ctypes.c_void_p()
        _check(lib().vk_create_cache(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h
        self._q_shape = (self.cfg.n_q_heads, self.cfg.head_dim)
        self._decode_fn = lib().vk_decode_attn

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("cache released")
        return self._h

    def append(self, k, v, seq_ids: Sequence[int], layer_begin: int = 0, stream=None) -> None:
        """k, v: [n_layers][n_seqs][n_tokens][Hkv][D] float16/bfloat16 device tensors."""
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 5:
            raise ValueError("k and v must have the same 5-d shape and dtype")
        if not (k.is_cuda and v.is_cuda and k.is_contiguous() and v.is_contiguous()):
            raise ValueError("k and v must be contiguous device tensors")
        if k.shape[1] != len(seq_ids) or k.shape[3] != self.cfg.n_kv_heads or k.shape[4] != self.cfg.head_dim:
            raise ValueError(f"k shape {tuple(k.shape)} does not match the cache / seq_ids")
        ids, n = _ids(seq_ids)
        _check(lib().vk_append(self.handle, layer_begin, k.shape[0], n, ids, k.shape[2], k.data_ptr(), v.data_ptr(),
                               _dtype_code(k), _stream(stream, k.get_device())))

    def append_ragged(self, k, v, seq_ids: Sequence[int], n_tokens: Sequence[int], layer_begin: int = 0,
                      stream=None) -> None:
        """k, v: [n_layers][sum(n_tokens)][Hkv][D] float16/bfloat16 device tensors; sequence i's
        tokens follow sequence i-1's within each layer."""
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
            raise ValueError("k and v must have the same 4-d shape and dtype")
        if not (k.is_cuda and v.is_cuda and k.is_contiguous() and v.is_contiguous()):
            raise ValueError("k and v must be contiguous device tensors")
        if len(n_tokens) != len(seq_ids) or k.shape[1] != sum(n_tokens) or k.shape[2] != self.cfg.n_kv_heads \
                or k.shape[3] != self.cfg.head_dim:
            raise ValueError(f"k shape {tuple(k.shape)} does not match the cache / n_tokens")
        ids, n = _ids(seq_ids)
        counts = (_c_i32 * n)(*[int(x) for x in n_tokens])
        _check(lib().vk_append_ragged(self.handle, layer_begin, k.shape[0], n, ids, counts, k.data_ptr(), v.data_ptr(),
                                      _dtype_code(k), _stream(stream, k.get_device())))

    def decode(self, q, seq_ids: Sequence[int], layer: int, window: int = -1, softmax_scale: float = 0.0,
               out=None, stream=None):
        """q: [n_seqs][Hq][D] device tensor -> float32 [n_seqs][Hq][D]."""
        import torch
        if not (q.is_cuda and q.is_contiguous()) or q.dim() != 3:
            raise ValueError("q must be a contiguous 3-d device tensor")
        ids, n = _ids(seq_ids)
        if q.shape[0] != n or q.shape[1:] != self._q_shape:
            raise ValueError(f"q shape {tuple(q.shape)} does not match the cache / seq_ids")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        elif out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor shaped like q")
        _check(self._decode_fn(self.handle, layer, n, ids, q.data_ptr(), _dtype_code(q), window, softmax_scale,
                               out.data_ptr(), _stream(stream, q.get_device())))
        return out

    def retier(self, seq_ids: Sequence[int], stream=None) -> int:
        """Moves the FP8 pages that left the recent window to the ternary tier; returns their count."""
        ids, n = _ids(seq_ids)
        out = ctypes.c_int64()
        _check(lib().vk_retier(self.handle, n, ids, ctypes.byref(out), _stream(stream)))
        return out.value

    def evict(self, seq_ids: Sequence[int], window: int, stream=None) -> int:
        """Frees the pages between the sinks and the last ``window`` tokens; returns their count."""
        ids, n = _ids(seq_ids)
        out = ctypes.c_int64()
        _check(lib().vk_evict(self.handle, n, ids, window, ctypes.byref(out), _stream(stream)))
        return out.value

    def reset(self, seq_ids: Sequence[int], stream=None) -> None:
        ids, n = _ids(seq_ids)
        _check(lib().vk_reset_seqs(self.handle, n, ids, _stream(stream)))

    def seq_length(self, seq: int) -> int:
        out = ctypes.c_int32()
        _check(lib().vk_seq_length(self.handle, seq, ctypes.byref(out)))
        return out.value

    def read_pages(self, layer: int, seq: int, page0: int, n_pages: int):
        """(bytes [n_pages, max page bytes] uint8, formats [n_pages], gamma [n_pages, 2])."""
        sizes = [page_bytes(self.cfg, f) for f in range(N_FORMATS)]
        if min(sizes) <= 0:
            raise RuntimeError("library reports no page size for some format")
        stride = max(sizes)   # the library lays pages out at the largest page size
        buf = np.zeros((n_pages, stride), dtype=np.uint8)
        fmt = np.zeros(n_pages, dtype=np.int32)
        gam = np.zeros((n_pages, 2), dtype=np.float32)
        _check(lib().vk_read_pages(self.handle, layer, seq, page0, n_pages, buf.ctypes.data_as(ctypes.c_void_p),
                                   fmt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   gam.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
        return buf, fmt, gam

    def stats(self) -> dict:
        s = Stats()
        _check(lib().vk_get_stats(self.handle, ctypes.byref(s)))
        return s.as_dict()

    def kernel_timing(self, enable: bool) -> None:
        """Start (clearing totals) or stop per-kernel event timing."""
        _check(lib().vk_set_kernel_timing(self.handle, 1 if enable else 0))

    def kernel_times(self) -> dict:
        """{kernel: (launches, milliseconds, algorithmic bytes)}; waits for the device."""
        n = len(KERNELS)
        la, ms, by = (ctypes.c_int64 * n)(), (ctypes.c_double * n)(), (ctypes.c_double * n)()
        _check(lib().vk_get_kernel_times(self.handle, la, ms, by))
        return {k: (int(la[i]), float(ms[i]), float(by[i])) for i, k in enumerate(KERNELS)}

    def close(self) -> None:
        if self._h is not None:
            h, self._h = self._h, None
            _check(lib().vk_release(h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quantize_pack_workspace_bytes(n: int) -> int:
    return int(lib().vk_quantize_pack_workspace_bytes(n))


def quantize_pack(x, eps: float = 1e-5, gamma=None, packed=None, gamma_out=None, workspace=None, stream=None):
    """Flat per-tensor quantise+pack of a float16/bfloat16 device tensor.

    Returns (packed uint8 [n/4], gamma float32 [1]) device tensors.  ``gamma``
    (a float32 device tensor of one element) replaces the computed mean |x|.
    """
    import torch
    if not (x.is_cuda and x.is_contiguous()):
        raise ValueError("x must be a contiguous device tensor")
    n = x.numel()
    if packed is None:
        packed = torch.empty(n // 4, dtype=torch.uint8, device=x.device)
    if gamma_out is None:
        gamma_out = torch.empty(1, dtype=torch.float32, device=x.device)
    wb = quantize_pack_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(wb, dtype=torch.uint8, device=x.device)
    gptr = ctypes.c_void_p(gamma.data_ptr()) if gamma is not None else ctypes.c_void_p(0)
    _check(lib().vk_quantize_pack(ctypes.c_void_p(x.data_ptr()), n, _dtype_code(x), eps, gptr,
                                  ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(gamma_out.data_ptr()),
                                  ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
    return packed, gamma_out


def quantize_pack_noalloc(x, packed, gamma_out, eps: float = 1e-5, gamma=None, stream=None):
    """vk_quantize_pack without a workspace (the library's own device scratch): the caller
    passes the input and both outputs (packed uint8 [n/4], gamma float32 [1])."""
    if not (x.is_cuda and x.is_contiguous()):
        raise ValueError("x must be a contiguous device tensor")
    n = x.numel()
    if packed.numel() != n // 4 or gamma_out.numel() < 1:
        raise ValueError("packed must hold n/4 bytes and gamma_out one float")
    gptr = ctypes.c_void_p(gamma.data_ptr()) if gamma is not None else ctypes.c_void_p(0)
    _check(lib().vk_quantize_pack_noalloc(ctypes.c_void_p(x.data_ptr()), n, _dtype_code(x), eps, gptr,
                                          ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(gamma_out.data_ptr()),
                                          _stream(stream)))
    return packed, gamma_out
