"""Python binding of libswa.so: sliding-window GQA attention over a rolling-buffer KV cache.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libswa.so`` (built in-tree by ``sliding_window_gqa_swa_amd.build``);
PyTorch provides device memory and the current HIP stream.  If the library is
missing, every entry point raises :class:`SwaLibraryMissing` -- there is no
fallback implementation.

The functions carry the names of the C entry points (``include/swa.h``):
``swa_abi_version``, ``swa_status_string``, ``swa_cache_write``,
``swa_prefill_chunk``, ``swa_decode_workspace_size``, ``swa_decode``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "SWA_DTYPE_BF16", "SWA_DTYPE_F32", "SWA_OK", "SWA_ERR_INVALID_ARGUMENT", "SWA_ERR_UNSUPPORTED",
    "SWA_ERR_WORKSPACE", "SWA_ERR_HIP", "SWA_ERR_INTERNAL", "SwaError", "SwaLibraryMissing",
    "SwaCacheC", "SwaBatchC", "Cache", "Batch", "lib", "lib_path",
    "swa_abi_version", "swa_status_string", "swa_cache_write", "swa_prefill_chunk", "swa_prefill_chunk_no_tile_skip",
    "swa_decode_workspace_size", "swa_decode", "swa_decode_step", "swa_decode_step_noalloc",
]

SWA_DTYPE_BF16 = 0
SWA_DTYPE_F32 = 1
SWA_OK = 0
SWA_ERR_INVALID_ARGUMENT = 1
SWA_ERR_UNSUPPORTED = 2
SWA_ERR_WORKSPACE = 3
SWA_ERR_HIP = 4
SWA_ERR_INTERNAL = 5

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libswa.so")
_lib = None


class SwaLibraryMissing(RuntimeError):
    pass


class SwaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {swa_status_string(code)} (status {code})")


class SwaCacheC(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_cache", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SwaBatchC(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("max_new_tokens", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("start_pos", ctypes.c_void_p), ("cache_idx", ctypes.c_void_p),
                ("h_cu_seqlens", ctypes.c_void_p), ("h_start_pos", ctypes.c_void_p),
                ("h_cache_idx", ctypes.c_void_p)]


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libswa.so (raises SwaLibraryMissing when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise SwaLibraryMissing(f"{_LIB_PATH} is missing: build it with "
                                "`python -m sliding_window_gqa_swa_amd.build` (no fallback exists)")
    # torch carries its own HIP runtime (SONAME libamdhip64.so.7) and loads it under
    # another file name.  Loaded first, it satisfies libswa.so's dependency, so the
    # library and torch share one runtime.  Loaded after libswa.so, it would come in
    # as a second runtime, and the library's launches on torch's memory and streams
    # would fail.
    import torch  # noqa: F401
    L = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    L.swa_abi_version.restype = ctypes.c_int
    L.swa_abi_version.argtypes = []
    L.swa_status_string.restype = ctypes.c_char_p
    L.swa_status_string.argtypes = [ctypes.c_int]
    L.swa_cache_write.restype = ctypes.c_int
    L.swa_cache_write.argtypes = [P(SwaCacheC), P(SwaBatchC), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.swa_prefill_chunk.restype = ctypes.c_int
    L.swa_prefill_chunk.argtypes = [P(SwaCacheC), P(SwaBatchC), ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.c_void_p]
    L.swa_prefill_chunk_no_tile_skip.restype = ctypes.c_int
    L.swa_prefill_chunk_no_tile_skip.argtypes = L.swa_prefill_chunk.argtypes
    L.swa_decode_workspace_size.restype = ctypes.c_size_t
    L.swa_decode_workspace_size.argtypes = [P(SwaCacheC), ctypes.c_int32, ctypes.c_int32]
    L.swa_decode.restype = ctypes.c_int
    L.swa_decode.argtypes = [P(SwaCacheC), P(SwaBatchC), ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.swa_decode_step.restype = ctypes.c_int
    L.swa_decode_step.argtypes = [P(SwaCacheC), P(SwaBatchC), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]
    L.swa_decode_step_noalloc.restype = ctypes.c_int
    L.swa_decode_step_noalloc.argtypes = [P(SwaCacheC), P(SwaBatchC), ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                          ctypes.c_void_p]
    _lib = L
    return L


# ----------------------------------------------------------------------------- marshalling

def _ptr(x) -> Optional[int]:
    """Device/host address of a torch tensor, numpy array or raw int (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()  # torch.Tensor


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SWA_DTYPE_BF16
    if t.dtype == torch.float32:
        return SWA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


class Cache:
    """A rolling-buffer cache: device tensors k, v of shape [n_cache, n_kv_heads, window, head_dim]."""

    def __init__(self, k, v):
        if k.shape != v.shape or k.dim() != 4 or k.dtype != v.dtype:
            raise ValueError("k and v must be 4-D tensors of one shape and dtype")
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("cache tensors must be contiguous")
        self.k, self.v = k, v

    @property
    def window(self) -> int:
        return int(self.k.shape[2])

    def c_struct(self) -> SwaCacheC:
        n_cache, hkv, w, d = (int(x) for x in self.k.shape)
        return SwaCacheC(_ptr(self.k), _ptr(self.v), n_cache, hkv, d, w, _dtype_code(self.k), 0)


def cache_struct(k, v, n_cache: int, n_kv_heads: int, head_dim: int, window: int, dtype: int) -> SwaCacheC:
    """C struct from raw pointers (k or v may be None)."""
    return SwaCacheC(_ptr(k), _ptr(v), n_cache, n_kv_heads, head_dim, window, dtype, 0)


class Batch:
    """Sequence metadata of one call: lengths of the new tokens, start positions, cache rows.

    Builds the device int32 arrays (on ``device``) and keeps host mirrors, which
    the library validates.
    """

    def __init__(self, lengths: Sequence[int], start_pos: Sequence[int], cache_idx: Optional[Sequence[int]] = None,
                 device="cuda", mirrors: bool = True):
        import torch
        n = len(lengths)
        self.h_cu = np.zeros(n + 1, dtype=np.int32)
        self.h_cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int32)
        self.h_sp = np.ascontiguousarray(start_pos, dtype=np.int32)
        self.h_ci = None if cache_idx is None else np.ascontiguousarray(cache_idx, dtype=np.int32)
        self.num_seqs = n
        self.total_tokens = int(self.h_cu[-1])
        self.max_new_tokens = int(max(lengths)) if n else 0
        self.cu = torch.from_numpy(self.h_cu.copy()).to(device)
        self.sp = torch.from_numpy(self.h_sp.copy()).to(device)
        self.ci = None if self.h_ci is None else torch.from_numpy(self.h_ci.copy()).to(device)
        self.mirrors = mirrors

    def c_struct(self) -> SwaBatchC:
        m = self.mirrors
        return SwaBatchC(self.num_seqs, self.total_tokens, self.max_new_tokens, 0,
                         _ptr(self.cu), _ptr(self.sp), _ptr(self.ci),
                         _ptr(self.h_cu) if m else None, _ptr(self.h_sp) if m else None,
                         _ptr(self.h_ci) if (m and self.h_ci is not None) else None)


def _as_cache(cache) -> SwaCacheC:
    return cache if isinstance(cache, SwaCacheC) else cache.c_struct()


def _as_batch(batch) -> SwaBatchC:
    return batch if isinstance(batch, SwaBatchC) else batch.c_struct()


def _check(code: int, where: str) -> int:
    if code != SWA_OK:
        raise SwaError(code, where)
    return code


# ----------------------------------------------------------------------------- entry points

def swa_abi_version() -> int:
    return lib().swa_abi_version()


def swa_status_string(code: int) -> str:
    return lib().swa_status_string(int(code)).decode()


def swa_cache_write(cache, batch, k_new, v_new, stream=None, check: bool = True) -> int:
    """Write the new tokens' K/V into ring slots position mod W (see include/swa.h)."""
    c, b = _as_cache(cache), _as_batch(batch)
    code = lib().swa_cache_write(ctypes.byref(c), ctypes.byref(b), _ptr(k_new), _ptr(v_new), _stream(stream))
    return _check(code, "swa_cache_write") if check else code


def swa_prefill_chunk(cache, batch, q, n_q_heads: int, k_new, v_new, sm_scale: float, out, stream=None,
                      check: bool = True) -> int:
    """Chunked sliding-window GQA prefill (reads the cache, never writes it)."""
    c, b = _as_cache(cache), _as_batch(batch)
    code = lib().swa_prefill_chunk(ctypes.byref(c), ctypes.byref(b), _ptr(q), int(n_q_heads), _ptr(k_new),
                                   _ptr(v_new), float(sm_scale), _ptr(out), _stream(stream))
    return _check(code, "swa_prefill_chunk") if check else code


def swa_prefill_chunk_no_tile_skip(cache, batch, q, n_q_heads: int, k_new, v_new, sm_scale: float, out,
                                   stream=None, check: bool = True) -> int:
    """swa_prefill_chunk without the band tile skip (every causal key tile visited, out-of-band keys
    masked): same result, for measuring what the skip saves."""
    c, b = _as_cache(cache), _as_batch(batch)
    code = lib().swa_prefill_chunk_no_tile_skip(ctypes.byref(c), ctypes.byref(b), _ptr(q), int(n_q_heads),
                                                _ptr(k_new), _ptr(v_new), float(sm_scale), _ptr(out),
                                                _stream(stream))
    return _check(code, "swa_prefill_chunk_no_tile_skip") if check else code


def swa_decode_workspace_size(cache, num_seqs: int, n_q_heads: int) -> int:
    c = _as_cache(cache)
    return int(lib().swa_decode_workspace_size(ctypes.byref(c), int(num_seqs), int(n_q_heads)))


def swa_decode(cache, batch, q, n_q_heads: int, sm_scale: float, out, workspace=None, workspace_bytes=None,
               stream=None, check: bool = True) -> int:
    """Single-token decode over the rolling buffer (the token must already be written)."""
    c, b = _as_cache(cache), _as_batch(batch)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().swa_decode(ctypes.byref(c), ctypes.byref(b), _ptr(q), int(n_q_heads), float(sm_scale), _ptr(out),
                            _ptr(workspace), int(workspace_bytes), _stream(stream))
    return _check(code, "swa_decode") if check else code


def swa_decode_step(cache, batch, q, n_q_heads: int, k_new, v_new, sm_scale: float, out, workspace=None,
                    workspace_bytes=None, stream=None, check: bool = True) -> int:
    """Fused decode step: writes the new token's K/V into its slot and attends, in one launch."""
    c, b = _as_cache(cache), _as_batch(batch)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().swa_decode_step(ctypes.byref(c), ctypes.byref(b), _ptr(q), int(n_q_heads), _ptr(k_new),
                                 _ptr(v_new), float(sm_scale), _ptr(out), _ptr(workspace), int(workspace_bytes),
                                 _stream(stream))
    return _check(code, "swa_decode_step") if check else code


def swa_decode_step_noalloc(cache, batch, q, n_q_heads: int, k_new, v_new, sm_scale: float, out, stream=None,
                            check: bool = True) -> int:
    """swa_decode_step with the merge partials in the library's own device array (no workspace argument)."""
    c, b = _as_cache(cache), _as_batch(batch)
    code = lib().swa_decode_step_noalloc(ctypes.byref(c), ctypes.byref(b), _ptr(q), int(n_q_heads), _ptr(k_new),
                                         _ptr(v_new), float(sm_scale), _ptr(out), _stream(stream))
    return _check(code, "swa_decode_step_noalloc") if check else code
