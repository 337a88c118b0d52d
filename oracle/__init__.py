"""Oracle for sliding-window GQA attention over a rolling-buffer KV cache.

TEST INFRASTRUCTURE ONLY.  The product package never imports this module;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` do.

Two independent CPU implementations live here:

* ``swa_oracle.c`` (built into ``liboracle.so`` with gcc + OpenMP): the plain
  definition in IEEE double, one (query, head) at a time, on absolute
  positions.  Wrapped by :func:`attend` and :func:`ring_write`.
* ``brute.py``: a dense numpy computation with an explicit N x N mask matrix,
  used to pin the C oracle on tiny inputs.

Source passages: Mistral 7B (Chinese translation), section 2 "Architectural
details" -- paragraphs "Sliding Window Attention", "Rolling Buffer Cache",
"Pre-fill and Chunking" and the captions of Figures 1-3; section 1 for GQA.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ORACLE_OK = 0
ORACLE_BAD_ARGUMENT = -1
ORACLE_MISSING_KEY = -2


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (-O2, OpenMP, strict IEEE double)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.swa_oracle_attend.restype = ctypes.c_int
    lib.swa_oracle_attend.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.swa_oracle_ring_write.restype = ctypes.c_int
    lib.swa_oracle_ring_write.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.swa_oracle_num_threads.restype = ctypes.c_int
    lib.swa_oracle_num_threads.argtypes = []
    lib.swa_oracle_set_num_threads.restype = None
    lib.swa_oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def num_threads() -> int:
    return _load().swa_oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads for the following oracle calls (timing only; results do not depend on it)."""
    _load().swa_oracle_set_num_threads(int(n))


def attend(q, q_pos, k, v, kv_pos0: int, window: int, scale: float) -> np.ndarray:
    """Sliding-window GQA attention of one sequence, on absolute positions.

    q: float32 [n_q, Hq, D] (exact input values); q_pos: int64 [n_q]
    k, v: float32 [n_kv, Hkv, D]; row t is absolute position ``kv_pos0 + t``
    Returns float64 [n_q, Hq, D].  Query position i attends to keys
    j in [max(0, i-W+1), i] (W keys: the Figure 1 caption bounds the window by W tokens).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    n_q, hq, d = q.shape
    n_kv, hkv, d2 = k.shape
    if d2 != d or v.shape != k.shape or q_pos.shape != (n_q,):
        raise ValueError("shape mismatch")
    out = np.empty((n_q, hq, d), dtype=np.float64)
    rc = lib.swa_oracle_attend(n_q, hq, hkv, d, int(window), float(scale),
                               q.ctypes.data, q_pos.ctypes.data, n_kv, int(kv_pos0),
                               k.ctypes.data, v.ctypes.data, out.ctypes.data)
    if rc != ORACLE_OK:
        raise ValueError(f"oracle attend failed with code {rc}")
    return out


def ring_write(ring: np.ndarray, rows: np.ndarray, cu_seqlens, start_pos, cache_idx=None) -> None:
    """Apply a batch of cache writes to ``ring`` in place (bytewise, in position order).

    ring: any-dtype array shaped [n_cache, Hkv, W, D]; rows: same dtype, [T, Hkv, D].
    """
    lib = _load()
    if not ring.flags.c_contiguous:
        raise ValueError("ring must be contiguous")
    rows = np.ascontiguousarray(rows)
    if rows.dtype != ring.dtype:
        raise ValueError("dtype mismatch")
    n_cache, hkv, window, d = ring.shape
    row_bytes = d * ring.dtype.itemsize
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    sp = np.ascontiguousarray(start_pos, dtype=np.int32)
    num_seqs = sp.shape[0]
    ci = None if cache_idx is None else np.ascontiguousarray(cache_idx, dtype=np.int32)
    rc = lib.swa_oracle_ring_write(ring.ctypes.data, n_cache, hkv, window, row_bytes,
                                   rows.ctypes.data, num_seqs, cu.ctypes.data, sp.ctypes.data,
                                   None if ci is None else ci.ctypes.data)
    if rc != ORACLE_OK:
        raise ValueError(f"oracle ring_write failed with code {rc}")
