"""Python entry to the C++ oracle (``oracle_topk.cpp``). TEST INFRASTRUCTURE ONLY.

The library is built with g++ on first use (or by ``build()``); it is plain host C++.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_topk.cpp")
# DS_ORACLE_LIB names another build of the same source (the sanitizer test's); it is then
# loaded as it is, not rebuilt
_LIB = os.environ.get("DS_ORACLE_LIB") or os.path.join(_HERE, "liboracle_topk.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle library in place (g++, -O2, pthreads). Returns its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.environ.get("DS_ORACLE_LIB"):
                build()
            lib = ctypes.CDLL(_LIB)
            lib.oracle_topk.restype = ctypes.c_int
            lib.oracle_topk.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
            lib.oracle_hw_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def hw_threads() -> int:
    return int(_load().oracle_hw_threads())


def topk(x: np.ndarray, k: int, values: bool = True, indices: bool = True,
         threads: Optional[int] = None) -> Tuple[Optional[np.ndarray], Optional[np.ndarray]]:
    """Top-k of every row of ``x`` (2-D; uint16 = bf16 bits, float32 = fp32).

    Returns (values [rows,k] in the input's dtype, indices [rows,k] int32); either may be
    skipped. Ordering: value descending, +0 before -0, then index ascending.
    """
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    if x.dtype == np.uint16:
        dtype = 0
    elif x.dtype == np.float32:
        dtype = 1
    else:
        raise ValueError("x must be uint16 (bf16 bits) or float32")
    x = np.ascontiguousarray(x)
    rows, n = x.shape
    vals = np.empty((rows, k), x.dtype) if values else None
    idx = np.empty((rows, k), np.int32) if indices else None
    rc = _load().oracle_topk(x.ctypes.data, rows, n, n, int(k), dtype,
                             vals.ctypes.data if vals is not None else None,
                             idx.ctypes.data if idx is not None else None, int(threads or 0))
    if rc != 0:
        raise ValueError(f"oracle_topk rejected the arguments (rows={rows}, n={n}, k={k})")
    return vals, idx


def padding_value(dtype) -> np.ndarray:
    """The value bit pattern of an output position past a short row's length: all ones (a
    NaN, which no input holds), as a 0-d array of the input's dtype."""
    return np.array(0xFFFF, np.uint16) if np.dtype(dtype) == np.uint16 else np.array(0xFFFFFFFF, np.uint32).view(np.float32)


def topk_ragged(x: np.ndarray, lens: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k of ragged rows: row r is x[r, :L] with L = min(max(lens[r], 0), n) (a per-row
    valid length, TileLang tutorial chapter 37, section 5.2(1)). A row of L < k elements
    gives its L top elements in order, then k - L padding positions (index -1, value bits
    all ones). Rows of one length are passed to ``topk`` together."""
    rows, n = x.shape
    L = np.clip(np.asarray(lens, np.int64), 0, n)
    vals = np.empty((rows, k), x.dtype)
    vals[...] = padding_value(x.dtype)
    idx = np.full((rows, k), -1, np.int32)
    for length in np.unique(L):
        kk = min(k, int(length))
        if kk == 0:
            continue
        sel = np.nonzero(L == length)[0]
        v, i = topk(x[sel, :int(length)], kk)
        vals[sel, :kk] = v
        idx[sel, :kk] = i
    return vals, idx
