"""ctypes front end of the fp64 dense attention oracle (``attention_dense.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The C source follows
the dense reference of the aiml.sh page "Speed up long contexts with
FlashAttention" (lab.py, standard_attention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_dense.c")
_LIB = os.path.join(_HERE, "liboracle_attention.so")
_lib = None

DTYPE_F32, DTYPE_BF16, DTYPE_F64 = 0, 1, 2


def default_threads() -> int:
    """Cores this process may run on, at most 16 (one GPU's share of an 8-GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def library_path() -> str:
    return _LIB


def build_library() -> str:
    """Compile the oracle with gcc (IEEE double, no contraction into FMA)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-shared", "-fPIC",
           "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_library()
        lib = ctypes.CDLL(_LIB)
        f = lib.oracle_attention_dense
        p, i64, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        f.argtypes = [p, p, p, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int, d,
                      p, i64, p, i64, p, p, ctypes.c_int, p]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _as_storage(x: np.ndarray, dtype_code: int) -> np.ndarray:
    want = {DTYPE_F32: np.float32, DTYPE_BF16: np.uint16, DTYPE_F64: np.float64}[dtype_code]
    if x.dtype != want:
        raise TypeError(f"expected {np.dtype(want)} storage for dtype code {dtype_code}, got {x.dtype}")
    return np.ascontiguousarray(x)


def attention_dense(q, k, v, causal: bool = True, scale: float | None = None,
                    dtype: str | None = None, bh_idx=None, row_idx=None, n_threads: int | None = None,
                    with_count: bool = False):
    """fp64 dense attention.

    ``q, k, v``: ``[B, H, S, D]`` (or ``[S, D]`` for one head) arrays in their
    storage type: float32, float64, or uint16 holding bfloat16 bit patterns
    (then pass ``dtype="bf16"``).  ``scale`` defaults to ``1/sqrt(D)`` in
    double.  ``bh_idx`` selects flattened ``b*H+h`` heads and ``row_idx`` query
    rows (default: all).  Returns ``(o, lse)`` as float64 with shapes
    ``[n_bh, n_rows, D]`` and ``[n_bh, n_rows]`` (plus the number of
    materialised score/probability elements when ``with_count``).
    """
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v)
    single = q.ndim == 2
    if single:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    B, H, S, D = q.shape
    if dtype is None:
        dtype = {np.dtype(np.float32): "f32", np.dtype(np.float64): "f64"}.get(q.dtype)
        if dtype is None:
            raise TypeError("pass dtype='bf16' for uint16 bfloat16 bit patterns")
    code = {"f32": DTYPE_F32, "bf16": DTYPE_BF16, "f64": DTYPE_F64}[dtype]
    q, k, v = (_as_storage(t, code) for t in (q, k, v))
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    bh = None if bh_idx is None else np.ascontiguousarray(bh_idx, dtype=np.int64)
    rows = None if row_idx is None else np.ascontiguousarray(row_idx, dtype=np.int64)
    n_bh = B * H if bh is None else bh.size
    n_rows = S if rows is None else rows.size
    o = np.empty((n_bh, n_rows, D), dtype=np.float64)
    lse = np.empty((n_bh, n_rows), dtype=np.float64)
    count = ctypes.c_int64(0)
    if n_threads is None:
        n_threads = default_threads()
    lib = _load()
    rc = lib.oracle_attention_dense(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, code, B, H, S, D, int(bool(causal)),
        float(scale), None if bh is None else bh.ctypes.data, n_bh,
        None if rows is None else rows.ctypes.data, n_rows, o.ctypes.data, lse.ctypes.data,
        int(n_threads), ctypes.addressof(count))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_dense failed with code {rc}")
    if single:
        o, lse = o[0], lse[0]
    return (o, lse, count.value) if with_count else (o, lse)
