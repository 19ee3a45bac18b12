"""Oracle: plain, slow CPU reference for fused indexer scoring + exact top-k.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``sparse_attention_indexer_fp8_amd``) and neither
imports the other.

What it computes (FlashTopK README, "Quick start", indexer-score equation):

    I[t,s] = sigma[s] * sum_{h<32} w[t,h] * ReLU(q[t,h,:] . kv[s,:])

for s in the half-open window [ks[t], ke[t]), then the topk keys by (score
desc, key index asc) -- README "What you can do": exact and deterministic,
ties keep the smallest key indices.  Short windows are padded with index -1 /
value -inf (DeepSelect README, "Variable-length rows").

The arithmetic lives in ``oracle.c`` (binary64 throughout, exact operand
decode, qsort); ``numpy_ref`` is an independent small-case twin in numpy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FP8_E4M3 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into oracle/_oracle.so with gcc + OpenMP."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-shared", "-fPIC",
           _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, dp, fp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_decode_e4m3fn.restype = ctypes.c_double
    lib.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_scores.restype = i32
    lib.oracle_scores.argtypes = [vp, vp, i32, fp, fp, i64, i64, i64, dp]
    lib.oracle_select.restype = i32
    lib.oracle_select.argtypes = [vp, vp, i32, fp, fp, vp, vp, i64, i64, i32, vp, i64,
                                  vp, vp, vp, vp, i32]
    lib.oracle_scores_h.restype = i32
    lib.oracle_scores_h.argtypes = [vp, vp, i32, i32, fp, fp, i64, i64, i64, dp]
    lib.oracle_select_h.restype = i32
    lib.oracle_select_h.argtypes = [vp, vp, i32, i32, fp, fp, vp, vp, i64, i64, i32, vp, i64,
                                    vp, vp, vp, vp, i32]
    lib.oracle_topk_rows.restype = i32
    lib.oracle_topk_rows.argtypes = [vp, i32, i64, i64, i64, vp, i32, vp, vp, i32]
    lib.oracle_max_threads.restype = i32
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _dtype_code(dtype) -> int:
    if dtype in (FP8_E4M3, "fp8", "fp8_e4m3", "e4m3"):
        return FP8_E4M3
    if dtype in (BF16, "bf16", "bfloat16"):
        return BF16
    raise ValueError(f"unsupported dtype {dtype!r}")


def _codes(a: np.ndarray, code: int) -> np.ndarray:
    want = np.uint8 if code == FP8_E4M3 else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"operand codes must be {want.__name__}, got {a.dtype}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode_e4m3fn(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_decode_e4m3fn(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def decode_bf16(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint16)
    return np.array([lib.oracle_decode_bf16(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def _heads(q, weights) -> int:
    """Head count from the operand shapes: q [num_q, heads, 128], weights [num_q, heads]."""
    h = int(q.shape[1])
    if np.shape(weights)[-1] != h:
        raise ValueError(f"weights have {np.shape(weights)[-1]} heads, q has {h}")
    return h


def scores(q, kv, dtype, kv_scales, weights, t: int, s_begin: int, s_end: int) -> np.ndarray:
    """Binary64 scores of query row t against keys [s_begin, s_end)."""
    lib = _load()
    code = _dtype_code(dtype)
    q, kv = _codes(q, code), _codes(kv, code)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    sc = None if kv_scales is None else np.ascontiguousarray(kv_scales, dtype=np.float32)
    out = np.empty(max(0, s_end - s_begin), dtype=np.float64)
    st = lib.oracle_scores_h(_ptr(q), _ptr(kv), code, _heads(q, w), _ptr(sc), _ptr(w), t, s_begin, s_end,
                             _ptr(out))
    if st != 0:
        raise ValueError("NaN operand code")
    return out


def select(q, kv, dtype, kv_scales, weights, ks, ke, topk: int, rows=None,
           nthreads: int = 0, all_scores: bool = False):
    """Exact top-k of the given rows (all rows when ``rows`` is None).

    Returns (idx int32 [n, topk], val float32 [n, topk], score float64 [n, topk],
    all float64 [n, num_kv] or None).  ``all`` holds every window score at its
    key position (NaN elsewhere).
    """
    lib = _load()
    code = _dtype_code(dtype)
    q, kv = _codes(q, code), _codes(kv, code)
    num_q, num_kv = q.shape[0], kv.shape[0]
    w = np.ascontiguousarray(weights, dtype=np.float32)
    sc = None if kv_scales is None else np.ascontiguousarray(kv_scales, dtype=np.float32)
    ks = np.ascontiguousarray(ks, dtype=np.int32)
    ke = np.ascontiguousarray(ke, dtype=np.int32)
    if rows is None:
        rows_arr = None
        n = num_q
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.shape[0]
    idx = np.empty((n, topk), dtype=np.int32)
    val = np.empty((n, topk), dtype=np.float32)
    sc64 = np.empty((n, topk), dtype=np.float64)
    allsc = np.empty((n, num_kv), dtype=np.float64) if all_scores else None
    st = lib.oracle_select_h(_ptr(q), _ptr(kv), code, _heads(q, w), _ptr(sc), _ptr(w), _ptr(ks), _ptr(ke),
                             num_q, num_kv, int(topk), _ptr(rows_arr), n, _ptr(idx), _ptr(val),
                             _ptr(sc64), _ptr(allsc), int(nthreads))
    if st != 0:
        raise ValueError(f"oracle_select failed with status {st}")
    return idx, val, sc64, allsc


def topk_rows(x, topk: int, ends=None, nthreads: int = 0):
    """Exact top-k of every row of a materialized score matrix.

    ``x``: float32 [rows, cols] or BF16 codes (uint16) [rows, cols]; ``ends``:
    per-row number of valid leading entries (None: all).  Returns (idx int32
    [rows, topk], val float32 [rows, topk]) ordered by value desc, index asc,
    padded with -1 / -inf."""
    lib = _load()
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        code = 0
    elif x.dtype == np.uint16:
        code = 1
    else:
        raise TypeError(f"x must be float32 or uint16 (BF16 codes), got {x.dtype}")
    rows, cols = x.shape
    e = None if ends is None else np.ascontiguousarray(ends, dtype=np.int32)
    idx = np.empty((rows, topk), dtype=np.int32)
    val = np.empty((rows, topk), dtype=np.float32)
    st = lib.oracle_topk_rows(_ptr(x), code, rows, cols, cols, _ptr(e), int(topk), _ptr(idx), _ptr(val),
                              int(nthreads))
    if st != 0:
        raise ValueError(f"oracle_topk_rows failed with status {st}")
    return idx, val


def max_threads() -> int:
    return int(_load().oracle_max_threads())
