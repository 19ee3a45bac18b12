"""Python binding of the gfx950 fused indexer top-k library (libflashtopk.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/flashtopk.h.  torch supplies
device memory and the stream.  The functions below carry the C entry points'
names; ``select`` mirrors the FlashTopK README "Usage" signature
``select(q, kv, weights, ks, ke, kv_scales=None, topk=2048, ...)``.

There is no fallback: if the HIP library is missing or no GPU is present the
calls raise.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashtopk.so")

FLASHTOPK_FP8_E4M3 = 0
FLASHTOPK_BF16 = 1
HEADS = 32
DIM = 128
MAX_TOPK = 4096
FLASHTOPK_SCORES_F32 = 0
FLASHTOPK_SCORES_BF16 = 1
FLASHTOPK_OUT_INDEX_ORDER = 1
FLASHTOPK_OUT_INT64 = 2
FLASHTOPK_INVALID_WINDOW = 1
FLASHTOPK_INVALID_Q = 2
FLASHTOPK_INVALID_KV = 4
FLASHTOPK_INVALID_WEIGHT = 8
FLASHTOPK_INVALID_SCALE = 16
FLASHTOPK_INVALID_PAGE = 32

PATH_AUTO, PATH_SCAN, PATH_PRUNE, PATH_RECOVER, PATH_FUSED = 0, 1, 2, 3, 4

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dtype", 3: "out of device memory",
          4: "HIP runtime error", 5: "call too large for the fixed scratch array"}
FLASHTOPK_ERR_WORKSPACE_LIMIT = 5
NOALLOC_SCRATCH_BYTES = 128 << 20


class FlashTopKError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status} ({STATUS.get(status, 'unknown')})")


class Options(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int),
        ("cand_capacity", ctypes.c_int),
        ("sample_rank_scale", ctypes.c_float),
        ("sample_target", ctypes.c_int),
        ("recover_budget_bytes", ctypes.c_int64),
        ("profile", ctypes.c_int),
        ("out_flags", ctypes.c_int),
        ("heads", ctypes.c_int),
        ("validate", ctypes.c_int),
    ]


class Info(ctypes.Structure):
    _fields_ = [
        ("status", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("rows_empty", ctypes.c_int64),
        ("rows_take_all", ctypes.c_int64),
        ("rows_sampled", ctypes.c_int64),
        ("rows_underflow", ctypes.c_int64),
        ("rows_overflow", ctypes.c_int64),
        ("rows_recovered", ctypes.c_int64),
        ("max_candidates", ctypes.c_int64),
        ("window_keys", ctypes.c_int64),
        ("pruned_keys", ctypes.c_int64),
        ("cand_capacity", ctypes.c_int32),
        ("sample_target", ctypes.c_int32),
        ("ms_sample", ctypes.c_float),
        ("ms_tau", ctypes.c_float),
        ("ms_filter", ctypes.c_float),
        ("ms_triage", ctypes.c_float),
        ("ms_select", ctypes.c_float),
        ("ms_recover", ctypes.c_float),
        ("invalid", ctypes.c_int32),
        ("candidates", ctypes.c_int64),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


# Every symbol include/flashtopk.h declares.
EXPORTS = ("flashtopk_select", "flashtopk_select_ex", "flashtopk_select_paged", "flashtopk_select_noalloc",
           "flashtopk_topk_rows", "flashtopk_reserve", "flashtopk_get_last_info", "flashtopk_get_last_recovered",
           "flashtopk_release", "flashtopk_status_string", "flashtopk_version", "flashtopk_probe_mfma")

_lib = None


def load_library():
    """Loads libflashtopk.so (no GPU needed to load it)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
    # torch first: the library then binds to the HIP runtime torch has loaded,
    # so the process holds one runtime whichever call comes first.
    _torch()
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sel = [P, P, P, P, P, P, I64, I64, I, I, P, P, P]
    lib.flashtopk_select.argtypes = sel
    lib.flashtopk_select.restype = I
    lib.flashtopk_select_ex.argtypes = sel + [ctypes.POINTER(Options)]
    lib.flashtopk_select_ex.restype = I
    lib.flashtopk_select_noalloc.argtypes = sel
    lib.flashtopk_select_noalloc.restype = I
    lib.flashtopk_select_paged.argtypes = [P, P, P, P, I, I64, P, P, P, I64, I64, I, I, P, P, P,
                                           ctypes.POINTER(Options)]
    lib.flashtopk_select_paged.restype = I
    lib.flashtopk_topk_rows.argtypes = [P, I, I64, I64, I64, P, I, P, P, P, I, P]
    lib.flashtopk_topk_rows.restype = I
    lib.flashtopk_reserve.argtypes = [I64, I64, I, I, P]
    lib.flashtopk_reserve.restype = I
    lib.flashtopk_get_last_info.argtypes = [P, ctypes.POINTER(Info)]
    lib.flashtopk_get_last_info.restype = I
    lib.flashtopk_get_last_recovered.argtypes = [P, P, I64, ctypes.POINTER(I64)]
    lib.flashtopk_get_last_recovered.restype = I
    lib.flashtopk_release.argtypes = []
    lib.flashtopk_release.restype = None
    lib.flashtopk_status_string.argtypes = [I]
    lib.flashtopk_status_string.restype = ctypes.c_char_p
    lib.flashtopk_version.argtypes = []
    lib.flashtopk_version.restype = I
    lib.flashtopk_probe_mfma.argtypes = [I, I, P, ctypes.POINTER(ctypes.c_double)]
    lib.flashtopk_probe_mfma.restype = I
    _lib = lib
    return lib


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FLASHTOPK_FP8_E4M3
    if t.dtype in (torch.bfloat16, torch.int16):
        return FLASHTOPK_BF16
    raise TypeError(f"q/kv must be float8_e4m3fn or bfloat16 (or their uint8/int16 codes), got {t.dtype}")


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name, t, dtypes=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def flashtopk_select_ex(q, kv, kv_scales, weights, ks, ke, topk, out_idx, out_val=None, stream=None,
                        options: Options | None = None) -> None:
    """Fills out_idx [T, topk] int32 (and out_val [T, topk] float32 if given)."""
    torch = _torch()
    lib = load_library()
    T, S = q.shape[0], kv.shape[0]
    code = _dtype_code(q)
    if _dtype_code(kv) != code:
        raise TypeError("q and kv must have the same dtype")
    heads = q.shape[1] if q.dim() == 3 else 0
    if heads not in (32, 64) or q.shape[2] != DIM or tuple(kv.shape[1:]) != (DIM,):
        raise ValueError("q must be [T, 32 or 64, 128] and kv [S, 128]")
    _check_dev("q", q)
    _check_dev("kv", kv)
    _check_dev("kv_scales", kv_scales, (torch.float32,), (S,))
    _check_dev("weights", weights, (torch.float32,), (T, heads))
    if heads != HEADS or (options is not None and options.heads not in (0, heads)):
        if options is not None and options.heads not in (0, heads):
            raise ValueError(f"options.heads {options.heads} does not match q's {heads} heads")
        options = Options() if options is None else Options.from_buffer_copy(options)
        options.heads = heads
    _check_dev("ks", ks, (torch.int32,), (T,))
    _check_dev("ke", ke, (torch.int32,), (T,))
    _check_dev("out_idx", out_idx, (torch.int32, torch.int64), (T, topk))
    _check_dev("out_val", out_val, (torch.float32,), (T, topk))
    flags = options.out_flags if options is not None else 0
    if (out_idx.dtype == torch.int64) != bool(flags & FLASHTOPK_OUT_INT64):
        raise TypeError("out_idx dtype and options.out_flags (FLASHTOPK_OUT_INT64) disagree")
    opt = ctypes.byref(options) if options is not None else None
    st = lib.flashtopk_select_ex(_ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(weights), _ptr(ks), _ptr(ke),
                                 T, S, code, int(topk), _ptr(out_idx), _ptr(out_val),
                                 ctypes.c_void_p(_stream_handle(stream)), opt)
    if st != 0:
        raise FlashTopKError(st, "flashtopk_select_ex")


def flashtopk_select_paged(q, kv_pages, scale_pages, block_table, num_kv, weights, ks, ke, topk, out_idx,
                           out_val=None, stream=None, options: Options | None = None) -> None:
    """flashtopk_select_ex over keys in a paged cache: kv_pages [num_pages,
    page_size, 128], scale_pages [num_pages, page_size] float32 or None,
    block_table [ceil(num_kv / page_size)] int32; num_kv logical keys."""
    torch = _torch()
    lib = load_library()
    T = q.shape[0]
    code = _dtype_code(q)
    if _dtype_code(kv_pages) != code:
        raise TypeError("q and kv_pages must have the same dtype")
    if kv_pages.dim() != 3 or kv_pages.shape[2] != DIM or tuple(q.shape[1:]) != (HEADS, DIM):
        raise ValueError("kv_pages must be [num_pages, page_size, 128] and q [T, 32, 128]")
    num_pages, page_size = kv_pages.shape[0], kv_pages.shape[1]
    nblk = (int(num_kv) + page_size - 1) // page_size
    _check_dev("q", q)
    _check_dev("kv_pages", kv_pages)
    _check_dev("scale_pages", scale_pages, (torch.float32,), (num_pages, page_size))
    _check_dev("block_table", block_table, (torch.int32,))
    if block_table.numel() < nblk:
        raise ValueError(f"block_table needs {nblk} entries")
    _check_dev("weights", weights, (torch.float32,), (T, HEADS))
    _check_dev("ks", ks, (torch.int32,), (T,))
    _check_dev("ke", ke, (torch.int32,), (T,))
    _check_dev("out_idx", out_idx, (torch.int32, torch.int64), (T, topk))
    _check_dev("out_val", out_val, (torch.float32,), (T, topk))
    flags = options.out_flags if options is not None else 0
    if (out_idx.dtype == torch.int64) != bool(flags & FLASHTOPK_OUT_INT64):
        raise TypeError("out_idx dtype and options.out_flags (FLASHTOPK_OUT_INT64) disagree")
    opt = ctypes.byref(options) if options is not None else None
    st = lib.flashtopk_select_paged(_ptr(q), _ptr(kv_pages), _ptr(scale_pages), _ptr(block_table), int(page_size),
                                    int(num_pages), _ptr(weights), _ptr(ks), _ptr(ke), T, int(num_kv), code,
                                    int(topk), _ptr(out_idx), _ptr(out_val), ctypes.c_void_p(_stream_handle(stream)),
                                    opt)
    if st != 0:
        raise FlashTopKError(st, "flashtopk_select_paged")


def flashtopk_select(q, kv, kv_scales, weights, ks, ke, topk, out_idx, out_val=None, stream=None) -> None:
    flashtopk_select_ex(q, kv, kv_scales, weights, ks, ke, topk, out_idx, out_val, stream, None)


def flashtopk_select_noalloc(q, kv, kv_scales, weights, ks, ke, topk, out_idx, out_val=None, stream=None) -> None:
    """flashtopk_select with no device allocation: its scratch is the library's
    fixed array (NOALLOC_SCRATCH_BYTES per GPU); a call that does not fit
    raises FlashTopKError with status FLASHTOPK_ERR_WORKSPACE_LIMIT."""
    torch = _torch()
    lib = load_library()
    T, S = q.shape[0], kv.shape[0]
    code = _dtype_code(q)
    if _dtype_code(kv) != code:
        raise TypeError("q and kv must have the same dtype")
    if tuple(q.shape[1:]) != (HEADS, DIM) or tuple(kv.shape[1:]) != (DIM,):
        raise ValueError("q must be [T, 32, 128] and kv [S, 128]")
    _check_dev("q", q)
    _check_dev("kv", kv)
    _check_dev("kv_scales", kv_scales, (torch.float32,), (S,))
    _check_dev("weights", weights, (torch.float32,), (T, HEADS))
    _check_dev("ks", ks, (torch.int32,), (T,))
    _check_dev("ke", ke, (torch.int32,), (T,))
    _check_dev("out_idx", out_idx, (torch.int32,), (T, topk))
    _check_dev("out_val", out_val, (torch.float32,), (T, topk))
    st = lib.flashtopk_select_noalloc(_ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(weights), _ptr(ks), _ptr(ke),
                                      T, S, code, int(topk), _ptr(out_idx), _ptr(out_val),
                                      ctypes.c_void_p(_stream_handle(stream)))
    if st != 0:
        raise FlashTopKError(st, "flashtopk_select_noalloc")


def flashtopk_topk_rows(x, topk, out_idx, out_val=None, ends=None, nan_flag=None, stream=None,
                        index_order=False) -> None:
    """Exact top-k of each row of x [rows, cols] (float32 or bfloat16; last
    dimension contiguous, row stride a multiple of 16 bytes).  Fills out_idx
    [rows, topk] int32 or int64 and out_val [rows, topk] float32 if given;
    ends [rows] int32 bounds each row; nan_flag (one int32) is set to 1 on a
    NaN; index_order lists each row's top k by ascending index."""
    torch = _torch()
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    if x.dtype == torch.float32:
        code = FLASHTOPK_SCORES_F32
    elif x.dtype == torch.bfloat16:
        code = FLASHTOPK_SCORES_BF16
    else:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    rows, cols = x.shape
    if cols > 1 and x.stride(1) != 1:
        raise ValueError("x's last dimension must be contiguous")
    _check_dev("ends", ends, (torch.int32,), (rows,))
    _check_dev("out_idx", out_idx, (torch.int32, torch.int64), (rows, topk))
    _check_dev("out_val", out_val, (torch.float32,), (rows, topk))
    _check_dev("nan_flag", nan_flag, (torch.int32,), (1,))
    flags = (FLASHTOPK_OUT_INDEX_ORDER if index_order else 0) | \
        (FLASHTOPK_OUT_INT64 if out_idx.dtype == torch.int64 else 0)
    st = lib.flashtopk_topk_rows(_ptr(x), code, rows, cols, x.stride(0), _ptr(ends), int(topk), _ptr(out_idx),
                                 _ptr(out_val), _ptr(nan_flag), flags, ctypes.c_void_p(_stream_handle(stream)))
    if st != 0:
        raise FlashTopKError(st, "flashtopk_topk_rows")


def topk_rows(x, topk, ends=None, return_values=True, sorted_index=False, indices_type=None, stream=None):
    """indices [rows, topk] (int32, or indices_type torch.int64) and values
    [rows, topk] float32 of the exact top-k of each row of x, by score or
    (sorted_index) by index; see flashtopk_topk_rows."""
    torch = _torch()
    rows = x.shape[0]
    idx = torch.empty((rows, topk), dtype=indices_type or torch.int32, device=x.device)
    val = torch.empty((rows, topk), dtype=torch.float32, device=x.device) if return_values else None
    flashtopk_topk_rows(x, topk, idx, val, ends, None, stream, index_order=sorted_index)
    return (idx, val) if return_values else idx


def flashtopk_reserve(max_q, max_kv, max_topk, dtype=FLASHTOPK_FP8_E4M3, stream=None) -> None:
    st = load_library().flashtopk_reserve(int(max_q), int(max_kv), int(max_topk), int(dtype),
                                          ctypes.c_void_p(_stream_handle(stream)))
    if st != 0:
        raise FlashTopKError(st, "flashtopk_reserve")


def flashtopk_get_last_info(stream=None) -> dict:
    info = Info()
    st = load_library().flashtopk_get_last_info(ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(info))
    if st != 0:
        raise FlashTopKError(st, "flashtopk_get_last_info")
    return info.as_dict()


def flashtopk_get_last_recovered(stream=None):
    """Row indices (sorted int32 numpy array) that the last call on the stream
    scored densely."""
    import numpy as np

    lib = load_library()
    h = ctypes.c_void_p(_stream_handle(stream))
    n = ctypes.c_int64(0)
    st = lib.flashtopk_get_last_recovered(h, None, 0, ctypes.byref(n))
    if st != 0:
        raise FlashTopKError(st, "flashtopk_get_last_recovered")
    out = np.zeros(n.value, dtype=np.int32)
    if n.value:
        st = lib.flashtopk_get_last_recovered(h, out.ctypes.data_as(ctypes.c_void_p), n.value, ctypes.byref(n))
        if st != 0:
            raise FlashTopKError(st, "flashtopk_get_last_recovered")
    return np.sort(out)


def flashtopk_release() -> None:
    load_library().flashtopk_release()


def flashtopk_status_string(status: int) -> str:
    return load_library().flashtopk_status_string(int(status)).decode()


def flashtopk_version() -> int:
    return int(load_library().flashtopk_version())


def flashtopk_probe_mfma(dtype: int, iters: int, stream=None) -> float:
    """Attainable TFLOP/s of the scan's MFMA instruction (FP8 16x16x128 or
    BF16 32x32x16) on the current device, from a register-only throughput
    kernel timed on `stream` (synchronises it)."""
    out = ctypes.c_double(0.0)
    st = load_library().flashtopk_probe_mfma(int(dtype), int(iters), ctypes.c_void_p(_stream_handle(stream)),
                                             ctypes.byref(out))
    if st != 0:
        raise FlashTopKError(st, "flashtopk_probe_mfma")
    return float(out.value)


def select(q, kv, weights, ks, ke, kv_scales=None, topk=2048, return_scores=False, options=None, stream=None,
           sorted_index=False, indices_type=None):
    """indices [T, topk] (int32, or indices_type torch.int64) and, with
    return_scores, scores [T, topk] float32; by score, or (sorted_index) by
    index."""
    torch = _torch()
    T = q.shape[0]
    o = Options() if options is None else Options.from_buffer_copy(options)
    if sorted_index:
        o.out_flags |= FLASHTOPK_OUT_INDEX_ORDER
    if indices_type == torch.int64:
        o.out_flags |= FLASHTOPK_OUT_INT64
    idx = torch.empty((T, topk), dtype=torch.int64 if o.out_flags & FLASHTOPK_OUT_INT64 else torch.int32,
                      device=q.device)
    val = torch.empty((T, topk), dtype=torch.float32, device=q.device) if return_scores else None
    flashtopk_select_ex(q, kv, kv_scales, weights, ks, ke, topk, idx, val, stream, o)
    return (idx, val) if return_scores else idx


def windows_from_cu_seqlens(cu_seqlens_q, cu_seqlens_k):
    """Causal windows of packed sequences (README "Usage"), bottom-right
    aligned: query i of a document with Lq queries and Lk keys sees keys
    [cu_k[j], cu_k[j] + Lk - Lq + i + 1).  Returns int32 (ks, ke)."""
    torch = _torch()
    cq = cu_seqlens_q.to(torch.int64)
    ck = cu_seqlens_k.to(torch.int64)
    lq = cq[1:] - cq[:-1]
    lk = ck[1:] - ck[:-1]
    T = int(cq[-1].item())
    doc = torch.repeat_interleave(torch.arange(lq.numel(), device=cq.device), lq)
    pos = torch.arange(T, device=cq.device) - cq[doc]
    ks = ck[doc]
    ke = torch.minimum(torch.maximum(ck[doc] + lk[doc] - lq[doc] + pos + 1, ks), ck[doc + 1])
    return ks.to(torch.int32), ke.to(torch.int32)
