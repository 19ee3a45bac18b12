"""Small-case numpy twin of the oracle (TEST INFRASTRUCTURE ONLY).

An independent restatement of the same definition for tiny inputs, written
without the C code: operand decode from the OCP E4M3FN / bfloat16 bit layouts
with numpy integer arithmetic, the indexer score in binary64 (FlashTopK
README, "Quick start", indexer-score equation), and selection with
``numpy.lexsort`` on (key index, -score), so an equal score at the k-th
place goes to the lower key index (tie rule of the FlashTopK README, "What
you can do").  Short windows pad with -1 /
-inf (DeepSelect README, "Variable-length rows").
"""
from __future__ import annotations

import numpy as np


def decode_e4m3fn(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def decode_bf16(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint16).astype(np.int64)
    sign = np.where(c & 0x8000, -1.0, 1.0)
    e = (c >> 7) & 0xFF
    m = c & 0x7F
    mag = np.where(e == 0, m * 2.0 ** -133, (1.0 + m / 128.0) * np.exp2(e.astype(np.float64) - 127.0))
    mag = np.where(e == 0xFF, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def decode(codes, dtype) -> np.ndarray:
    if dtype in ("fp8", 0):
        return decode_e4m3fn(codes)
    return decode_bf16(codes)


def score_matrix(qd: np.ndarray, kd: np.ndarray, weights, kv_scales) -> np.ndarray:
    """I[t, s] for decoded qd [T,32,128] and kd [S,128], binary64."""
    x = np.einsum("thd,sd->ths", qd, kd)                 # per-head dot products
    r = np.maximum(x, 0.0)                               # ReLU per head
    acc = np.einsum("th,ths->ts", np.asarray(weights, np.float64), r)  # weighted head sum
    sigma = np.ones(kd.shape[0]) if kv_scales is None else np.asarray(kv_scales, np.float64)
    return acc * sigma[None, :]


def select(q, kv, dtype, kv_scales, weights, ks, ke, topk):
    qd = decode(q, dtype)
    kd = decode(kv, dtype)
    I = score_matrix(qd, kd, weights, kv_scales)
    T = qd.shape[0]
    idx = np.full((T, topk), -1, dtype=np.int32)
    val = np.full((T, topk), -np.inf, dtype=np.float32)
    for t in range(T):
        s = np.arange(int(ks[t]), int(ke[t]))
        if s.size == 0:
            continue
        order = np.lexsort((s, -I[t, s]))               # score desc, then index asc
        take = s[order][:topk]
        idx[t, : take.size] = take
        v = I[t, take].astype(np.float32)
        v[v == 0] = 0.0                                  # -0 written as +0
        val[t, : take.size] = v
    return idx, val, I
