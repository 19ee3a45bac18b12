"""Seeded synthetic inputs for the indexer top-k path.

This module only draws and quantizes inputs; it holds none of the method's
arithmetic.  Both the oracle-side tests and the HIP-side tests / benchmark use
it, so the two sides always see byte-identical operands.

Shapes and value distributions follow the FlashTopK README "Quick start"
example (a causal chunk of 4096 queries over 128K FP8 keys, 32 heads x 128,
per-key fp32 scales, per-head fp32 weights, topk 2048) and the packed-sequence
window helper of its "Usage" section.  Every array is produced on the host with
``numpy.random.default_rng(seed)`` and quantized on the CPU with torch's
round-to-nearest-even casts to ``float8_e4m3fn`` / ``bfloat16``.

A workload is a plain dict:
    q        uint8 [T,32,128] (FP8 E4M3FN codes) or uint16 (BF16 codes)
    kv       uint8 [S,128] / uint16 [S,128]
    dtype    "fp8" | "bf16"
    kv_scales float32 [S] or None (all ones)
    weights  float32 [T,32]
    ks, ke   int32 [T]
    topk     int
    name     str
"""
from __future__ import annotations

import hashlib

import numpy as np

HEADS = 32
DIM = 128


def _quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "fp8":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def causal_windows(T: int, S: int):
    """Query i of a chunk of the last T tokens sees keys [0, S - T + i + 1)
    (README "Quick start": causal prefill chunk)."""
    ke = np.arange(S - T + 1, S + 1, dtype=np.int64)
    ks = np.zeros(T, dtype=np.int64)
    return ks.astype(np.int32), ke.astype(np.int32)


def packed_windows(cu_seqlens_q, cu_seqlens_k):
    """Causal windows of packed sequences (README "Usage": windows_from_cu_seqlens).

    Document j holds queries [cu_q[j], cu_q[j+1]) and keys [cu_k[j], cu_k[j+1]).
    Reading: bottom-right aligned, as in the causal-chunk example, so query i of
    a document with Lq queries and Lk keys sees keys
    [cu_k[j], cu_k[j] + Lk - Lq + i + 1).
    """
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    T = int(cu_q[-1])
    ks = np.zeros(T, dtype=np.int64)
    ke = np.zeros(T, dtype=np.int64)
    for j in range(len(cu_q) - 1):
        lq = cu_q[j + 1] - cu_q[j]
        lk = cu_k[j + 1] - cu_k[j]
        i = np.arange(lq)
        ks[cu_q[j]: cu_q[j + 1]] = cu_k[j]
        ke[cu_q[j]: cu_q[j + 1]] = np.clip(cu_k[j] + lk - lq + i + 1, cu_k[j], cu_k[j + 1])
    return ks.astype(np.int32), ke.astype(np.int32)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def gaussian(T, S, topk, dtype, seed, *, weight_scale=1.0, scales="uniform01",
             windows="causal", docs=None, name=None, heads=HEADS):
    """q, kv ~ N(0,1); weights ~ N(0,1) * weight_scale; kv_scales per ``scales``.

    Draw order: q, kv, weights, kv_scales."""
    rng = np.random.default_rng(seed)
    q = _quantize(_normal(rng, (T, heads, DIM)), dtype)
    kv = _quantize(_normal(rng, (S, DIM)), dtype)
    w = (_normal(rng, (T, heads)) * np.float32(weight_scale)).astype(np.float32)
    if scales == "ones":
        sc = None
    elif scales == "uniform01":
        sc = rng.random(S, dtype=np.float32)
    else:
        raise ValueError(scales)
    ks, ke = _windows(T, S, windows, docs)
    return dict(q=q, kv=kv, dtype=dtype, kv_scales=sc, weights=w, ks=ks, ke=ke, topk=int(topk),
                name=name or f"gaussian_{dtype}_{T}x{S}_k{topk}")


def integer(T, S, topk, dtype, seed, *, windows="causal", docs=None, name=None, heads=HEADS):
    """Tie-heavy exact data: q, kv integers uniform in [-4, 4]; weights uniform in
    {+-1/4, +-1/2, +-1}; kv_scales uniform in {1/2, 1, 2}.  Every partial sum of
    the score is a multiple of 1/8 below 2^18, so binary32 arithmetic is exact.

    Draw order: q, kv, weights, kv_scales."""
    rng = np.random.default_rng(seed)
    q = _quantize(rng.integers(-4, 5, size=(T, heads, DIM)).astype(np.float32), dtype)
    kv = _quantize(rng.integers(-4, 5, size=(S, DIM)).astype(np.float32), dtype)
    wv = np.array([-1.0, -0.5, -0.25, 0.25, 0.5, 1.0], dtype=np.float32)
    w = wv[rng.integers(0, 6, size=(T, heads))]
    sv = np.array([0.5, 1.0, 2.0], dtype=np.float32)
    sc = sv[rng.integers(0, 3, size=S)]
    ks, ke = _windows(T, S, windows, docs)
    return dict(q=q, kv=kv, dtype=dtype, kv_scales=sc, weights=w, ks=ks, ke=ke, topk=int(topk),
                name=name or f"integer_{dtype}_{T}x{S}_k{topk}")


def trained_shaped(T, S, topk, dtype, seed, *, heavy_frac=0.03, windows="causal", docs=None,
                   name=None, heads=HEADS):
    """Heavy-tailed rows, shaped like a trained indexer.

    u = normalize(N(0, I_128)); per head c_h ~ U(0.5, 1.5) (shared by all
    queries); q[t,h] = c_h u + 0.5 N(0, I); each key is heavy with probability
    heavy_frac, g ~ N(4, 1) if heavy else N(0, 1); kv[s] = g_s u + 0.5 N(0, I);
    kv_scales ~ U(0.5, 1); weights ~ |N(0, 1)|.

    Draw order: u, c, heavy, g, q noise, kv noise, weights, kv_scales."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(DIM)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    c = rng.uniform(0.5, 1.5, size=heads).astype(np.float32)
    heavy = rng.random(S) < heavy_frac
    g = np.where(heavy, rng.normal(4.0, 1.0, size=S), rng.normal(0.0, 1.0, size=S)).astype(np.float32)
    qf = c[None, :, None] * u[None, None, :] + np.float32(0.5) * _normal(rng, (T, heads, DIM))
    q = _quantize(qf, dtype)
    del qf
    kf = g[:, None] * u[None, :] + np.float32(0.5) * _normal(rng, (S, DIM))
    kv = _quantize(kf, dtype)
    del kf
    w = np.abs(_normal(rng, (T, heads))).astype(np.float32)
    sc = rng.uniform(0.5, 1.0, size=S).astype(np.float32)
    ks, ke = _windows(T, S, windows, docs)
    return dict(q=q, kv=kv, dtype=dtype, kv_scales=sc, weights=w, ks=ks, ke=ke, topk=int(topk),
                name=name or f"trained_{dtype}_{T}x{S}_k{topk}")


def blocky(T, S, topk, dtype, seed, *, hot_frac=0.1, exact=False, windows="causal", docs=None, name=None):
    """Keys with block locality, for the score-bound pruning path.

    Keys come in aligned blocks of 64; a block is hot with probability
    hot_frac.  Hot blocks hold independent keys; a quiet block's keys are one
    per-block centroid plus small noise, so its per-dimension key range is
    narrow and its scores are low.

    exact=False: q ~ N(0,1); hot keys ~ N(0,1); quiet keys = 0.1 N(0,1)
    (centroid) + 0.01 N(0,1) (per key); weights ~ |N(0,1)|; kv_scales ~ U(0.5, 1).
    exact=True (integer-valued, exact in binary32): q, hot keys ~ U{-4..4};
    a quiet block's centroid is +-1 on 2 random dimensions and 0 elsewhere,
    and each quiet key adds, on each dimension with probability 1/512, a
    step of +-1; weights ~ U{1/4, 1/2, 1}; kv_scales ~ U{1/2, 1, 2}.

    Draw order: q, hot flags, hot keys, centroids, noise, weights, kv_scales."""
    rng = np.random.default_rng(seed)
    nb = (S + 63) // 64
    if exact:
        qf = rng.integers(-4, 5, size=(T, HEADS, DIM)).astype(np.float32)
    else:
        qf = _normal(rng, (T, HEADS, DIM))
    q = _quantize(qf, dtype)
    del qf
    hot = np.repeat(rng.random(nb) < hot_frac, 64)[:S]
    if exact:
        hk = rng.integers(-4, 5, size=(S, DIM)).astype(np.float32)
        sup = np.argsort(rng.random((nb, DIM)), axis=1)[:, :2]
        c = np.zeros((nb, DIM), np.float32)
        np.put_along_axis(c, sup, rng.choice(np.array([-1.0, 1.0], np.float32), size=(nb, 2)), axis=1)
        cen = np.repeat(c, 64, axis=0)[:S]
        step = rng.integers(-1, 2, size=(S, DIM)) * (rng.random((S, DIM)) < 1.0 / 512)
        quiet = cen + step.astype(np.float32)
    else:
        hk = _normal(rng, (S, DIM))
        cen = np.repeat(np.float32(0.1) * _normal(rng, (nb, DIM)), 64, axis=0)[:S]
        quiet = cen + np.float32(0.01) * _normal(rng, (S, DIM))
    kv = _quantize(np.where(hot[:, None], hk, quiet), dtype)
    del hk, cen, quiet
    if exact:
        wv = np.array([0.25, 0.5, 1.0], dtype=np.float32)
        w = wv[rng.integers(0, 3, size=(T, HEADS))]
        sv = np.array([0.5, 1.0, 2.0], dtype=np.float32)
        sc = sv[rng.integers(0, 3, size=S)]
    else:
        w = np.abs(_normal(rng, (T, HEADS))).astype(np.float32)
        sc = rng.uniform(0.5, 1.0, size=S).astype(np.float32)
    ks, ke = _windows(T, S, windows, docs)
    kind = "int" if exact else "gauss"
    return dict(q=q, kv=kv, dtype=dtype, kv_scales=sc, weights=w, ks=ks, ke=ke, topk=int(topk),
                name=name or f"blocky_{kind}_{dtype}_{T}x{S}_k{topk}")


def _windows(T, S, windows, docs):
    if windows == "causal":
        return causal_windows(T, S)
    if windows == "packed":
        cu = np.concatenate([[0], np.cumsum(np.asarray(docs, dtype=np.int64))])
        if cu[-1] != T or T != S:
            raise ValueError("packed windows need T == S == sum(docs)")
        return packed_windows(cu, cu)
    if windows == "full":
        return np.zeros(T, np.int32), np.full(T, S, np.int32)
    raise ValueError(windows)


# The five named workloads and their exact-arithmetic twins.
PACKED_DOCS = (8192, 16384, 24576, 16384)


def config(n: int, *, integer_twin: bool = False):
    """Named workloads 1..9 (integer twins for 3..5, 7, 8 with integer_twin=True)."""
    if integer_twin:
        if n == 3:
            return integer(4096, 131072, 4096, "fp8", 13, name="untrained_int_fp8_4096x131072_k4096")
        if n == 4:
            return integer(4096, 131072, 2048, "fp8", 14, name="trained_int_fp8_4096x131072_k2048")
        if n == 5:
            return integer(65536, 65536, 512, "bf16", 15, windows="packed", docs=PACKED_DOCS,
                           name="packed_int_bf16_65536_k512")
        if n == 7:
            return integer(1, 131072, 2048, "fp8", 17, name="decode_int_fp8_1x131072_k2048")
        if n == 8:
            return integer(64, 131072, 2048, "fp8", 18, name="decode_int_fp8_64x131072_k2048")
        raise ValueError(n)
    if n == 1:
        return gaussian(64, 2048, 64, "bf16", 1, weight_scale=32 ** -0.5, scales="ones",
                        name="smallest_bf16_64x2048_k64")
    if n == 2:
        return integer(256, 8192, 512, "fp8", 2, name="tieheavy_fp8_256x8192_k512")
    if n == 3:
        return gaussian(4096, 131072, 4096, "fp8", 3, name="untrained_fp8_4096x131072_k4096")
    if n == 4:
        return trained_shaped(4096, 131072, 2048, "fp8", 4, name="trained_fp8_4096x131072_k2048")
    if n == 5:
        return gaussian(65536, 65536, 512, "bf16", 5, weight_scale=32 ** -0.5, scales="ones",
                        windows="packed", docs=PACKED_DOCS, name="packed_bf16_65536_k512")
    if n == 6:
        # not one of the pages' workloads: keys with block locality, where
        # score-bound pruning has something to skip
        return blocky(4096, 131072, 2048, "fp8", 6, name="blocky_fp8_4096x131072_k2048")
    if n == 7:
        # decode: one query row over the whole 128K-key context
        return trained_shaped(1, 131072, 2048, "fp8", 7, name="decode_fp8_1x131072_k2048")
    if n == 8:
        # decode with a small batch / speculative tokens: 64 query rows
        return trained_shaped(64, 131072, 2048, "fp8", 8, name="decode_fp8_64x131072_k2048")
    if n == 9:
        # the headline chunk for a 64-head indexer (DeepSeek-V3.2's head count)
        return trained_shaped(4096, 131072, 2048, "fp8", 9, heads=64, name="trained_h64_fp8_4096x131072_k2048")
    raise ValueError(n)


def digest(wl) -> str:
    """SHA-256 over every operand byte, in a fixed order."""
    h = hashlib.sha256()
    for k in ("q", "kv", "kv_scales", "weights", "ks", "ke"):
        a = wl[k]
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    h.update(str(wl["topk"]).encode())
    h.update(wl["dtype"].encode())
    return h.hexdigest()


def window_sum(wl) -> int:
    return int(np.maximum(wl["ke"].astype(np.int64) - wl["ks"].astype(np.int64), 0).sum())


# ---------------------------------------------------------------------------
# Materialized score rows for the standalone row top-k (DeepSelect README,
# "Supported Cases": BF16 rows of any batch size and vocabulary for the
# indexer scenario, float32 rows of about 128K entries for sampling, topk up
# to 4096 and mostly 512; "Variable-length rows": a per-row end).

ROW_KINDS = ("normal", "ties", "skewed", "special")


def _row_values(rng, rows, cols, kind):
    if kind == "normal":
        return rng.standard_normal((rows, cols), dtype=np.float32)
    if kind == "ties":
        # few distinct values: whole binades of equal entries
        return rng.integers(-4, 5, size=(rows, cols)).astype(np.float32)
    if kind == "skewed":
        # the shape of indexer scores: weighted sums of rectified products,
        # with many exact zeros and a long right tail
        z = rng.standard_normal((4, rows, cols), dtype=np.float32)
        w = np.array([1.0, 0.5, 0.25, -0.125], np.float32)[:, None, None]
        return (w * np.maximum(z, 0.0)).sum(axis=0).astype(np.float32)
    if kind == "special":
        x = rng.standard_normal((rows, cols), dtype=np.float32)
        u = rng.random((rows, cols))
        x[u < 0.01] = 0.0
        x[(u >= 0.01) & (u < 0.02)] = -0.0
        x[(u >= 0.02) & (u < 0.0202)] = np.inf
        x[(u >= 0.0202) & (u < 0.0204)] = -np.inf
        return x
    raise ValueError(kind)


def score_rows(rows, cols, dtype, seed, *, kind="normal", topk=512, ends=None, stride=None, name=None):
    """Score rows on the host.  dtype "f32" | "bf16"; ends None, an int32
    array, or "ragged" (uniform in [0, cols + 16], clamped by the callee) or
    "causal" (row r of the last `rows` positions of a sequence of `cols`
    tokens keeps cols - rows + r + 1 entries).  stride >= cols pads each row
    (padding filled with a large value that must never be selected).
    Returns dict(x, dtype, ends, topk, cols, name); x is float32 or BF16
    codes (uint16) [rows, stride]."""
    rng = np.random.default_rng(seed)
    v = _row_values(rng, rows, cols, kind)
    if isinstance(ends, str):
        if ends == "ragged":
            ends = rng.integers(0, cols + 17, size=rows).astype(np.int32)
        elif ends == "causal":
            ends = (cols - rows + 1 + np.arange(rows)).clip(0, cols).astype(np.int32)
        else:
            raise ValueError(ends)
    stride = cols if stride is None else stride
    if stride > cols:
        v = np.concatenate([v, np.full((rows, stride - cols), 1e30, np.float32)], axis=1)
    x = v if dtype == "f32" else _quantize(v, "bf16")
    return dict(x=x, dtype=dtype, ends=ends, topk=topk, cols=cols,
                name=name or f"rows_{kind}_{dtype}_{rows}x{cols}_k{topk}")


def score_rows_device(rows, cols, dtype, seed, *, kind="normal", dev="cuda:0"):
    """Large score rows drawn on the device with torch's seeded generator
    (the host generator is too slow at gigabyte sizes): "normal" or "skewed"
    values, returned as a float32 / bfloat16 device tensor [rows, cols]."""
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = torch.empty((rows, cols), dtype=tdt, device=dev)
    step = max(1, (1 << 26) // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        if kind == "normal":
            out[r0:r1] = torch.randn((r1 - r0, cols), generator=g, device=dev).to(tdt)
        elif kind == "skewed":
            z = torch.randn((4, r1 - r0, cols), generator=g, device=dev)
            w = torch.tensor([1.0, 0.5, 0.25, -0.125], device=dev)[:, None, None]
            out[r0:r1] = (w * z.clamp_min(0.0)).sum(0).to(tdt)
        else:
            raise ValueError(kind)
    return out


# Named score-row workloads of the standalone row top-k: (rows, cols, dtype,
# topk, value kind, ends).  The first three follow the DeepSelect README's
# "Supported Cases" / "Performance" shapes (BF16 indexer rows with topk 512 at
# a large and a small batch; float32 sampling rows of vocab 129280, topk 512);
# the last is the headline indexer chunk's score matrix (4096 causal rows of
# a 128K context, topk 2048) for comparison with the fused path.
ROW_CONFIGS = {
    "indexer_bf16_4096x131072_k512": (4096, 131072, "bf16", 512, "normal", None),
    "indexer_bf16_64x131072_k512": (64, 131072, "bf16", 512, "normal", None),
    "sampling_f32_1024x129280_k512": (1024, 129280, "f32", 512, "normal", None),
    "chunk_bf16_causal_4096x131072_k2048": (4096, 131072, "bf16", 2048, "skewed", "causal"),
}
