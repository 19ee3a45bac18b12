"""Seeded random shapes against the oracle, bit-exact (MI355X only).

Each case draws the row count, key count, topk, dtype, head count and a
window per row at random (empty, one-key, short, take-all, sampled, windows
that start anywhere and end anywhere, rows out of order), on integer-valued
inputs where fp32 accumulation is exact, and runs it on the default path and
forced through the fused path (sample, threshold, scan, selection,
recovery), both checked against the oracle on every row; the same shapes on
Gaussian data are checked with the tolerance rule, on FP8 floored at the
matrix cores' dot-product error.
"""
import numpy as np
import pytest

import sparse_attention_indexer_fp8_amd as ftk
import workloads

from gpu_util import fp8_dot_floor, opts, parity, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 32


def _case(seed, data="integer"):
    rng = np.random.default_rng(9000 + seed)
    dtype = "fp8" if seed % 2 == 0 else "bf16"
    heads = 64 if seed % 5 == 3 else 32
    T = int(rng.integers(1, 300))
    S = int(rng.integers(1, 40000))
    topk = int(rng.choice([1, 7, 64, 100, 512, 1000, 2048, 4096]))
    if data == "integer":
        wl = workloads.integer(T, S, topk, dtype, 500 + seed, windows="full", heads=heads)
    else:
        wl = workloads.gaussian(T, S, topk, dtype, 600 + seed, windows="full", heads=heads,
                                weight_scale=heads ** -0.5)
    kind = rng.integers(0, 6, size=T)
    lo = rng.integers(0, S + 1, size=T)
    ln = np.where(kind == 0, 0,                                   # empty
         np.where(kind == 1, 1,                                   # one key
         np.where(kind == 2, rng.integers(1, max(2, topk + 1), size=T),   # at most topk
                  rng.integers(0, S + 1, size=T))))               # anything
    hi = np.minimum(lo + ln, S)
    full = kind == 5
    lo[full], hi[full] = 0, S                                     # whole key set
    wl["ks"] = lo.astype(np.int32)
    wl["ke"] = hi.astype(np.int32)
    wl["name"] = f"random_{data}_{seed}_{dtype}_h{heads}_{T}x{S}_k{topk}"
    return wl, heads


@pytest.mark.parametrize("seed", range(N_CASES))
@pytest.mark.parametrize("path", [ftk.PATH_AUTO, ftk.PATH_FUSED], ids=["auto", "fused"])
def test_random_shape_bit_exact(seed, path):
    wl, heads = _case(seed)
    print("case", wl["name"], "path", path, flush=True)
    idx, val = run_gpu(wl, options=opts(path=path, heads=heads))
    rep = parity(wl, idx, val, "exact")
    assert rep["ok"], rep


@pytest.mark.parametrize("seed", range(16))
@pytest.mark.parametrize("path", [ftk.PATH_AUTO, ftk.PATH_FUSED], ids=["auto", "fused"])
def test_random_shape_gaussian_within_tolerance(seed, path):
    """The same shapes on Gaussian data: the tolerance rule on every row.  On
    FP8 a row's tolerance does not go below the matrix cores' own dot-product
    error (rows of a few keys whose head terms cancel)."""
    wl, heads = _case(seed, data="gaussian")
    print("case", wl["name"], "path", path, flush=True)
    idx, val = run_gpu(wl, options=opts(path=path, heads=heads))
    floor = fp8_dot_floor(wl) if wl["dtype"] == "fp8" else None
    rep = parity(wl, idx, val, "tolerance", floor=floor)
    assert rep["ok"], rep


def test_fp8_short_windows_plain_form():
    """FP8 Gaussian rows with windows around the plain-form bound (4096 keys)
    and far below it, mixed in tiles with long rows: the tolerance rule on
    every row (floored at the matrix cores' dot-product error), and the same
    bits on every path and in every batch (the form is the row's own)."""
    rng = np.random.default_rng(4242)
    T, S, topk = 96, 50000, 512
    wl = workloads.gaussian(T, S, topk, "fp8", 4243, windows="full", weight_scale=32 ** -0.5)
    lens = np.array([1, 2, 3, 5, 17, 100, 511, 512, 4095, 4096, 4097, 5000, 30000, S])
    ln = lens[rng.integers(0, len(lens), size=T)]
    lo = rng.integers(0, S + 1, size=T)
    lo = np.minimum(lo, S - ln)
    wl["ks"] = lo.astype(np.int32)
    wl["ke"] = (lo + ln).astype(np.int32)
    wl["name"] = "fp8_short_windows"
    print("case", wl["name"], flush=True)
    base = run_gpu(wl, options=opts(path=ftk.PATH_AUTO))
    rep = parity(wl, base[0], base[1], "tolerance", floor=fp8_dot_floor(wl))
    assert rep["ok"], rep
    for path in (ftk.PATH_FUSED, ftk.PATH_RECOVER):
        idx, val = run_gpu(wl, options=opts(path=path))
        assert np.array_equal(idx, base[0]), path
        assert np.array_equal(val.view(np.uint32), base[1].view(np.uint32)), path
    for rows in ([0], [5, 50, 90], list(range(20, 37))):
        sub = dict(wl)
        for k in ("q", "weights", "ks", "ke"):
            sub[k] = np.ascontiguousarray(wl[k][rows])
        idx, val = run_gpu(sub)
        assert np.array_equal(idx, base[0][rows]), rows
        assert np.array_equal(val.view(np.uint32), base[1][rows].view(np.uint32)), rows
