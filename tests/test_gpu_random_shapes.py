"""Seeded random shapes against the oracle, bit-exact (MI355X only).

Each case draws the row count, key count, topk, dtype, head count and a
window per row at random (empty, one-key, short, take-all, sampled, windows
that start anywhere and end anywhere, rows out of order), on integer-valued
inputs where fp32 accumulation is exact, and runs it on the default path and
forced through the fused path (sample, threshold, scan, selection,
recovery), both checked against the oracle on every row.
"""
import numpy as np
import pytest

import sparse_attention_indexer_fp8_amd as ftk
import workloads

from gpu_util import opts, parity, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 32


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = "fp8" if seed % 2 == 0 else "bf16"
    heads = 64 if seed % 5 == 3 else 32
    T = int(rng.integers(1, 300))
    S = int(rng.integers(1, 40000))
    topk = int(rng.choice([1, 7, 64, 100, 512, 1000, 2048, 4096]))
    wl = workloads.integer(T, S, topk, dtype, 500 + seed, windows="full", heads=heads)
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
    wl["name"] = f"random_{seed}_{dtype}_h{heads}_{T}x{S}_k{topk}"
    return wl, heads


@pytest.mark.parametrize("seed", range(N_CASES))
@pytest.mark.parametrize("path", [ftk.PATH_AUTO, ftk.PATH_FUSED], ids=["auto", "fused"])
def test_random_shape_bit_exact(seed, path):
    wl, heads = _case(seed)
    print("case", wl["name"], "path", path, flush=True)
    idx, val = run_gpu(wl, options=opts(path=path, heads=heads))
    rep = parity(wl, idx, val, "exact")
    assert rep["ok"], rep
