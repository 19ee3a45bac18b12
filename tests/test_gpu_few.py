"""Calls with at most four query rows (decode and a few speculative tokens),
which score with the heads-on-M kernel in every mode.

Integer data is compared with the oracle bit-exactly, Gaussian data within
the tolerance rule; forced paths (dense recovery of every row, a capacity
small enough to overflow, the prune option, which such calls ignore) must
return the default path's bits, since every mode of the call shares the
kernel's arithmetic.
"""
import numpy as np
import pytest

import workloads

from gpu_util import opts, parity, run_gpu, to_device

pytestmark = pytest.mark.gpu

SCAN, PRUNE, RECOVER = 1, 2, 3


def _say(*a):
    print(*a, flush=True)


def _same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def _windows(wl, kind, seed):
    T, S = wl["q"].shape[0], wl["kv"].shape[0]
    ks, ke = wl["ks"].copy(), wl["ke"].copy()
    rng = np.random.default_rng(seed)
    if kind == "ragged":
        for t in range(T):
            a, b = np.sort(rng.integers(0, S + 1, size=2))
            ks[t], ke[t] = a, b
        if T >= 3:
            ks[1], ke[1] = 100, 100              # empty
            ks[2], ke[2] = 5000, 5000 + 37        # shorter than topk
    return dict(wl, ks=ks.astype(np.int32), ke=ke.astype(np.int32))


CASES = [
    # (T, S, topk, dtype, windows)
    (1, 40000, 512, "fp8", "causal"),
    (2, 33333, 300, "fp8", "ragged"),
    (3, 50000, 2048, "bf16", "ragged"),
    (4, 65536, 1024, "bf16", "causal"),
    (4, 20001, 64, "fp8", "ragged"),
]


@pytest.mark.parametrize("case", CASES, ids=["_".join(map(str, c)) for c in CASES])
def test_few_rows_integer_exact(case):
    T, S, topk, dt, win = case
    _say("few integer", case)
    wl = _windows(workloads.integer(T, S, topk, dt, 970 + T + S), win, 971)
    d = to_device(wl)
    got = run_gpu(wl, d)
    rep = parity(wl, got[0], got[1], "exact")
    assert rep["ok"], rep
    # every forced path returns the same bits
    for o in (opts(path=RECOVER), opts(path=PRUNE), opts(path=SCAN, cand_capacity=topk)):
        assert _same(run_gpu(wl, d, options=o), got)


@pytest.mark.parametrize("T,dt", [(1, "bf16"), (3, "fp8")])
def test_few_rows_gaussian_tolerance_and_paths(T, dt):
    _say("few gaussian", T, dt)
    wl = workloads.gaussian(T, 131072, 2048, dt, 980 + T)
    d = to_device(wl)
    got = run_gpu(wl, d)
    rep = parity(wl, got[0], got[1], "tolerance")
    assert rep["ok"], rep
    assert _same(run_gpu(wl, d, options=opts(path=RECOVER)), got)
    assert _same(run_gpu(wl, d, options=opts(sample_rank_scale=0.02)), got)  # threshold too high: recovery
    assert _same(run_gpu(wl, d), got)  # repeatable


def test_few_rows_trained_shaped_decode():
    wl = workloads.trained_shaped(2, 131072, 2048, "fp8", 990)
    got = run_gpu(wl)
    rep = parity(wl, got[0], got[1], "tolerance")
    assert rep["ok"], rep
