"""Calls of few query rows (decode, a few speculative tokens) and the
independence of a row's results from the rest of the call.

By default such calls take the dense path: every row's window scores are
materialised and the row top-k kernels select from them, each row split
over several workgroups.  Integer data is compared with the oracle
bit-exactly, Gaussian data within the tolerance rule.  The fused path
forced on the same call (sampled threshold, filter, selection, recovery of
misjudged rows) and its forced variants must return the dense path's bits:
every path scores a (row, key) pair with the same instructions.  For the
same reason a row's bits must not depend on which other rows share its call.
"""
import numpy as np
import pytest

import workloads

from gpu_util import opts, parity, run_gpu, to_device

pytestmark = pytest.mark.gpu

SCAN, PRUNE, RECOVER, FUSED = 1, 2, 3, 4


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
    (16, 30000, 4096, "fp8", "ragged"),
    (61, 9000, 100, "bf16", "ragged"),
]

FORCED = [
    ("recover", dict(path=RECOVER)),
    ("fused", dict(path=FUSED)),
    ("prune", dict(path=PRUNE)),
    ("scan_cap_topk", dict(path=SCAN, cand_capacity=4096)),
    ("fused_underflow", dict(path=FUSED, sample_rank_scale=0.02)),
    ("dense_small_budget", dict(path=RECOVER, recover_budget_bytes=4 << 20)),
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
    for label, kw in FORCED:
        kw = dict(kw)
        if "cand_capacity" in kw:
            kw["cand_capacity"] = topk
        assert _same(run_gpu(wl, d, options=opts(**kw)), got), label


@pytest.mark.parametrize("T,dt", [(1, "bf16"), (3, "fp8"), (64, "fp8")])
def test_few_rows_gaussian_tolerance_and_paths(T, dt):
    _say("few gaussian", T, dt)
    wl = workloads.gaussian(T, 131072, 2048, dt, 980 + T)
    d = to_device(wl)
    got = run_gpu(wl, d)
    rep = parity(wl, got[0], got[1], "tolerance")
    assert rep["ok"], rep
    for label, kw in FORCED:
        if "cand_capacity" in kw:
            continue
        assert _same(run_gpu(wl, d, options=opts(**kw)), got), label
    assert _same(run_gpu(wl, d), got)  # repeatable


def test_few_rows_trained_shaped_decode():
    wl = workloads.trained_shaped(2, 131072, 2048, "fp8", 990)
    got = run_gpu(wl)
    rep = parity(wl, got[0], got[1], "tolerance")
    assert rep["ok"], rep


def _rows_of(wl, rows):
    """The workload restricted to the given rows (same keys)."""
    out = dict(wl)
    for k in ("q", "weights", "ks", "ke"):
        out[k] = np.ascontiguousarray(wl[k][rows])
    return out


@pytest.mark.parametrize("dt,maker", [("fp8", "gaussian"), ("bf16", "gaussian"), ("fp8", "trained")])
def test_row_bits_do_not_depend_on_the_call(dt, maker):
    # The same rows scored in calls of 1, 3, 4, 5, 17 and 300 rows, on the dense and
    # the fused path, give the same bits (Gaussian data: the scores are not
    # exact, so this checks that every path runs the same arithmetic).
    _say("batch invariance", dt, maker)
    T, S, topk = 300, 20000, 256
    if maker == "gaussian":
        wl = _windows(workloads.gaussian(T, S, topk, dt, 995), "ragged", 996)
    else:
        wl = _windows(workloads.trained_shaped(T, S, topk, dt, 997), "ragged", 998)
    big = run_gpu(wl, options=opts(path=FUSED))
    big_dense = run_gpu(wl, options=opts(path=RECOVER))
    assert _same(big, big_dense)
    for rows in ([123], [2, 150, 299], [10, 11, 12, 13], [0, 7, 150, 298, 299], list(range(40, 57))):
        sub = _rows_of(wl, np.asarray(rows))
        for path in (0, FUSED, RECOVER):
            got = run_gpu(sub, options=opts(path=path))
            assert np.array_equal(got[0], big[0][rows]), (rows, path)
            assert np.array_equal(got[1].view(np.uint32), big[1][rows].view(np.uint32)), (rows, path)
