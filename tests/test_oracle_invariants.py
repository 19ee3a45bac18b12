"""Invariants of the exact top-k that hold at any size (CPU only).

I1 count = min(topk, L); I2 indices unique and inside [ks, ke); I3 -1 only as
a tail; I4 strictly ordered by (value desc, index asc); I5 every returned
score >= every excluded score, and on equality every excluded index is larger
than every returned index with that score; I6 each value is the row's score
of its index; metamorphic: doubling every kv_scale doubles every value exactly
and keeps the indices; jointly permuting the heads of q and weights changes
nothing (exact data).
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle import numpy_ref

import checker


def _run(wl, **kw):
    return oracle.select(wl["q"], wl["kv"], wl["dtype"], wl["kv_scales"], wl["weights"],
                         wl["ks"], wl["ke"], wl["topk"], all_scores=True, **kw)


WLS = [
    lambda: workloads.gaussian(33, 700, 37, "fp8", 31),
    lambda: workloads.gaussian(20, 300, 64, "bf16", 32, weight_scale=0.2),
    lambda: workloads.integer(40, 500, 50, "fp8", 33),
    lambda: workloads.trained_shaped(25, 900, 40, "fp8", 34),
    lambda: workloads.integer(48, 48, 8, "bf16", 35, windows="packed", docs=(7, 20, 21)),
]


@pytest.mark.parametrize("make", WLS)
def test_invariants(make):
    wl = make()
    idx, val, sc, allsc = _run(wl)
    T = idx.shape[0]
    for t in range(T):
        ks, ke, k = int(wl["ks"][t]), int(wl["ke"][t]), wl["topk"]
        assert not checker.structure_failures(idx[t], val[t], ks, ke, k)        # I1-I4
        L = max(0, ke - ks)
        n = min(k, L)
        sel = idx[t, :n].astype(np.int64)
        assert np.array_equal(val[t, :n], allsc[t, sel].astype(np.float32) + np.float32(0))  # I6
        excluded = np.setdiff1d(np.arange(ks, ke), sel)
        if excluded.size and n:
            worst = allsc[t, sel].min()
            best_out = allsc[t, excluded].max()
            assert worst >= best_out                                              # I5
            if worst == best_out:
                tied_in = sel[allsc[t, sel] == worst]
                tied_out = excluded[allsc[t, excluded] == worst]
                assert tied_in.max() < tied_out.min()


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_scale_doubling_doubles_values(dtype):
    wl = workloads.gaussian(17, 400, 30, dtype, 41)
    idx, val, _, _ = _run(wl)
    wl2 = dict(wl, kv_scales=wl["kv_scales"] * np.float32(2))
    idx2, val2, _, _ = _run(wl2)
    assert np.array_equal(idx, idx2)
    fin = idx >= 0
    assert np.array_equal(val2[fin], val[fin] * np.float32(2))


def test_head_permutation_is_a_symmetry_on_exact_data():
    wl = workloads.integer(16, 300, 25, "fp8", 42)
    perm = np.random.default_rng(5).permutation(32)
    wl2 = dict(wl, q=np.ascontiguousarray(wl["q"][:, perm, :]),
               weights=np.ascontiguousarray(wl["weights"][:, perm]))
    a = _run(wl)
    b = _run(wl2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_integer_data_is_exact_in_binary32():
    """On the integer workloads every partial sum is a dyadic rational small
    enough for binary32, so rounding the binary64 score to binary32 is exact."""
    wl = workloads.integer(12, 256, 16, "fp8", 43)
    qd = numpy_ref.decode(wl["q"], "fp8")
    kd = numpy_ref.decode(wl["kv"], "fp8")
    x = np.einsum("thd,sd->ths", qd, kd)
    assert np.abs(x).max() < 2 ** 24
    I = numpy_ref.score_matrix(qd, kd, wl["weights"], wl["kv_scales"])
    assert np.array_equal(I.astype(np.float32).astype(np.float64), I)
    assert np.all(np.abs(I) * 8 < 2 ** 24)


def test_twin_agrees_on_small_random_inputs():
    for make in WLS:
        wl = make()
        if wl["q"].shape[0] * wl["kv"].shape[0] > 40000:
            continue
        idx, val, _, _ = _run(wl)
        i2, v2, _ = numpy_ref.select(wl["q"], wl["kv"], wl["dtype"], wl["kv_scales"],
                                     wl["weights"], wl["ks"], wl["ke"], wl["topk"])
        assert np.array_equal(idx, i2)
        assert np.array_equal(val.view(np.uint32), v2.view(np.uint32))


def test_row_subset_matches_full_run():
    wl = workloads.gaussian(30, 333, 20, "fp8", 44)
    idx, val, sc, allsc = _run(wl)
    rows = np.array([29, 0, 7, 7, 15])
    i2, v2, s2, a2 = _run(wl, rows=rows)
    assert np.array_equal(i2, idx[rows]) and np.array_equal(v2, val[rows])
    assert np.array_equal(np.nan_to_num(a2, nan=7.0), np.nan_to_num(allsc[rows], nan=7.0))


def test_empty_and_degenerate_windows():
    wl = workloads.gaussian(4, 64, 8, "bf16", 45)
    ks = np.array([0, 5, 63, 10], np.int32)
    ke = np.array([0, 5, 64, 11], np.int32)
    idx, val, _, _ = oracle.select(wl["q"], wl["kv"], "bf16", wl["kv_scales"], wl["weights"],
                                   ks, ke, 8)
    assert np.all(idx[0] == -1) and np.all(idx[1] == -1)
    assert idx[2, 0] == 63 and np.all(idx[2, 1:] == -1)
    assert idx[3, 0] == 10
