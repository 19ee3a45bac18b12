"""Seeded generators and the parity checker (CPU only).

The checker must accept the oracle's own output and reject planted mistakes
(a swapped index, a duplicate, an out-of-window index, wrong padding, a tie
broken the wrong way, a perturbed value)."""
import numpy as np
import pytest

import oracle
import workloads

import checker


def test_generators_are_seeded_and_stable():
    for make in (lambda: workloads.gaussian(8, 100, 4, "fp8", 1),
                 lambda: workloads.integer(8, 100, 4, "bf16", 2),
                 lambda: workloads.trained_shaped(8, 100, 4, "fp8", 3)):
        assert workloads.digest(make()) == workloads.digest(make())
    a = workloads.gaussian(8, 100, 4, "fp8", 1)
    b = workloads.gaussian(8, 100, 4, "fp8", 2)
    assert workloads.digest(a) != workloads.digest(b)


def test_causal_and_packed_windows():
    ks, ke = workloads.causal_windows(4, 10)
    assert ks.tolist() == [0, 0, 0, 0] and ke.tolist() == [7, 8, 9, 10]
    cu = [0, 3, 8]
    ks, ke = workloads.packed_windows(cu, cu)
    assert ks.tolist() == [0, 0, 0, 3, 3, 3, 3, 3]
    assert ke.tolist() == [1, 2, 3, 4, 5, 6, 7, 8]
    # unequal query / key lengths: bottom-right aligned
    ks, ke = workloads.packed_windows([0, 2], [0, 5])
    assert ks.tolist() == [0, 0] and ke.tolist() == [4, 5]


def test_named_workload_shapes_small():
    wl = workloads.config(1)
    assert wl["q"].shape == (64, 32, 128) and wl["q"].dtype == np.uint16
    assert wl["kv"].shape == (2048, 128) and wl["kv_scales"] is None
    assert wl["ke"][0] == 2048 - 64 + 1 and wl["ke"][-1] == 2048
    assert workloads.window_sum(wl) == 129056
    wl = workloads.config(2)
    assert wl["q"].dtype == np.uint8 and wl["topk"] == 512
    assert workloads.window_sum(wl) == 2064512
    assert set(np.unique(wl["kv_scales"]).tolist()) == {0.5, 1.0, 2.0}


def test_packed_config_window_sum():
    ks, ke = workloads._windows(65536, 65536, "packed", workloads.PACKED_DOCS)
    assert int((ke.astype(np.int64) - ks).sum()) == 604012544
    assert int(np.sum((ke - ks) < 512)) == 4 * 511


def _oracle(wl):
    return oracle.select(wl["q"], wl["kv"], wl["dtype"], wl["kv_scales"], wl["weights"],
                         wl["ks"], wl["ke"], wl["topk"], all_scores=True)


@pytest.fixture(scope="module")
def ref():
    wl = workloads.integer(24, 400, 30, "fp8", 51)
    return wl, _oracle(wl)


@pytest.fixture(scope="module")
def ref_random():
    wl = workloads.gaussian(24, 400, 30, "fp8", 52)
    return wl, _oracle(wl)


def _chk(wl, r, idx, val, mode):
    return checker.check(idx, val, wl["ks"], wl["ke"], wl["topk"], o_idx=r[0], o_val=r[1],
                         o_score=r[2], all_scores=r[3], mode=mode)


@pytest.mark.parametrize("mode", ["exact", "tolerance"])
def test_checker_accepts_oracle_output(ref, ref_random, mode):
    for wl, r in (ref, ref_random):
        rep = _chk(wl, r, r[0].copy(), r[1].copy(), mode)
        assert rep["ok"], rep
        assert rep["precision"] == 1.0 and rep["identical_rows"] == 1.0


def _mutations(wl, r):
    idx, val = r[0], r[1]
    t = 10
    k = wl["topk"]
    out = {}
    a, b = idx.copy(), val.copy()
    a[t, [0, 1]] = a[t, [1, 0]]
    b[t, [0, 1]] = b[t, [1, 0]]
    out["swapped"] = (a, b)
    a, b = idx.copy(), val.copy()
    a[t, 3] = a[t, 2]
    out["duplicate"] = (a, b)
    a, b = idx.copy(), val.copy()
    a[t, 5] = wl["ke"][t]
    out["outside"] = (a, b)
    a, b = idx.copy(), val.copy()
    short = int(np.argmin(wl["ke"] - wl["ks"]))
    a[short, -1] = 0
    out["padding"] = (a, b)
    a, b = idx.copy(), val.copy()
    # the best excluded key replaces the last selected one
    allsc = r[3][t]
    sel = set(idx[t].tolist())
    win = np.arange(wl["ks"][t], wl["ke"][t])
    excl = [s for s in win if s not in sel]
    s_out = max(excl, key=lambda s: (allsc[s], -s))
    a[t, k - 1] = s_out
    b[t, k - 1] = np.float32(allsc[s_out])
    out["boundary"] = (a, b)
    a, b = idx.copy(), val.copy()
    b[t, 4] = b[t, 4] + np.float32(abs(b[t, 4]) * 0.01 + 1)
    out["value"] = (a, b)
    return out


def test_checker_rejects_planted_mistakes_exact(ref):
    wl, r = ref
    for name, (a, b) in _mutations(wl, r).items():
        rep = _chk(wl, r, a, b, "exact")
        assert not rep["ok"], name


def test_checker_rejects_planted_mistakes_tolerance(ref_random):
    wl, r = ref_random
    for name, (a, b) in _mutations(wl, r).items():
        rep = _chk(wl, r, a, b, "tolerance")
        if name == "boundary":
            # replacing the k-th by the (k+1)-th is only an error if they are
            # further apart than the tolerance
            k = wl["topk"]
            t = 10
            gap = abs(r[2][t, k - 1] - r[3][t][a[t, k - 1]])
            tol = 1e-3 * np.nanmax(np.abs(r[3][t]))
            if gap <= tol:
                continue
        assert not rep["ok"], name


def test_checker_rejects_wrong_tie_break(ref):
    """Integer data has exact ties; break one the wrong way."""
    wl, r = ref
    idx, val, sc = r[0], r[1], r[2]
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1] - 1):
            if idx[t, j + 1] >= 0 and val[t, j] == val[t, j + 1]:
                a = idx.copy()
                a[t, [j, j + 1]] = a[t, [j + 1, j]]
                rep = _chk(wl, r, a, val.copy(), "exact")
                assert not rep["ok"]
                return
    pytest.skip("no tie in this draw")
