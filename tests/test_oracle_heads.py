"""Pins of the oracle for indexers with 64 heads (FlashTopK README,
"Roadmap": indexers with a head count other than 32, 64 being the case
named there; the score keeps its definition with the head sum running over
all heads).

* The numpy twin (an independent formulation whose head count comes from
  the operand shapes) agrees on random 64-head inputs.
* A 64-head problem whose upper 32 heads have zero weight is the 32-head
  problem on the lower heads, score for score.
* The head sum splits: with sigma = 1, the 64-head score is the sum of the
  two 32-head scores of the halves (binary64, to rounding).
* Jointly permuting the 64 heads of q and weights leaves integer-valued
  selections bit-identical.
"""
import numpy as np

import oracle
import workloads
from oracle import numpy_ref


def _decoded(wl):
    return numpy_ref.decode(wl["q"], wl["dtype"]), numpy_ref.decode(wl["kv"], wl["dtype"])


def test_numpy_twin_agrees_on_64_heads():
    for dtype, seed in (("fp8", 1101), ("bf16", 1102)):
        wl = workloads.gaussian(6, 300, 40, dtype, seed, heads=64)
        qd, kd = _decoded(wl)
        want = numpy_ref.score_matrix(qd, kd, wl["weights"], wl["kv_scales"])
        for t in range(6):
            got = oracle.scores(wl["q"], wl["kv"], dtype, wl["kv_scales"], wl["weights"], t, 0, 300)
            assert np.allclose(got, want[t], rtol=1e-12, atol=1e-12)
        idx, val, _, _ = oracle.select(wl["q"], wl["kv"], dtype, wl["kv_scales"], wl["weights"], wl["ks"], wl["ke"], 40)
        tidx, tval = numpy_ref.select(wl["q"], wl["kv"], dtype, wl["kv_scales"], wl["weights"], wl["ks"], wl["ke"], 40)[:2]
        assert np.array_equal(idx, tidx)
        assert np.array_equal(val, tval)


def test_zero_upper_heads_reduce_to_32_heads():
    wl = workloads.integer(5, 200, 30, "fp8", 1103, heads=64)
    w = wl["weights"].copy()
    w[:, 32:] = 0.0
    lo_q = np.ascontiguousarray(wl["q"][:, :32])
    for t in range(5):
        a = oracle.scores(wl["q"], wl["kv"], "fp8", wl["kv_scales"], w, t, 0, 200)
        b = oracle.scores(lo_q, wl["kv"], "fp8", wl["kv_scales"], np.ascontiguousarray(w[:, :32]), t, 0, 200)
        assert np.array_equal(a, b)


def test_head_sum_splits_into_halves():
    wl = workloads.gaussian(4, 150, 20, "bf16", 1104, heads=64, scales="ones")
    q, w = wl["q"], wl["weights"]
    for t in range(4):
        full = oracle.scores(q, wl["kv"], "bf16", None, w, t, 0, 150)
        lo = oracle.scores(np.ascontiguousarray(q[:, :32]), wl["kv"], "bf16", None, np.ascontiguousarray(w[:, :32]),
                           t, 0, 150)
        hi = oracle.scores(np.ascontiguousarray(q[:, 32:]), wl["kv"], "bf16", None, np.ascontiguousarray(w[:, 32:]),
                           t, 0, 150)
        assert np.allclose(full, lo + hi, rtol=1e-13, atol=1e-13)


def test_joint_head_permutation_keeps_integer_selection():
    wl = workloads.integer(8, 500, 64, "bf16", 1105, heads=64)
    perm = np.random.default_rng(1106).permutation(64)
    a = oracle.select(wl["q"], wl["kv"], "bf16", wl["kv_scales"], wl["weights"], wl["ks"], wl["ke"], 64)
    b = oracle.select(np.ascontiguousarray(wl["q"][:, perm]), wl["kv"], "bf16", wl["kv_scales"],
                      np.ascontiguousarray(wl["weights"][:, perm]), wl["ks"], wl["ke"], 64)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1], b[1])
