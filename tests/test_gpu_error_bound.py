"""Accuracy of the GPU's binary32 scores against the oracle's binary64 ones.

The FP8 path evaluates sum_h w[h] ReLU(x_h) as (sum_h w[h] |x_h| + qbar . k) / 2,
with qbar = sum_h w[h] q_h carried into the matrix cores as three truncated
E4M3 parts of a power-of-two-scaled copy: every component keeps 12
significant bits, so |qbar' - qbar| <= 2^-11 |qbar| componentwise and

    |sigma/2 * (qbar' - qbar) . k| <= 2^-12 * sigma * kabs * Q1,

with kabs = max_d |k_d| of the key and Q1 = sum_h |w[h]| ||q_h||_1 of the row
(|qbar_d| <= sum_h |w[h]| |q_h,d|).  binary32 rounding of the 128-term
products, the 32-term head sum and the scale adds about 2^-18 of the same
quantity, and the FP8 matrix cores do not round their 128-term dot products
correctly: their error reaches 2^-16.5 of sum_d |q_d k_d| (measured below on
one-head, one-key rows, which isolate a single dot product).  Rows of at
most 4096 keys take the plain form, without the truncated query sum.  The score-bound skip test adds a margin built on
|I_gpu - I| < 2^-9 * sigma * kabs * Q1; this test checks that bound on every
returned (row, key) pair, and the tighter 2^-11 that the analysis gives.
BF16 operands multiply exactly in binary32, so only the sums round: the
test asserts 2^-16 there.
"""
import numpy as np
import pytest

import oracle
import workloads

from gpu_util import run_gpu

pytestmark = pytest.mark.gpu


def _decode(codes, dtype):
    import torch

    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().numpy()
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(torch.bfloat16).float().numpy()


def _check(wl, rows, bound_exp):
    idx, val = run_gpu(wl)
    dt = wl["dtype"]
    kv = _decode(wl["kv"], dt).astype(np.float64)
    kabs = np.abs(kv).max(axis=1)
    q = _decode(wl["q"][rows], dt).astype(np.float64)
    q1 = (np.abs(wl["weights"][rows].astype(np.float64)) * np.abs(q).sum(axis=2)).sum(axis=1)
    sigma = np.ones(kv.shape[0]) if wl["kv_scales"] is None else wl["kv_scales"].astype(np.float64)
    o = oracle.select(wl["q"], wl["kv"], dt, wl["kv_scales"], wl["weights"], wl["ks"], wl["ke"], wl["topk"],
                      rows=rows, all_scores=True)
    allsc = o[3]
    worst = 0.0
    n = 0
    for i, t in enumerate(rows):
        sel = idx[t] >= 0
        s = idx[t][sel].astype(np.int64)
        exact = allsc[i][s]
        err = np.abs(val[t][sel].astype(np.float64) - exact)
        scale = sigma[s] * kabs[s] * q1[i]
        ok = scale > 0
        assert np.all(err[~ok] == 0.0), t
        ratio = err[ok] / scale[ok]
        if ratio.size:
            worst = max(worst, float(ratio.max()))
        n += int(sel.sum())
        assert np.all(err <= 2.0 ** -9 * scale), (t, float(ratio.max()) if ratio.size else 0.0)
    print(wl["name"], "pairs", n, "worst |I_gpu - I| / (sigma kabs Q1) = 2^%.2f" % np.log2(max(worst, 1e-300)),
          flush=True)
    assert worst <= 2.0 ** bound_exp, worst


@pytest.mark.parametrize("name,make,step,bound_exp", [
    ("gaussian_fp8", lambda: workloads.gaussian(256, 20000, 512, "fp8", 1401), 1, -11),
    ("trained_fp8", lambda: workloads.trained_shaped(256, 20000, 512, "fp8", 1402), 1, -11),
    ("gaussian_fp8_small_weights", lambda: workloads.gaussian(128, 9000, 256, "fp8", 1403, weight_scale=1e-3), 1, -11),
    ("untrained_fp8_4096x131072", lambda: workloads.config(3), 64, -11),
    ("trained_fp8_4096x131072", lambda: workloads.config(4), 64, -11),
    ("gaussian_bf16", lambda: workloads.gaussian(128, 20000, 512, "bf16", 1404), 1, -16),
])
def test_scores_within_the_rounding_bound(name, make, step, bound_exp):
    print("case", name, flush=True)
    wl = make()
    T = wl["q"].shape[0]
    rows = np.arange(0, T, step, dtype=np.int64)
    _check(wl, rows, bound_exp)


@pytest.mark.parametrize("dt,bound_exp", [("fp8", -15), ("bf16", -22)])
def test_matrix_core_dot_product_error(dt, bound_exp):
    # One key per row and one head of weight 1 (sigma = 1): the returned score
    # is ReLU of the matrix core's q.k (the plain form), and ReLU takes no
    # error in, so its distance from ReLU of the exact dot product, relative
    # to sum_d |q_d k_d|, bounds the dot product's error where q.k > 0.
    T = 2048
    wl = workloads.gaussian(T, T, 1, dt, 1405, windows="full")
    w = np.zeros((T, 32), np.float32)
    w[:, 0] = 1.0
    wl.update(weights=w, kv_scales=None, ks=np.arange(T, dtype=np.int32), ke=np.arange(1, T + 1, dtype=np.int32))
    idx, val = run_gpu(wl)
    assert np.array_equal(idx[:, 0], np.arange(T))
    q = _decode(wl["q"][:, 0], dt).astype(np.float64)
    k = _decode(wl["kv"], dt).astype(np.float64)
    x = (q * k).sum(axis=1)
    l1 = (np.abs(q) * np.abs(k)).sum(axis=1)
    nz = l1 > 0
    assert np.all(val[~nz, 0] == 0.0)
    rel = np.abs(val[nz, 0].astype(np.float64) - np.maximum(x[nz], 0.0)) / l1[nz]
    pos = x[nz] > 0  # the median over rows that return q.k itself
    print(dt, "rows", int(nz.sum()), "max err / sum|q k| = 2^%.2f" % np.log2(max(rel.max(), 1e-300)),
          "median (q.k > 0) 2^%.2f" % np.log2(max(np.median(rel[pos]), 1e-300)), flush=True)
    assert rel.max() <= 2.0 ** bound_exp


def test_short_fp8_rows_take_the_plain_form():
    # Rows whose 32 heads are one FP8 vector q_t, with weights of full binary32
    # precision: the query sum (sum_h w_h) q_t needs far more than the 12 bits
    # the linear identity carries, so the identity's error shows, while the
    # plain form's error is the matrix cores' own.  Windows of 4096 keys take
    # the plain form; the same keys in windows of 4097 the identity.  The
    # plain rows' median error over keys with q.k > 0 is at the matrix cores'
    # level (about 2^-20 of sum_d |q_d k_d|).
    T, S = 64, 4096 + 64 + 1
    rng = np.random.default_rng(1406)
    base = workloads.gaussian(T, S, 4096, "fp8", 1407, windows="full")
    q = np.repeat(base["q"][:, :1, :], 32, axis=1)
    w = rng.uniform(0.5, 1.5, size=(T, 32)).astype(np.float32)
    out = {}
    for L in (4096, 4097):
        wl = dict(base, q=np.ascontiguousarray(q), weights=w, kv_scales=None,
                  ks=np.arange(T, dtype=np.int32), ke=np.arange(T, dtype=np.int32) + L)
        idx, val = run_gpu(wl)
        qd = _decode(q[:, 0], "fp8").astype(np.float64)
        kd = _decode(wl["kv"], "fp8").astype(np.float64)
        x = qd @ kd.T                                   # [T, S] exact dot products
        l1 = np.abs(qd) @ np.abs(kd).T
        W = w.astype(np.float64).sum(axis=1)
        rel, pos = [], []
        for t in range(T):
            s = idx[t][idx[t] >= 0].astype(np.int64)
            assert s.size == 4096
            exact = W[t] * np.maximum(x[t, s], 0.0)
            rel.append(np.abs(val[t][: s.size].astype(np.float64) - exact) / (W[t] * l1[t, s]))
            pos.append(x[t, s] > 0)
        rel, pos = np.concatenate(rel), np.concatenate(pos)
        out[L] = (float(np.median(rel[pos])), float(rel.max()))
        print("window", L, "median error / (W sum|q k|) = 2^%.2f, max 2^%.2f"
              % (np.log2(max(out[L][0], 1e-300)), np.log2(max(out[L][1], 1e-300))), flush=True)
    assert out[4096][0] <= 2.0 ** -19 and out[4096][1] <= 2.0 ** -15
    assert out[4097][1] <= 2.0 ** -11
