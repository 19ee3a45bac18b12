"""Indexers with 64 heads (FlashTopK README, "Roadmap": head counts besides
32, with 64 as the named case).  Each row's two 32-head halves are
neighbouring tile columns whose head sums are added before the threshold.

Integer data bit-exact against the oracle (which takes the head count from
the operand shapes), forced paths bit-identical to the default, Gaussian
data within the tolerance rule, and a full-size chunk on sampled rows.
"""
import numpy as np
import pytest

import workloads

from gpu_util import opts, parity, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def _ragged(wl, seed):
    T, S = wl["q"].shape[0], wl["kv"].shape[0]
    rng = np.random.default_rng(seed)
    ks, ke = wl["ks"].copy(), wl["ke"].copy()
    for t in range(0, T, 3):
        a, b = np.sort(rng.integers(0, S + 1, size=2))
        ks[t], ke[t] = a, b
    ks[1], ke[1] = 7, 7                   # empty
    if T > 5:
        ks[5], ke[5] = 100, 100 + 31      # shorter than topk
    return dict(wl, ks=ks.astype(np.int32), ke=ke.astype(np.int32))


CASES = [
    (40, 9000, 300, "fp8"),
    (33, 12001, 512, "bf16"),
    (1, 20000, 2048, "fp8"),
    (3, 7000, 64, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=["_".join(map(str, c)) for c in CASES])
def test_64_heads_integer_exact_and_paths(case):
    T, S, topk, dt = case
    print("heads64", case, flush=True)
    wl = workloads.integer(T, S, topk, dt, 1200 + T, heads=64)
    if T > 3:
        wl = _ragged(wl, 1201)
    d = to_device(wl)
    got = run_gpu(wl, d)
    rep = parity(wl, got[0], got[1], "exact")
    assert rep["ok"], rep
    for o in (opts(path=3), opts(path=2), opts(path=4), opts(path=4, cand_capacity=topk),
              opts(path=4, sample_rank_scale=0.02)):
        assert _same(run_gpu(wl, d, options=o), got)


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_64_heads_gaussian(dt):
    wl = workloads.gaussian(128, 32768, 1024, dt, 1210, heads=64)
    got = run_gpu(wl)
    rep = parity(wl, got[0], got[1], "tolerance")
    assert rep["ok"], rep


def test_64_heads_full_size_parity():
    # every 16th row, the first and last 64 and every rescored row
    import sparse_attention_indexer_fp8_amd as ftk

    wl = workloads.config(9)
    got = run_gpu(wl)
    recovered = ftk.flashtopk_get_last_recovered()
    T = wl["q"].shape[0]
    rows = np.unique(np.concatenate([np.arange(0, T, 16), np.arange(64), np.arange(T - 64, T),
                                     recovered.astype(np.int64)])).astype(np.int64)
    print("oracle rows", len(rows), "recovered", len(recovered), flush=True)
    rep = parity(wl, got[0], got[1], "tolerance", rows=rows)
    assert rep["ok"], rep
