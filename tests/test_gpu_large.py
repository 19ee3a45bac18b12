"""Full-size workloads on the GPU, in the launch configuration bench.py times,
checked against the oracle (MI355X only).

* 4096 queries x 128K FP8 keys, causal, topk 4096 (flat Gaussian rows) and
  topk 2048 (heavy-tailed rows);
* 64K x 64K BF16 packed sequence of four documents, topk 512, rows shorter
  than topk padded;
* decode shapes: one and 64 query rows over the whole 128K context, topk 2048
  (the dense path: every row's scores materialised, each row's selection
  split over several workgroups), and the 64-row shape forced through the
  fused path (each tile's sample split over many workgroups);
* the integer-valued twins of all of them, checked bit-exact;
* block-local integer keys at the headline's size on the pruned scan (FP8
  auto, BF16 forced), bit-exact.
Rows checked against the oracle: every 16th row, the first and the last 64
rows, every row the call rescored densely, and (packed) the rows around
every document start and the short-window boundaries; decode shapes on
every row.  The structure of every row (count, uniqueness, windows,
padding, order) is checked on all rows.
"""
import numpy as np
import pytest

import workloads

from gpu_util import parity, run_gpu

pytestmark = pytest.mark.gpu


def _rows(wl, extra=(), recovered=()):
    """Every 16th row, the first and last 64, the rows the call rescored and
    the extra rows (all rows when there are at most 64)."""
    T = wl["q"].shape[0]
    if T <= 64:
        return np.arange(T, dtype=np.int64)
    rows = np.concatenate([np.arange(0, T, 16), np.arange(min(64, T)), np.arange(max(0, T - 64), T),
                           np.asarray(recovered, np.int64), np.asarray(extra, np.int64)])
    return np.unique(rows[(rows >= 0) & (rows < T)]).astype(np.int64)


def _packed_extra():
    starts = np.cumsum((0,) + workloads.PACKED_DOCS[:-1])
    extra = []
    for s in starts:
        extra += [s, s + 1, s + 255, s + 510, s + 511, s + 512, s + 2047, s + 2048, s + 2049]
    return extra


def _check_row_classes(wl, info):
    """The call's row classes and window total, recomputed on the host."""
    T = wl["q"].shape[0]
    lens = np.maximum(wl["ke"].astype(np.int64) - wl["ks"].astype(np.int64), 0)
    cap = info["cand_capacity"]
    assert info["rows"] == T
    assert info["rows_empty"] == int((lens == 0).sum())
    assert info["rows_take_all"] == int(((lens > 0) & (lens <= cap)).sum())
    assert info["rows_sampled"] == int((lens > cap).sum())
    assert info["window_keys"] == int(lens.sum())
    assert info["rows_recovered"] == info["rows_underflow"] + info["rows_overflow"]


CASES = [
    ("untrained_fp8_k4096", 3, False, "tolerance"),
    ("trained_fp8_k2048", 4, False, "tolerance"),
    ("packed_bf16_k512", 5, False, "tolerance"),
    ("untrained_int_fp8_k4096", 3, True, "exact"),
    ("trained_int_fp8_k2048", 4, True, "exact"),
    ("packed_int_bf16_k512", 5, True, "exact"),
    ("decode_fp8_1x131072", 7, False, "tolerance"),
    ("decode_fp8_64x131072", 8, False, "tolerance"),
    ("decode_int_fp8_1x131072", 7, True, "exact"),
    ("decode_int_fp8_64x131072", 8, True, "exact"),
    ("decode_fused_fp8_64x131072", 8, False, "tolerance"),
    ("decode_fused_int_fp8_64x131072", 8, True, "exact"),
]


@pytest.mark.parametrize("name,n,twin,mode", CASES, ids=[c[0] for c in CASES])
def test_full_size_parity(name, n, twin, mode):
    import sparse_attention_indexer_fp8_amd as ftk

    from gpu_util import opts

    print("case", name, flush=True)
    wl = workloads.config(n, integer_twin=twin)
    idx, val = run_gpu(wl, options=opts(path=4) if "fused" in name else None)
    info = ftk.flashtopk_get_last_info()
    recovered = ftk.flashtopk_get_last_recovered()
    print("info", info, "recovered", recovered[:20], flush=True)
    assert len(recovered) == info["rows_recovered"]
    if n in (3, 4, 5):
        _check_row_classes(wl, info)
    rows = _rows(wl, _packed_extra() if n == 5 else (), recovered)
    print("oracle rows", len(rows), flush=True)
    rep = parity(wl, idx, val, mode, rows=rows)
    assert rep["ok"], rep
    # every row has the right structure
    import checker

    T = wl["q"].shape[0]
    for t in range(T):
        assert not checker.structure_failures(idx[t], val[t], wl["ks"][t], wl["ke"][t], wl["topk"]), t
    if n == 5:
        short = (wl["ke"] - wl["ks"]) < wl["topk"]
        assert short.sum() == 4 * 511
        assert np.all(idx[short][:, -1] == -1)


def test_many_rows_mixed_windows():
    # 20001 rows (more than one triage workgroup's 4096, the last one
    # partial): empty, take-all and sampled windows mixed; class counts on
    # every row, parity on sampled rows.
    import sparse_attention_indexer_fp8_amd as ftk

    wl = workloads.integer(20001, 3000, 64, "fp8", 2301, windows="full")
    rng = np.random.default_rng(2302)
    kind = rng.integers(0, 3, size=20001)
    lo = rng.integers(0, 3000, size=20001)
    ln = np.where(kind == 0, 0, np.where(kind == 1, rng.integers(1, 257, size=20001), rng.integers(257, 3001, size=20001)))
    lo = np.minimum(lo, 3000 - ln)
    wl["ks"] = lo.astype(np.int32)
    wl["ke"] = (lo + ln).astype(np.int32)
    print("case many rows", flush=True)
    idx, val = run_gpu(wl)
    info = ftk.flashtopk_get_last_info()
    print("info", info, flush=True)
    assert info["cand_capacity"] == 256
    _check_row_classes(wl, info)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(20001 - 8, 20001),
                                     rng.choice(20001, size=24, replace=False)])).astype(np.int64)
    rep = parity(wl, idx, val, "exact", rows=rows)
    assert rep["ok"], rep


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_full_size_block_local_parity(dt):
    # Block-local integer keys at the headline's size: the scan's work items
    # hold whole windows (up to 2048 key steps), so the step-list compaction
    # of the pruned scan runs several rounds per thread.  FP8 takes the auto
    # path (its planner picks pruning), BF16 is forced onto it.
    import sparse_attention_indexer_fp8_amd as ftk

    from gpu_util import opts

    name = f"blocky_int_{dt}_4096x131072_k2048"
    print("case", name, flush=True)
    wl = workloads.blocky(4096, 131072, 2048, dt, 610 if dt == "fp8" else 611, exact=True, name=name)
    idx, val = run_gpu(wl, options=None if dt == "fp8" else opts(path=2))
    info = ftk.flashtopk_get_last_info()
    recovered = ftk.flashtopk_get_last_recovered()
    print("info", info, flush=True)
    assert info["path"] == ftk.PATH_PRUNE, info
    assert info["pruned_keys"] > info["window_keys"] // 4, info
    _check_row_classes(wl, info)
    rows = _rows(wl, (), recovered)
    print("oracle rows", len(rows), flush=True)
    rep = parity(wl, idx, val, "exact", rows=rows)
    assert rep["ok"], rep
    import checker

    for t in range(wl["q"].shape[0]):
        assert not checker.structure_failures(idx[t], val[t], wl["ks"][t], wl["ke"][t], wl["topk"]), t
