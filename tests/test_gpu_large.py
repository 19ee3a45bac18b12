"""Full-size workloads on the GPU, in the launch configuration bench.py times,
checked against the oracle on sampled rows (MI355X only).

* 4096 queries x 128K FP8 keys, causal, topk 4096 (flat Gaussian rows) and
  topk 2048 (heavy-tailed rows);
* 64K x 64K BF16 packed sequence of four documents, topk 512, rows shorter
  than topk padded;
* decode shapes: one and 64 query rows over the whole 128K context, topk 2048
  (the launch configuration splits each tile's sample over many workgroups);
* the integer-valued twins of all five, checked bit-exact.
Sampled rows: the first and last rows, random rows, and (packed) rows at
every document start and in the short-window region.
"""
import numpy as np
import pytest

import workloads

from gpu_util import parity, run_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _rows(wl, extra=()):
    T = wl["q"].shape[0]
    if T <= 64:
        return np.arange(0, T, 4 if T > 16 else 1, dtype=np.int64)
    rows = sample_rows(T, n_mid=20, edge=6, seed=T)
    return np.unique(np.concatenate([rows, np.asarray(extra, np.int64)])).astype(np.int64)


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
]


@pytest.mark.parametrize("name,n,twin,mode", CASES, ids=[c[0] for c in CASES])
def test_full_size_sampled_rows(name, n, twin, mode):
    import sparse_attention_indexer_fp8_amd as ftk

    print("case", name, flush=True)
    wl = workloads.config(n, integer_twin=twin)
    idx, val = run_gpu(wl)
    info = ftk.flashtopk_get_last_info()
    print("info", info, flush=True)
    if n in (3, 4, 5):
        _check_row_classes(wl, info)
    rows = _rows(wl, _packed_extra() if n == 5 else ())
    rep = parity(wl, idx, val, mode, rows=rows)
    assert rep["ok"], rep
    # every row, sampled or not, has the right structure
    import checker

    T = wl["q"].shape[0]
    for t in range(0, T, max(1, T // 512)):
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
