"""Standalone exact top-k over materialized score rows (DeepSelect README,
"Usage" and "Variable-length rows") through the C ABI, against the oracle.

Selection is integer work on given values, so the bar is bit-exact indices
and value bits.  Cases span BF16 and float32 rows, several 4096-entry
stretches of a row with a ragged tail, padded strides, per-row ends (empty,
shorter than topk, beyond cols), heavy ties that overflow the gathered set
(the streamed fallback), signed zeros and infinities, topk 1 and 4096, and
the benchmark's sizes on sampled rows.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _dev(wl):
    import torch

    x = wl["x"]
    if wl["dtype"] == "f32":
        t = torch.from_numpy(x).cuda()
    else:
        t = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    cols = wl["cols"]
    t = t[:, :cols]  # keeps the padded row stride
    e = None if wl["ends"] is None else torch.from_numpy(np.asarray(wl["ends"], np.int32)).cuda()
    return t, e


def _run(wl, topk=None, values=True, nan_flag=None):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    t, e = _dev(wl)
    k = topk or wl["topk"]
    idx = torch.full((t.shape[0], k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((t.shape[0], k), 7.0, dtype=torch.float32, device="cuda") if values else None
    ftk.flashtopk_topk_rows(t, k, idx, val, e, nan_flag)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (val.cpu().numpy() if values else None)


def _oracle(wl, topk=None, rows=None):
    x = np.ascontiguousarray(wl["x"][:, :wl["cols"]])
    e = wl["ends"]
    if rows is not None:
        x = x[rows]
        e = None if e is None else np.asarray(e)[rows]
    return oracle.topk_rows(x, topk or wl["topk"], ends=e)


def _check(wl, got, topk=None):
    want = _oracle(wl, topk)
    assert np.array_equal(got[0], want[0]), np.argwhere(got[0] != want[0])[:5]
    if got[1] is not None:
        assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))


CASES = [
    # (rows, cols, dtype, kind, topk, ends, stride)
    (8, 20000, "bf16", "normal", 512, None, None),
    (8, 20001, "f32", "normal", 512, None, 20004),
    (16, 12345, "bf16", "skewed", 300, "ragged", 12352),
    (6, 65536, "f32", "ties", 512, None, None),          # overflows the gathered set
    (6, 30000, "bf16", "ties", 64, "ragged", None),
    (12, 9000, "f32", "special", 700, "ragged", None),   # +-0, +-inf
    (4, 50000, "bf16", "normal", 4096, None, None),
    (4, 50000, "f32", "skewed", 1, None, None),
    (3, 7, "bf16", "normal", 16, None, 8),                # shorter than topk
    (5, 4100, "f32", "normal", 4096, "ragged", None),
    (64, 1000, "bf16", "normal", 2048, "causal", 1000),
]


@pytest.mark.parametrize("case", CASES, ids=["_".join(map(str, c)) for c in CASES])
def test_rows_match_oracle(case):
    rows, cols, dtype, kind, topk, ends, stride = case
    _say("rows case", case)
    wl = workloads.score_rows(rows, cols, dtype, 900 + rows + cols, kind=kind, topk=topk, ends=ends,
                              stride=stride)
    _check(wl, _run(wl))


def test_rows_without_values_and_empty_rows():
    wl = workloads.score_rows(8, 5000, "bf16", 911, topk=100,
                              ends=np.array([0, 5000, -3, 1, 99, 100, 101, 7000], np.int32))
    idx, _ = _run(wl, values=False)
    want = _oracle(wl)
    assert np.array_equal(idx, want[0])
    assert np.all(idx[0] == -1) and np.all(idx[2] == -1)


def test_rows_single_row_any_cols():
    # one row: no stride requirement, odd length
    wl = workloads.score_rows(1, 100003, "bf16", 912, topk=512)
    _check(wl, _run(wl))


def test_rows_nan_flag():
    import torch

    wl = workloads.score_rows(4, 3000, "f32", 913, topk=50)
    wl["x"][2, 1234] = np.nan
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx, val = _run(wl, nan_flag=flag)
    assert int(flag.item()) == 1
    clean = [0, 1, 3]
    want = oracle.topk_rows(np.ascontiguousarray(wl["x"][clean]), 50)
    assert np.array_equal(idx[clean], want[0])
    assert np.array_equal(val[clean].view(np.uint32), want[1].view(np.uint32))
    # the NaN row's selection is unspecified but in range
    assert np.all((idx[2] >= -1) & (idx[2] < 3000))
    wl["x"][2, 1234] = 0.0
    flag.zero_()
    _run(wl, nan_flag=flag)
    assert int(flag.item()) == 0


@pytest.mark.parametrize("dtype,rows,cols,kind", [("bf16", 4096, 131072, "normal"),
                                                  ("bf16", 64, 131072, "skewed"),
                                                  ("f32", 256, 129280, "normal")])
def test_rows_benchmark_sizes_sampled(dtype, rows, cols, kind):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    _say("rows bench size", dtype, rows, cols, kind)
    x = workloads.score_rows_device(rows, cols, dtype, 920, kind=kind)
    idx, val = ftk.topk_rows(x, 512)
    torch.cuda.synchronize()
    pick = np.random.default_rng(921).choice(rows, size=min(rows, 48), replace=False)
    sub = x[torch.from_numpy(pick).cuda()]
    h = sub.cpu().float().numpy() if dtype == "f32" else sub.view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.topk_rows(np.ascontiguousarray(h), 512)
    got_i = idx.cpu().numpy()[pick]
    got_v = val.cpu().numpy()[pick]
    assert np.array_equal(got_i, want[0])
    assert np.array_equal(got_v.view(np.uint32), want[1].view(np.uint32))


@pytest.mark.parametrize("level", [100.0, -100.0])
def test_rows_misleading_sample_falls_back(level):
    # The kernel samples 64 runs of 128 bytes at lines floor(j * lines / 64).
    # With 2048 lines per row those are the lines divisible by 32: shifting
    # just them makes the sample overstate (+100: too few entries reach the
    # threshold) or understate (-100: far too many) the row's top, so the
    # exact digit-histogram path has to finish the row.  Any other sampling
    # layout merely skips the fallback; the result must match either way.
    rows, cols = 6, 131072
    wl = workloads.score_rows(rows, cols, "bf16", 931, topk=512)
    x = wl["x"].view(np.int16)
    import torch

    vals = torch.from_numpy(x.copy()).view(torch.bfloat16).float().numpy()
    lines = vals.reshape(rows, -1, 64)
    lines[:, ::32, :] += level
    wl["x"] = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _check(wl, _run(wl))


def _random_rows_case(seed):
    rng = np.random.default_rng(7700 + seed)
    rows = int(rng.choice([1, 2, 5, 17, 64, 130, 300]))
    cols = int(rng.integers(1, 70000)) if rows <= 64 else int(rng.integers(1, 20000))
    dtype = "bf16" if seed % 2 == 0 else "f32"
    kind = ["normal", "skewed", "ties", "special"][seed % 4]
    topk = int(rng.choice([1, 5, 64, 300, 512, 1024, 2048, 4096]))
    ends = [None, "ragged", "causal"][seed % 3]
    stride = None if rows == 1 or seed % 5 else cols + int(rng.integers(0, 3)) * 8 + (-cols) % 8
    return rows, cols, dtype, kind, topk, ends, stride


@pytest.mark.parametrize("seed", range(24))
def test_rows_random_shapes(seed):
    """Seeded random row counts, lengths, strides, ends, topk and value kinds
    (including the split-row form for few rows), bit-exact."""
    rows, cols, dtype, kind, topk, ends, stride = _random_rows_case(seed)
    _say("random rows", seed, rows, cols, dtype, kind, topk, ends, stride)
    if rows > 1 and stride is None and cols % 8:
        stride = cols + (-cols) % 8  # rows start 16-byte aligned
    wl = workloads.score_rows(rows, cols, dtype, 7800 + seed, kind=kind, topk=topk, ends=ends, stride=stride)
    _check(wl, _run(wl))
