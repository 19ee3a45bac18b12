"""Output options (DeepSelect README, "Usage": sorted_index, indices_type;
"Recommendations": return_value=False) on both entry points.

Index order must list exactly the score-ordered call's top-k keys, by
ascending index, with each value beside its own index and the padding last;
int64 indices must equal the int32 ones.  Checked on the fused call (the
candidate selection and the forced dense-recovery selection) and on the row
top-k against the oracle's sets.
"""
import numpy as np
import pytest

import oracle
import workloads

from gpu_util import opts, parity, run_gpu, to_device

pytestmark = pytest.mark.gpu

INDEX_ORDER, INT64 = 1, 2


def _say(*a):
    print(*a, flush=True)


def _by_index(idx, val):
    """Score-ordered rows re-listed by ascending index (padding last)."""
    oi = np.full_like(idx, -1)
    ov = np.full_like(val, -np.inf)
    for r in range(idx.shape[0]):
        m = idx[r] >= 0
        o = np.argsort(idx[r][m], kind="stable")
        oi[r, :m.sum()] = idx[r][m][o]
        ov[r, :m.sum()] = val[r][m][o]
    return oi, ov


def _run(wl, d, flags, path=0):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    o = opts(path=path, out_flags=flags)
    T, k = wl["q"].shape[0], wl["topk"]
    idx = torch.empty((T, k), dtype=torch.int64 if flags & INT64 else torch.int32, device="cuda")
    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ftk.flashtopk_select_ex(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], k, idx, val,
                            options=o)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def _packed_int():
    # windows starting inside the keys (ks > 0), several shorter than topk
    return workloads.integer(600, 600, 64, "fp8", 2501, windows="packed", docs=(40, 300, 20, 240))


@pytest.mark.parametrize("make", [lambda: workloads.config(2), _packed_int], ids=["tieheavy", "packed"])
@pytest.mark.parametrize("path", [4, 3], ids=["candidates", "recover_all"])
def test_fused_index_order_and_int64(path, make):
    wl = make()  # tie-heavy integer data; rows shorter than topk
    d = to_device(wl)
    base = _run(wl, d, 0, path)
    rep = parity(wl, base[0], base[1], "exact")
    assert rep["ok"], rep
    want = _by_index(*base)
    got = _run(wl, d, INDEX_ORDER, path)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))
    got64 = _run(wl, d, INDEX_ORDER | INT64, path)
    assert got64[0].dtype == np.int64
    assert np.array_equal(got64[0], want[0].astype(np.int64))
    s64 = _run(wl, d, INT64, path)
    assert np.array_equal(s64[0], base[0].astype(np.int64))
    assert np.array_equal(s64[1].view(np.uint32), base[1].view(np.uint32))


def test_fused_index_order_binding_helpers():
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    wl = workloads.config(1)
    d = to_device(wl)
    i32, v32 = ftk.select(d["q"], d["kv"], d["weights"], d["ks"], d["ke"], d["kv_scales"], topk=64,
                          return_scores=True)
    i64 = ftk.select(d["q"], d["kv"], d["weights"], d["ks"], d["ke"], d["kv_scales"], topk=64,
                     sorted_index=True, indices_type=torch.int64)
    torch.cuda.synchronize()
    want = _by_index(i32.cpu().numpy(), v32.cpu().numpy())[0]
    assert i64.dtype == torch.int64
    assert np.array_equal(i64.cpu().numpy(), want)


@pytest.mark.parametrize("dtype,topk,ends", [("bf16", 512, "ragged"), ("f32", 4096, None), ("bf16", 1, None),
                                             ("f32", 100, "ragged")])
def test_rows_index_order_and_int64(dtype, topk, ends):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    _say("rows outputs", dtype, topk, ends)
    wl = workloads.score_rows(12, 20000, dtype, 950 + topk, kind="ties" if topk == 100 else "normal",
                              topk=topk, ends=ends)
    x = torch.from_numpy(wl["x"]).cuda() if dtype == "f32" else \
        torch.from_numpy(wl["x"].view(np.int16)).cuda().view(torch.bfloat16)
    e = None if wl["ends"] is None else torch.from_numpy(wl["ends"]).cuda()
    want = oracle.topk_rows(wl["x"], topk, ends=wl["ends"])
    want_i = _by_index(*want)
    for itype in (torch.int32, torch.int64):
        idx, val = ftk.topk_rows(x, topk, ends=e, sorted_index=True, indices_type=itype)
        torch.cuda.synchronize()
        assert idx.dtype == itype
        assert np.array_equal(idx.cpu().numpy(), want_i[0].astype(idx.cpu().numpy().dtype))
        assert np.array_equal(val.cpu().numpy().view(np.uint32), want_i[1].view(np.uint32))
        idx, val = ftk.topk_rows(x, topk, ends=e, indices_type=itype)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), want[0].astype(idx.cpu().numpy().dtype))
        assert np.array_equal(val.cpu().numpy().view(np.uint32), want[1].view(np.uint32))


def test_rows_index_order_large_batch_uses_pre_pass():
    # more rows than resident workgroups: thresholds come from the pre-pass,
    # parked in the int64 output's first bytes
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    x = workloads.score_rows_device(2048, 65536, "bf16", 960)
    i32, v32 = ftk.topk_rows(x, 512)
    i64, v64 = ftk.topk_rows(x, 512, sorted_index=True, indices_type=torch.int64)
    torch.cuda.synchronize()
    want = _by_index(i32.cpu().numpy(), v32.cpu().numpy())
    assert np.array_equal(i64.cpu().numpy(), want[0].astype(np.int64))
    assert np.array_equal(v64.cpu().numpy().view(np.uint32), want[1].view(np.uint32))
