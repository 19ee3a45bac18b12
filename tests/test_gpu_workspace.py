"""The workspace contract (FlashTopK README, "Usage": the Selector owns the
workspace and prepares up front): after flashtopk_reserve, calls up to the
reserved sizes allocate nothing (the device's free memory is unchanged), on
the fused and the dense path, with 32 and 64 heads, and for the row top-k of
few rows; after flashtopk_release, calls work again with the same bits."""
import numpy as np
import pytest

import workloads

from gpu_util import opts, to_device

pytestmark = pytest.mark.gpu


def _call(ftk, d, wl, idx, val, stream, path=0):
    o = opts(path=path)
    ftk.flashtopk_select_ex(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], wl["topk"], idx, val,
                            stream=stream, options=o)


def test_calls_after_reserve_allocate_nothing():
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    s = torch.cuda.Stream()
    cases = [
        (workloads.trained_shaped(600, 40000, 1024, "fp8", 1601), 0),      # fused (24M pairs)
        (workloads.gaussian(30, 40000, 1024, "fp8", 1602), 0),             # dense (1.2M pairs)
        (workloads.gaussian(600, 40000, 1024, "fp8", 1603), 3),            # dense, forced
        (workloads.integer(300, 40000, 512, "fp8", 1604, heads=64), 0),    # 64 heads
    ]
    outs = []
    for wl, path in cases:
        d = to_device(wl)
        T, k = wl["q"].shape[0], wl["topk"]
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        val = torch.empty((T, k), dtype=torch.float32, device="cuda")
        outs.append((wl, path, d, idx, val))
    rows = torch.randn(40, 40000, device="cuda")
    ridx = torch.empty((40, 1024), dtype=torch.int32, device="cuda")
    ftk.flashtopk_reserve(600, 40000, 1024, ftk.FLASHTOPK_FP8_E4M3, stream=s)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    with torch.cuda.stream(s):
        for wl, path, d, idx, val in outs:
            print("reserved call", wl["name"], path, flush=True)
            _call(ftk, d, wl, idx, val, s, path)
        ftk.flashtopk_topk_rows(rows, 1024, ridx, stream=s)
    s.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)


def test_release_then_call_again():
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    wl = workloads.gaussian(200, 50000, 512, "bf16", 1605)
    d = to_device(wl)
    T, k = wl["q"].shape[0], wl["topk"]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
    _call(ftk, d, wl, idx, val, None)
    torch.cuda.synchronize()
    ref = (idx.cpu().numpy(), val.cpu().numpy())
    ftk.flashtopk_release()
    idx.fill_(-7)
    _call(ftk, d, wl, idx, val, None)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref[0])
    assert np.array_equal(val.cpu().numpy().view(np.uint32), ref[1].view(np.uint32))
    assert ftk.flashtopk_get_last_info()["rows"] == T
