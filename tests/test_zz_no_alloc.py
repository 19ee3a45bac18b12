"""flashtopk_select_noalloc (for callers that cannot allocate device memory):
its results must be the bits of flashtopk_select on the same inputs, on two
calls in a row of which the second is smaller (the fixed array keeps the
first call's contents), on the dense and the fused path; it must leave the
device's free memory unchanged, and reject a call whose workspace does not
fit its fixed array without touching the outputs."""
import numpy as np
import pytest

import workloads

from gpu_util import run_gpu, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _noalloc(wl, d):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    T, k = wl["q"].shape[0], wl["topk"]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    val = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    ftk.flashtopk_select_noalloc(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], k, idx, val)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return idx.cpu().numpy(), val.cpu().numpy(), free0, free1


@pytest.mark.parametrize("pair", ["dense", "fused"])
def test_noalloc_matches_select_on_two_calls(pair):
    if pair == "dense":
        big = workloads.trained_shaped(64, 65536, 2048, "fp8", 1501)            # 4M (row, key) pairs: dense
        small = workloads.gaussian(5, 20000, 300, "bf16", 1502)
    else:
        big = workloads.gaussian(512, 20000, 256, "fp8", 1503)                  # 10M pairs: fused
        small = workloads.integer(300, 30000, 100, "bf16", 1504)                # 9M pairs: fused
    for wl in (big, small):
        _say("noalloc", pair, wl["name"])
        d = to_device(wl)
        ref = run_gpu(wl, d)
        got = _noalloc(wl, d)
        assert got[2] == got[3], "the call changed the device's free memory"
        assert np.array_equal(got[0], ref[0])
        assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32))


def test_noalloc_rejects_a_call_too_large():
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    wl = workloads.gaussian(4096, 16384, 4096, "fp8", 1505)  # candidates alone: 4096 * 16384 * 8 B = 512 MiB
    d = to_device(wl)
    T, k = wl["q"].shape[0], wl["topk"]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(ftk.FlashTopKError) as err:
        ftk.flashtopk_select_noalloc(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], k, idx)
    assert err.value.status == ftk.FLASHTOPK_ERR_WORKSPACE_LIMIT
    torch.cuda.synchronize()
    assert bool((idx == -7).all())
