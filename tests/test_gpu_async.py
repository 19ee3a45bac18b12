"""The call does not wait on the GPU (every decision stays on the device):
it returns while earlier work on its stream is still running, on the fused
path (with and without rows that need dense rescoring) and on the dense
path, and the results are the bits of an ordinary call.  With its workspace
reserved, a call can be captured into a HIP graph and replayed."""
import numpy as np
import pytest

import workloads

from gpu_util import opts, run_gpu, to_device

pytestmark = pytest.mark.gpu

FUSED, RECOVER = 4, 3


def _say(*a):
    print(*a, flush=True)


def _busy(torch, ms_target=150.0):
    """Enqueues float32 matrix products that keep the stream busy for a while."""
    a = torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    # time one product to size the queue
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    b = a @ a
    e1.record()
    torch.cuda.synchronize()
    n = int(max(4, min(400, ms_target / max(e0.elapsed_time(e1), 0.05))))
    for _ in range(n):
        b = a @ b
        b = b * (1.0 / 4096.0)
    return b


@pytest.mark.parametrize("label,kw", [
    ("fused", dict(path=FUSED)),
    ("fused_with_rescoring", dict(path=FUSED, cand_capacity=256)),
    ("dense", dict(path=RECOVER)),
    ("auto", dict()),
])
def test_call_returns_while_the_stream_is_busy(label, kw):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    _say("async", label)
    wl = workloads.gaussian(512, 40000, 256, "fp8", 1301)
    d = to_device(wl)
    ref = run_gpu(wl, d, options=opts(**kw))  # also grows the workspace
    stream = torch.cuda.current_stream()
    _busy(torch)
    idx, val = ftk.select(d["q"], d["kv"], d["weights"], d["ks"], d["ke"], d["kv_scales"], topk=wl["topk"],
                          return_scores=True, options=opts(**kw))
    still_busy = not stream.query()
    torch.cuda.synchronize()
    assert still_busy, "the call waited for the GPU"
    assert np.array_equal(idx.cpu().numpy(), ref[0])
    assert np.array_equal(val.cpu().numpy().view(np.uint32), ref[1].view(np.uint32))
    if "cand_capacity" in kw:
        assert ftk.flashtopk_get_last_info()["rows_recovered"] > 0


@pytest.mark.parametrize("path", [FUSED, RECOVER])
def test_graph_capture_replays_the_call(path):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    _say("graph", path)
    wl = workloads.gaussian(96, 30000, 512, "bf16", 1302)
    d = to_device(wl)
    ref = run_gpu(wl, d, options=opts(path=path))
    s = torch.cuda.Stream()
    T, k = wl["q"].shape[0], wl["topk"]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
    o = opts(path=path)
    with torch.cuda.stream(s):
        ftk.flashtopk_reserve(T, wl["kv"].shape[0], k, ftk.FLASHTOPK_BF16, stream=s)
        ftk.flashtopk_select_ex(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], k, idx, val,
                                stream=s, options=o)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ftk.flashtopk_select_ex(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], k, idx, val,
                                stream=s, options=o)
    for rep in range(4):
        idx.fill_(-7)
        val.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref[0]), rep
        assert np.array_equal(val.cpu().numpy().view(np.uint32), ref[1].view(np.uint32)), rep
