"""Calls on different streams: each (device, stream) pair owns its workspace,
so calls issued concurrently from two host threads on two streams give the
same bits as one at a time on the default stream, and each stream's last-call
record describes that stream's own call."""
import threading

import numpy as np
import pytest

import workloads

from gpu_util import run_gpu, to_device

pytestmark = pytest.mark.gpu


def test_two_streams_from_two_threads():
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    cases = [workloads.integer(300, 5000, 128, "fp8", 2401), workloads.integer(200, 7000, 256, "bf16", 2402)]
    devs = [to_device(wl) for wl in cases]
    refs = [run_gpu(wl, d) for wl, d in zip(cases, devs)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    reps = 6
    outs = [[None] * reps for _ in cases]
    errors = []

    def work(j):
        wl, d, s = cases[j], devs[j], streams[j]
        T, k = wl["q"].shape[0], wl["topk"]
        try:
            with torch.cuda.stream(s):
                for i in range(reps):
                    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
                    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
                    ftk.flashtopk_select_ex(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], k,
                                            idx, val, stream=s)
                    outs[j][i] = (idx, val)
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    print("streams: two threads", flush=True)
    threads = [threading.Thread(target=work, args=(j,)) for j in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j, wl in enumerate(cases):
        for i in range(reps):
            idx, val = outs[j][i]
            assert np.array_equal(idx.cpu().numpy(), refs[j][0]), (j, i)
            assert np.array_equal(val.cpu().numpy().view(np.uint32), refs[j][1].view(np.uint32)), (j, i)
        info = ftk.flashtopk_get_last_info(stream=streams[j])
        assert info["status"] == 0 and info["rows"] == wl["q"].shape[0], (j, info)
