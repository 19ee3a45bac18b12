"""Keys in a paged cache (FlashTopK README, "Roadmap": paged KV cache).

A workload's keys are scattered over a shuffled page pool with garbage in
the unused pages; the paged call must return the contiguous call's bits,
and the oracle's result on the logical keys (bit-exact on integer data).
The fused path gathers the keys first; the dense path (the default for
calls of few (row, key) pairs, and forced recovery) reads each key from its
page.  Both are run on every case.
"""
import numpy as np
import pytest

import workloads

from gpu_util import parity, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _pool(wl, page_size, seed):
    """Page pool, scale pool and block table holding wl's keys."""
    S = wl["kv"].shape[0]
    nblk = (S + page_size - 1) // page_size
    num_pages = nblk + 5
    rng = np.random.default_rng(seed)
    table = rng.permutation(num_pages)[:nblk].astype(np.int32)
    kv = wl["kv"]
    pool = rng.integers(0, 256 if kv.dtype == np.uint8 else 65536, size=(num_pages, page_size, 128)).astype(kv.dtype)
    if kv.dtype == np.uint16:
        pool &= np.uint16(0x3FFF)  # finite garbage
    else:
        pool &= np.uint8(0x77)
    spool = rng.random((num_pages, page_size)).astype(np.float32) * 7.0
    for b in range(nblk):
        n = min(page_size, S - b * page_size)
        pool[table[b], :n] = kv[b * page_size: b * page_size + n]
        if wl["kv_scales"] is not None:
            spool[table[b], :n] = wl["kv_scales"][b * page_size: b * page_size + n]
    return pool, (spool if wl["kv_scales"] is not None else None), table


def _run_paged(wl, page_size, seed, options=None):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    pool, spool, table = _pool(wl, page_size, seed)
    d = to_device(wl)
    if wl["dtype"] == "fp8":
        kp = torch.from_numpy(pool).cuda().view(torch.float8_e4m3fn)
    else:
        kp = torch.from_numpy(pool.view(np.int16)).cuda().view(torch.bfloat16)
    sp = None if spool is None else torch.from_numpy(spool).cuda()
    tb = torch.from_numpy(table).cuda()
    T, k = wl["q"].shape[0], wl["topk"]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ftk.flashtopk_select_paged(d["q"], kp, sp, tb, wl["kv"].shape[0], d["weights"], d["ks"], d["ke"], k, idx, val,
                               options=options)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


CASES = [
    ("int_fp8_256x8192_k512_p64", lambda: workloads.config(2), 64, "exact"),
    ("int_bf16_96x20001_k300_p100", lambda: workloads.integer(96, 20001, 300, "bf16", 1001), 100, "exact"),
    ("int_fp8_3x30000_k1024_p16", lambda: workloads.integer(3, 30000, 1024, "fp8", 1002), 16, "exact"),
    ("int_bf16_2x50000_k2048_p37", lambda: workloads.integer(2, 50000, 2048, "bf16", 1004), 37, "exact"),
    ("gauss_bf16_64x2048_k64_p7_noscales", lambda: workloads.config(1), 7, "tolerance"),
    ("trained_fp8_1x131072_k2048_p64", lambda: workloads.trained_shaped(1, 131072, 2048, "fp8", 1003), 64,
     "tolerance"),
]


@pytest.mark.parametrize("name,make,page_size,mode", CASES, ids=[c[0] for c in CASES])
def test_paged_matches_contiguous_and_oracle(name, make, page_size, mode):
    print("paged case", name, flush=True)
    wl = make()
    got = _run_paged(wl, page_size, 1010)
    ref = run_gpu(wl)
    assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32))
    rep = parity(wl, got[0], got[1], mode)
    assert rep["ok"], rep
    from gpu_util import opts

    for path in (3, 4):  # dense (pages read in place), fused (pages gathered)
        other = _run_paged(wl, page_size, 1010, options=opts(path=path))
        assert np.array_equal(other[0], got[0]), path
        assert np.array_equal(other[1].view(np.uint32), got[1].view(np.uint32)), path
