"""Score-bound pruning (FlashTopK README, "Highlights": per-key-block score
bounds skip whole blocks below the row's threshold, decided per call).

Pruning may only change speed: the forced prune path, the planner's choice
and the plain scan must return identical bits, and the oracle must agree
(bit-exact on integer data).  Block-local data makes the bound skip blocks;
untrained-shaped data must leave the planner on the scan.
"""
import numpy as np
import pytest

import workloads

from gpu_util import opts, parity, run_gpu, to_device

pytestmark = pytest.mark.gpu

SCAN, PRUNE, FUSED = 1, 2, 4


def _say(*a):
    print(*a, flush=True)


def _info():
    import sparse_attention_indexer_fp8_amd as ftk

    return ftk.flashtopk_get_last_info()


def _same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


CASES = [
    ("blocky_int_fp8_96x20000_k128", lambda: workloads.blocky(96, 20000, 128, "fp8", 501, exact=True), "exact"),
    ("blocky_int_bf16_80x17000_k64", lambda: workloads.blocky(80, 17000, 64, "bf16", 502, exact=True), "exact"),
    ("blocky_gauss_fp8_128x40000_k256", lambda: workloads.blocky(128, 40000, 256, "fp8", 503), "tolerance"),
    ("blocky_gauss_bf16_64x30001_k100", lambda: workloads.blocky(64, 30001, 100, "bf16", 504), "tolerance"),
]


@pytest.mark.parametrize("name,make,mode", CASES, ids=[c[0] for c in CASES])
def test_forced_prune_matches_scan_and_oracle(name, make, mode):
    _say("case", name)
    wl = make()
    d = to_device(wl)
    scan = run_gpu(wl, d, options=opts(path=SCAN))
    assert _info()["pruned_keys"] == 0
    pr = run_gpu(wl, d, options=opts(path=PRUNE))
    info = _info()
    assert info["path"] == PRUNE, info
    assert info["pruned_keys"] > 0, info
    assert _same(pr, scan)
    auto = run_gpu(wl, d)
    assert _same(auto, scan)
    planned = run_gpu(wl, d, options=opts(path=FUSED))
    assert _same(planned, scan)
    rep = parity(wl, pr[0], pr[1], mode)
    assert rep["ok"], rep


def test_planner_prunes_block_local_keys():
    wl = workloads.blocky(256, 65536, 512, "fp8", 505)
    d = to_device(wl)
    scan = run_gpu(wl, d, options=opts(path=SCAN))
    auto = run_gpu(wl, d, options=opts(path=FUSED))
    info = _info()
    _say("auto", info)
    assert info["path"] == PRUNE, info
    assert info["pruned_keys"] > info["window_keys"] // 4, info
    assert _same(auto, scan)


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_planner_scans_untrained_keys(dtype):
    wl = workloads.gaussian(128, 32768, 256, dtype, 506)
    d = to_device(wl)
    scan = run_gpu(wl, d, options=opts(path=SCAN))
    auto = run_gpu(wl, d, options=opts(path=FUSED))
    info = _info()
    assert info["path"] == SCAN, info
    assert info["pruned_keys"] == 0, info
    assert _same(auto, scan)
    pr = run_gpu(wl, d, options=opts(path=PRUNE))
    assert _same(pr, scan)


def test_negative_scale_blocks_are_never_skipped():
    # Outside the kv_scales >= 0 precondition the bound does not hold; blocks
    # holding a negative scale must simply not be skipped.
    wl = workloads.blocky(64, 12000, 64, "fp8", 507, exact=True)
    sc = wl["kv_scales"].copy()
    rng = np.random.default_rng(5070)
    for b in rng.choice(12000 // 64, size=40, replace=False):
        sc[64 * b + rng.integers(0, 64)] = -2.0
    wl = dict(wl, kv_scales=sc)
    d = to_device(wl)
    scan = run_gpu(wl, d, options=opts(path=SCAN))
    pr = run_gpu(wl, d, options=opts(path=PRUNE))
    assert _same(pr, scan)
    rep = parity(wl, pr[0], pr[1], "exact")
    assert rep["ok"], rep


def test_prune_with_short_and_empty_windows():
    wl = workloads.blocky(48, 9000, 200, "bf16", 508, exact=True)
    ks = wl["ks"].copy()
    ke = wl["ke"].copy()
    ks[:8], ke[:8] = 500, 500                      # empty
    ks[8:16], ke[8:16] = 1000, 1000 + np.arange(8) * 20  # shorter than topk
    ks[16:24] = np.arange(8) * 1000                # ragged starts
    wl = dict(wl, ks=ks, ke=ke)
    d = to_device(wl)
    scan = run_gpu(wl, d, options=opts(path=SCAN))
    pr = run_gpu(wl, d, options=opts(path=PRUNE))
    assert _same(pr, scan)
    rep = parity(wl, pr[0], pr[1], "exact")
    assert rep["ok"], rep
