"""options.validate: the device check of the data preconditions (windows
inside [0, num_kv] with ks <= ke, no NaN / infinity codes in q and kv, finite
weights, finite non-negative key scales, page ids inside the pool).  Clean
inputs give the same bits as without the check and no flags; each planted
violation sets its own bit and fails the call before a scoring kernel runs,
leaving the outputs untouched.
"""
import numpy as np
import pytest

import workloads

from gpu_util import opts, run_gpu, to_device

pytestmark = pytest.mark.gpu

ERR_INVALID_ARGUMENT = 1  # FLASHTOPK_ERR_INVALID_ARGUMENT


def _say(*a):
    print(*a, flush=True)


def _info():
    import sparse_attention_indexer_fp8_amd as ftk

    return ftk.flashtopk_get_last_info()


def _call(wl, d):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    T, k = wl["q"].shape[0], wl["topk"]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((T, k), 3.0, dtype=torch.float32, device="cuda")
    err = None
    try:
        ftk.flashtopk_select_ex(d["q"], d["kv"], d["kv_scales"], d["weights"], d["ks"], d["ke"], k, idx, val,
                                options=opts(validate=1))
    except ftk.FlashTopKError as e:
        err = e
    torch.cuda.synchronize()
    return err, idx.cpu().numpy(), val.cpu().numpy()


def _copy(wl):
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in wl.items()}


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_clean_inputs_same_outputs_no_flags(dt):
    wl = workloads.integer(20, 3000, 64, dt, 1201)
    _say("validate clean", dt)
    d = to_device(wl)
    ref = run_gpu(wl, d)
    err, idx, val = _call(wl, d)
    assert err is None
    assert np.array_equal(ref[0], idx) and np.array_equal(ref[1].view(np.uint32), val.view(np.uint32))
    info = _info()
    assert info["invalid"] == 0 and info["status"] == 0


@pytest.mark.parametrize("dt", ["fp8", "bf16"])
def test_each_violation_sets_its_bit_and_fails(dt):
    import sparse_attention_indexer_fp8_amd as ftk

    wl = workloads.integer(20, 3000, 64, dt, 1202)
    nan_code = 0x7F if dt == "fp8" else 0x7FC0   # E4M3 NaN; BF16 quiet NaN
    big_code = 0xFF if dt == "fp8" else 0xFF80   # E4M3 negative NaN; BF16 -infinity
    cases = [
        ("q", ftk.FLASHTOPK_INVALID_Q, lambda w: w["q"].__setitem__((3, 7, 11), nan_code)),
        ("q last", ftk.FLASHTOPK_INVALID_Q, lambda w: w["q"].__setitem__((19, 31, 127), big_code)),
        ("kv", ftk.FLASHTOPK_INVALID_KV, lambda w: w["kv"].__setitem__((2500, 100), big_code)),
        ("kv last", ftk.FLASHTOPK_INVALID_KV, lambda w: w["kv"].__setitem__((2999, 127), nan_code)),
        ("weight inf", ftk.FLASHTOPK_INVALID_WEIGHT, lambda w: w["weights"].__setitem__((5, 30), np.inf)),
        ("weight nan", ftk.FLASHTOPK_INVALID_WEIGHT, lambda w: w["weights"].__setitem__((19, 31), np.nan)),
        ("scale neg", ftk.FLASHTOPK_INVALID_SCALE, lambda w: w["kv_scales"].__setitem__(17, -1.0)),
        ("scale nan", ftk.FLASHTOPK_INVALID_SCALE, lambda w: w["kv_scales"].__setitem__(2999, np.nan)),
        ("window past end", ftk.FLASHTOPK_INVALID_WINDOW, lambda w: w["ke"].__setitem__(9, 3001)),
        ("window negative", ftk.FLASHTOPK_INVALID_WINDOW, lambda w: w["ks"].__setitem__(0, -1)),
        ("window reversed", ftk.FLASHTOPK_INVALID_WINDOW,
         lambda w: (w["ks"].__setitem__(19, 50), w["ke"].__setitem__(19, 40))),
    ]
    for name, bit, plant in cases:
        w2 = _copy(wl)
        plant(w2)
        _say("validate", dt, name)
        err, idx, val = _call(w2, to_device(w2))
        assert err is not None and err.status == ERR_INVALID_ARGUMENT, name
        info = _info()
        assert info["status"] == ERR_INVALID_ARGUMENT and info["invalid"] == bit, (name, info["invalid"])
        assert (idx == -7).all() and (val == 3.0).all(), name  # nothing written
    # several at once: every bit
    w2 = _copy(wl)
    for _, _, plant in cases:
        plant(w2)
    err, _, _ = _call(w2, to_device(w2))
    allbits = (ftk.FLASHTOPK_INVALID_Q | ftk.FLASHTOPK_INVALID_KV | ftk.FLASHTOPK_INVALID_WEIGHT
               | ftk.FLASHTOPK_INVALID_SCALE | ftk.FLASHTOPK_INVALID_WINDOW)
    assert err is not None and _info()["invalid"] == allbits
    # the stream is usable afterwards and the last info is the new call's
    d = to_device(wl)
    ref = run_gpu(wl, d)
    err, idx, _ = _call(wl, d)
    assert err is None and np.array_equal(idx, ref[0]) and _info()["invalid"] == 0


def test_largest_finite_codes_are_valid():
    # E4M3 +-448 (S.1111.110) and BF16 +-max finite are not flagged.  A planted
    # window violation stops each call before scoring (such codes can overflow
    # the score), so the flags alone are checked: only the window bit is set.
    import sparse_attention_indexer_fp8_amd as ftk

    for dt, code in (("fp8", 0x7E), ("fp8", 0xFE), ("bf16", 0x7F7F), ("bf16", 0xFF7F)):
        wl = workloads.integer(4, 300, 16, dt, 1205)
        wl["kv"][123, 45] = code
        wl["q"][1, 2, 3] = code
        wl["ke"][2] = 301
        _say("validate max finite", dt, hex(code))
        err, _, _ = _call(wl, to_device(wl))
        assert err is not None and _info()["invalid"] == ftk.FLASHTOPK_INVALID_WINDOW


def test_paged_page_id_out_of_range_fails():
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    wl = workloads.integer(12, 1000, 32, "fp8", 1204)
    d = to_device(wl)
    ps, S = 16, 1000
    nblk = (S + ps - 1) // ps
    table = torch.arange(nblk, dtype=torch.int32, device="cuda")
    pool = torch.zeros((nblk * ps, 128), dtype=d["kv"].dtype, device="cuda")
    pool[:S] = d["kv"]
    spool = torch.ones(nblk * ps, dtype=torch.float32, device="cuda")
    spool[:S] = d["kv_scales"]
    ref = run_gpu(wl, d)
    for bad in (None, nblk + 5, -1):
        if bad is not None:
            table[3] = bad
        _say("validate paged", bad)
        idx = torch.full((12, 32), -7, dtype=torch.int32, device="cuda")
        val = torch.empty((12, 32), dtype=torch.float32, device="cuda")
        call = lambda: ftk.flashtopk_select_paged(d["q"], pool.view(nblk, ps, 128), spool.view(nblk, ps), table,
                                                  S, d["weights"], d["ks"], d["ke"], 32, idx, val,
                                                  options=opts(validate=1))
        if bad is None:
            call()
            torch.cuda.synchronize()
            assert _info()["invalid"] == 0
            assert np.array_equal(idx.cpu().numpy(), ref[0])
        else:
            with pytest.raises(ftk.FlashTopKError):
                call()
            torch.cuda.synchronize()
            assert _info()["invalid"] == ftk.FLASHTOPK_INVALID_PAGE
            assert (idx.cpu().numpy() == -7).all()
