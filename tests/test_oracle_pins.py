"""Pins of the oracle to facts outside itself (CPU only).

* operand decode against the OCP E4M3FN / bfloat16 definitions (spot values)
  and torch's CPU casts (a library routine), for every code;
* the hand-worked examples in tests/golden (FlashTopK README, "Quick start"
  equation and "What you can do" tie rule);
* a special case that reduces to a library matrix-vector product;
* brute force over all subsets on tiny windows, in exact rational arithmetic;
* the closed form for windows no longer than topk.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import numpy_ref

import golden_cases


# ---------------------------------------------------------------- decode ----

def test_fp8_decode_spot_values_from_format_definition():
    # s.eeee.mmm, bias 7: 0x38 = 2^0, 0x7E = 1.75 * 2^8, 0x08 = 2^-6 (smallest
    # normal), 0x01 = 2^-9 (smallest subnormal), 0x44 = 1.5 * 2^1, 0x48 = 2^2.
    spots = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x44: 3.0,
             0x48: 4.0, 0x00: 0.0, 0xB8: -1.0, 0x07: 7 * 2.0 ** -9, 0xFE: -448.0}
    for code, want in spots.items():
        assert oracle.decode_e4m3fn([code])[0] == want, hex(code)
    assert np.isnan(oracle.decode_e4m3fn([0x7F])[0]) and np.isnan(oracle.decode_e4m3fn([0xFF])[0])
    assert np.signbit(oracle.decode_e4m3fn([0x80])[0])


def test_fp8_decode_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    twin = numpy_ref.decode_e4m3fn(codes)
    assert np.array_equal(twin[ok], ref[ok])


def test_bf16_decode_all_codes_match_torch_cast():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    twin = numpy_ref.decode_bf16(codes)
    assert np.array_equal(twin[ok], ref[ok])


# ------------------------------------------------------- golden examples ----

@pytest.mark.parametrize("cid,ex,case,dtype", list(golden_cases.all_cases()),
                         ids=[c[0] for c in golden_cases.all_cases()])
def test_hand_worked_examples(cid, ex, case, dtype):
    wl, exp_idx, exp_val = golden_cases.build(ex, case, dtype)
    idx, val, sc, allsc = oracle.select(wl["q"], wl["kv"], dtype, wl["kv_scales"], wl["weights"],
                                        wl["ks"], wl["ke"], wl["topk"], all_scores=True)
    assert np.array_equal(idx, exp_idx)
    assert np.array_equal(val.view(np.uint32), exp_val.view(np.uint32))  # +0 written, not -0
    # every listed score, straight from the scorer
    s = oracle.scores(wl["q"], wl["kv"], dtype, wl["kv_scales"], wl["weights"], 0, 0, ex["num_kv"])
    assert np.array_equal(s, np.asarray(ex["scores"], np.float64))
    for reading, vals in ex.get("wrong_readings", {}).items():
        assert not np.array_equal(s, np.asarray(vals)), reading


def test_signed_zero_example_really_produces_both_zeros():
    ex = [e for e in golden_cases.load() if e["name"] == "C_signed_zero"][0]
    wl, _, _ = golden_cases.build(ex, ex["cases"][0], "fp8")
    s = oracle.scores(wl["q"], wl["kv"], "fp8", wl["kv_scales"], wl["weights"], 0, 0, 2)
    assert s[0] == 0 and np.signbit(s[0]) and s[1] == 0 and not np.signbit(s[1])


# ------------------------------------------------- library special case ----

@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_single_head_positive_reduces_to_matvec(dtype):
    """One active head with weight 1, unit scales and all dot products positive:
    I[t, s] = q[t,0] . kv[s], a plain matrix-vector product."""
    rng = np.random.default_rng(11)
    T, S = 3, 50
    qf = np.zeros((T, 32, 128), np.float32)
    qf[:, 0, :] = np.abs(rng.standard_normal((T, 128))) + 0.1
    kf = np.abs(rng.standard_normal((S, 128))).astype(np.float32) + 0.1
    q, kv = workloads._quantize(qf, dtype), workloads._quantize(kf, dtype)
    w = np.zeros((T, 32), np.float32)
    w[:, 0] = 1.0
    tdt = torch.float8_e4m3fn if dtype == "fp8" else torch.bfloat16
    view = (lambda a: torch.from_numpy(a).view(tdt)) if dtype == "fp8" else \
        (lambda a: torch.from_numpy(a.view(np.int16)).view(tdt))
    qd = view(q).to(torch.float64).numpy()
    kd = view(kv).to(torch.float64).numpy()
    for t in range(T):
        got = oracle.scores(q, kv, dtype, None, w, t, 0, S)
        want = kd @ qd[t, 0]
        np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)


# ------------------------------------------------------------ brute force --

def _exact_scores(wl, t):
    """Exact rational scores of row t (integer operands, dyadic w and sigma)."""
    qd = numpy_ref.decode(wl["q"], wl["dtype"])[t]
    kd = numpy_ref.decode(wl["kv"], wl["dtype"])
    out = []
    for s in range(kd.shape[0]):
        acc = Fraction(0)
        for h in range(32):
            x = sum(int(a) * int(b) for a, b in zip(qd[h], kd[s]))
            if x > 0:
                acc += Fraction(float(wl["weights"][t, h])) * x
        out.append(Fraction(float(wl["kv_scales"][s])) * acc)
    return out


def _best_subset(scores, lo, hi, k):
    """Enumerate every k-subset of [lo, hi) and keep the best one under the
    order: compare the (score desc, index asc) sorted lists element by element."""
    best = None
    for sub in itertools.combinations(range(lo, hi), k):
        key = sorted(sub, key=lambda s: (-scores[s], s))
        rank = [(-scores[s], s) for s in key]
        if best is None or rank < best[0]:
            best = (rank, key)
    return best[1] if best else []


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_subsets_tiny_windows(seed):
    rng = np.random.default_rng(100 + seed)
    S = 12
    T = 4
    wl = workloads.integer(T, S, 1, "fp8", 200 + seed, windows="full")
    # sparsify so the exact rational evaluation stays fast and ties are common
    mask = rng.random(wl["q"].shape) < 0.03
    q = np.where(mask, wl["q"], 0).astype(np.uint8)
    kmask = rng.random(wl["kv"].shape) < 0.3
    kv = np.where(kmask, wl["kv"], 0).astype(np.uint8)
    wl = dict(wl, q=q, kv=kv)
    for t in range(T):
        ex = _exact_scores(wl, t)
        lo = int(rng.integers(0, 4))
        hi = int(rng.integers(lo, S + 1))
        for k in range(1, hi - lo + 3):
            ks = np.full(T, lo, np.int32)
            ke = np.full(T, hi, np.int32)
            idx, val, _, _ = oracle.select(wl["q"], wl["kv"], "fp8", wl["kv_scales"], wl["weights"],
                                           ks, ke, k, rows=[t])
            best = _best_subset(ex, lo, hi, min(k, hi - lo))
            assert list(idx[0][: len(best)]) == best
            assert np.all(idx[0][len(best):] == -1)
            for j, s in enumerate(best):
                assert val[0][j] == np.float32(float(ex[s]))


# ------------------------------------------------------------ closed form --

@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_window_not_longer_than_topk_returns_whole_window_sorted(dtype):
    wl = workloads.gaussian(9, 40, 16, dtype, 21)
    ks = np.arange(9, dtype=np.int32) * 3
    ke = ks + np.arange(9, dtype=np.int32) + 5   # lengths 5..13, all <= 16
    idx, val, sc, allsc = oracle.select(wl["q"], wl["kv"], dtype, wl["kv_scales"], wl["weights"],
                                        ks, ke, 16, all_scores=True)
    for t in range(9):
        L = ke[t] - ks[t]
        win = np.arange(ks[t], ke[t])
        assert sorted(idx[t, :L].tolist()) == win.tolist()
        assert np.all(idx[t, L:] == -1) and np.all(np.isneginf(val[t, L:]))
        s = allsc[t, idx[t, :L]]
        assert np.all(np.diff(s) <= 0)
