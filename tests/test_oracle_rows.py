"""Pins of the oracle's top-k over materialized score rows (DeepSelect README,
"Usage" and "Variable-length rows": each row keeps its topk largest values
among its first end[r] entries; short rows are padded with fill values).

The oracle sorts with the C library's qsort; here it is checked against
brute force over all subsets of tiny rows, against numpy's lexsort on larger
rows, and on hand-built tie, signed-zero and padding cases.
"""
import itertools

import numpy as np
import pytest

import oracle


def _bruteforce(vals, k):
    """Best k-subset under (value desc, index asc): the sorted tuple of
    (-value, index) pairs is lexicographically smallest."""
    n = len(vals)
    k = min(k, n)
    best = None
    for sub in itertools.combinations(range(n), k):
        key = sorted((-float(vals[i]) + 0.0, i) for i in sub)
        if best is None or key < best:
            best = key
    return [i for _, i in best]


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_tiny_rows(seed):
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 10))
    vals = rng.integers(-3, 4, size=n).astype(np.float32)  # many ties
    vals[rng.random(n) < 0.2] = -0.0
    for k in range(1, n + 3):
        idx, val = oracle.topk_rows(vals[None, :], k)
        want = _bruteforce(vals, k)
        assert list(idx[0, :len(want)]) == want
        assert np.all(idx[0, len(want):] == -1)
        assert np.all(np.isneginf(val[0, len(want):]))
        assert np.array_equal(val[0, :len(want)], np.abs(vals[want]) * np.sign(vals[want]) + 0.0)


def _lexsort_topk(x, k, ends):
    rows, cols = x.shape
    idx = np.full((rows, k), -1, np.int32)
    val = np.full((rows, k), -np.inf, np.float32)
    for r in range(rows):
        n = cols if ends is None else int(np.clip(ends[r], 0, cols))
        v = x[r, :n].astype(np.float64) + 0.0  # -0 -> +0
        order = np.lexsort((np.arange(n), -v))[:k]
        idx[r, :len(order)] = order
        val[r, :len(order)] = v[order]
    return idx, val


def test_matches_lexsort_float32_with_ends():
    rng = np.random.default_rng(710)
    x = rng.standard_normal((40, 3000)).astype(np.float32)
    x[:, ::7] = np.round(x[:, ::7])  # ties
    ends = rng.integers(-5, 3100, size=40).astype(np.int32)
    got = oracle.topk_rows(x, 300, ends=ends)
    want = _lexsort_topk(x, 300, ends)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))


def test_matches_lexsort_bf16():
    import torch

    rng = np.random.default_rng(711)
    xf = rng.standard_normal((16, 2000)).astype(np.float32)
    codes = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    decoded = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = oracle.topk_rows(codes, 100)
    want = _lexsort_topk(decoded, 100, None)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])


def test_signed_zero_and_padding_cases():
    x = np.array([[0.0, -0.0, -1.0, 0.0],
                  [5.0, 5.0, 5.0, 5.0]], np.float32)
    idx, val = oracle.topk_rows(x, 3, ends=np.array([4, 2], np.int32))
    # +0 and -0 are equal: indices 0, 1, 3 by position; -0 is written +0
    assert list(idx[0]) == [0, 1, 3]
    assert np.array_equal(val[0].view(np.uint32), np.zeros(3, np.float32).view(np.uint32))
    # end 2: the two leading entries, then padding
    assert list(idx[1]) == [0, 1, -1]
    assert val[1, 2] == -np.inf
    idx, _ = oracle.topk_rows(x, 2, ends=np.array([0, 9], np.int32))  # empty row; end clamped to cols
    assert list(idx[0]) == [-1, -1] and list(idx[1]) == [0, 1]


def test_nan_entry_rejected():
    x = np.array([[1.0, np.nan]], np.float32)
    with pytest.raises(ValueError):
        oracle.topk_rows(x, 1)
