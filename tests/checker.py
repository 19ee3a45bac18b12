"""Parity checker: compares a selection against the oracle's.

Two modes (FlashTopK README, "What you can do": exact and deterministic):
  * exact      -- indices and binary32 values bit-identical.  Used where every
                  binary32 partial sum is exact (integer-valued inputs), so the
                  oracle's rounded binary64 score equals any exact binary32
                  evaluation.
  * tolerance  -- for random inputs: with tol = rel_tol * max|I_row| over the
                  row's window, every returned value is within tol of the
                  oracle's score of that index, and every index in the
                  symmetric difference of the two selections scores within tol
                  of the oracle's k-th score.

Both modes also check the structure that holds at any size: min(topk, L)
valid entries, unique, inside [ks, ke), strictly ordered by (value desc,
index asc), then -1 / -inf padding.  The retrieval precision
p = |sel & oracle| / k (overlap of two top-k sets) is reported per row.
"""
from __future__ import annotations

import numpy as np


def structure_failures(idx, val, ks, ke, topk):
    """Structural problems of one row's output (no oracle needed)."""
    out = []
    L = max(0, int(ke) - int(ks))
    k = min(int(topk), L)
    idx = np.asarray(idx)
    val = np.asarray(val, dtype=np.float32)
    sel = idx[:k].astype(np.int64)
    if np.any(sel < ks) or np.any(sel >= ke):
        out.append("index outside window")
    if np.unique(sel).size != k:
        out.append("duplicate index")
    if np.any(idx[k:] != -1):
        out.append("padding index not -1")
    if np.any(~(np.isneginf(val[k:]))):
        out.append("padding value not -inf")
    if not np.all(np.isfinite(val[:k])):
        out.append("non-finite value in selection")
    if k > 1:
        v0, v1 = val[:k - 1], val[1:k]
        i0, i1 = sel[:-1], sel[1:]
        ok = (v0 > v1) | ((v0 == v1) & (i0 < i1))
        if not np.all(ok):
            out.append("not ordered by (value desc, index asc)")
    return out


def exact_row(idx, val, o_idx, o_val):
    f = []
    if not np.array_equal(np.asarray(idx), np.asarray(o_idx)):
        f.append("indices differ")
    a = np.asarray(val, dtype=np.float32).view(np.uint32)
    b = np.asarray(o_val, dtype=np.float32).view(np.uint32)
    if not np.array_equal(a, b):
        f.append("values differ")
    return f


def tolerance_row(idx, val, o_idx, o_score, all_scores, ks, ke, topk, rel_tol=1e-3, floor=0.0):
    """Returns (failures, precision p).  ``floor``: an absolute lower limit
    of the row's tolerance (the arithmetic's own error bound), or 0."""
    f = []
    L = max(0, int(ke) - int(ks))
    k = min(int(topk), L)
    if k == 0:
        return f, 1.0
    win = all_scores[int(ks):int(ke)]
    tol = max(rel_tol * float(np.max(np.abs(win))), float(floor))
    sel = np.asarray(idx[:k], dtype=np.int64)
    osel = np.asarray(o_idx[:k], dtype=np.int64)
    if np.any(sel < ks) or np.any(sel >= ke):
        return ["index outside window"], 0.0
    got = np.asarray(val[:k], dtype=np.float64)
    ref = all_scores[sel]
    bad = np.abs(got - ref) > tol
    if np.any(bad):
        j = int(np.argmax(bad))
        f.append(f"value of index {sel[j]} is {got[j]!r}, oracle {ref[j]!r}, tol {tol:.3g}")
    kth = float(o_score[k - 1])
    diff = np.setxor1d(sel, osel)
    if diff.size:
        far = np.abs(all_scores[diff] - kth) > tol
        if np.any(far):
            s = int(diff[np.argmax(far)])
            f.append(f"index {s} differs with score {all_scores[s]!r} far from k-th {kth!r}")
    p = np.intersect1d(sel, osel).size / k
    return f, p


def check(idx, val, ks, ke, topk, *, o_idx, o_val=None, o_score=None, all_scores=None,
          rows=None, mode="exact", rel_tol=1e-3, floor=None, max_report=5):
    """Check a [n, topk] selection against oracle outputs for the same rows.

    ``rows`` maps each output row to its query index (for ks/ke); None means
    rows 0..n-1.  ``floor`` (tolerance mode, indexed like ``rows``): per-row
    absolute lower limits of the tolerance, or None.  Returns a report dict with failures (first few), the number
    of failing rows, the mean precision and the bit-identical row fraction.
    """
    idx = np.asarray(idx)
    val = np.asarray(val, dtype=np.float32)
    n = idx.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    failures, nbad, ps, same = [], 0, [], 0
    for r in range(n):
        t = int(rows[r])
        fr = structure_failures(idx[r], val[r], ks[t], ke[t], topk)
        if mode == "exact":
            fr += exact_row(idx[r], val[r], o_idx[r], o_val[r])
            p = 1.0 if not fr else np.intersect1d(idx[r][idx[r] >= 0], o_idx[r][o_idx[r] >= 0]).size / max(1, min(topk, int(ke[t]) - int(ks[t])))
        else:
            ft, p = tolerance_row(idx[r], val[r], o_idx[r], o_score[r], all_scores[r], ks[t], ke[t],
                                  topk, rel_tol, 0.0 if floor is None else floor[r])
            fr += ft
        if o_val is not None and np.array_equal(idx[r], o_idx[r]) and np.array_equal(
                val[r].view(np.uint32), np.asarray(o_val[r], np.float32).view(np.uint32)):
            same += 1
        ps.append(p)
        if fr:
            nbad += 1
            if len(failures) < max_report:
                failures.append(f"row {t}: " + "; ".join(fr))
    return dict(ok=nbad == 0, bad_rows=nbad, failures=failures,
                precision=float(np.mean(ps)) if ps else 1.0,
                identical_rows=same / max(1, n))
