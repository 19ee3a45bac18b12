"""Helpers of the GPU tests: move a workload to the device, run the HIP path
through the C ABI, run the oracle, check parity."""
import numpy as np

import oracle
import workloads

import checker


def to_device(wl, dev="cuda:0"):
    import torch

    if wl["dtype"] == "fp8":
        q = torch.from_numpy(wl["q"]).to(dev).view(torch.float8_e4m3fn)
        kv = torch.from_numpy(wl["kv"]).to(dev).view(torch.float8_e4m3fn)
    else:
        q = torch.from_numpy(wl["q"].view(np.int16)).to(dev).view(torch.bfloat16)
        kv = torch.from_numpy(wl["kv"].view(np.int16)).to(dev).view(torch.bfloat16)
    sc = None if wl["kv_scales"] is None else torch.from_numpy(wl["kv_scales"]).to(dev)
    return dict(q=q, kv=kv, kv_scales=sc, weights=torch.from_numpy(wl["weights"]).to(dev),
                ks=torch.from_numpy(wl["ks"]).to(dev), ke=torch.from_numpy(wl["ke"]).to(dev))


def run_gpu(wl, d=None, options=None, topk=None):
    import torch

    import sparse_attention_indexer_fp8_amd as ftk

    d = d or to_device(wl)
    k = topk or wl["topk"]
    idx, val = ftk.select(d["q"], d["kv"], d["weights"], d["ks"], d["ke"], d["kv_scales"], topk=k,
                          return_scores=True, options=options)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def run_oracle(wl, rows=None, topk=None):
    k = topk or wl["topk"]
    return oracle.select(wl["q"], wl["kv"], wl["dtype"], wl["kv_scales"], wl["weights"], wl["ks"], wl["ke"],
                         k, rows=rows, all_scores=True)


def parity(wl, idx, val, mode, rows=None, ref=None, topk=None, floor=None):
    k = topk or wl["topk"]
    o = ref if ref is not None else run_oracle(wl, rows=rows, topk=k)
    if rows is not None:
        idx, val = idx[rows], val[rows]
    rep = checker.check(idx, val, wl["ks"], wl["ke"], k, o_idx=o[0], o_val=o[1], o_score=o[2],
                        all_scores=o[3], rows=rows, mode=mode, floor=floor)
    return rep


# The FP8 matrix cores do not round a 128-term dot product correctly: on
# MI355X its error reaches 2^-16.5 of sum_d |q_d k_d| (measured by
# test_gpu_error_bound.py).  A weighted head sum inherits at most
# sum_h |w_h| times that.  This is the per-row floor, with a 2^1.5 margin,
# below which no FP8 score can be resolved, whatever the summation.
FP8_DOT_REL = 2.0 ** -15


def fp8_dot_floor(wl):
    """Per row: FP8_DOT_REL * max over the window of sigma_s *
    sum_h |w[t,h]| sum_d |q[t,h,d] k[s,d]| (0 for an empty window)."""
    import torch

    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double().numpy()
    q, k = np.abs(dec(wl["q"])), np.abs(dec(wl["kv"]))
    a = np.einsum("th,thd->td", np.abs(wl["weights"].astype(np.float64)), q)
    m = a @ k.T
    if wl["kv_scales"] is not None:
        m = m * wl["kv_scales"].astype(np.float64)[None, :]
    out = np.zeros(q.shape[0])
    for t in range(q.shape[0]):
        lo, hi = int(wl["ks"][t]), int(wl["ke"][t])
        if hi > lo:
            out[t] = FP8_DOT_REL * m[t, lo:hi].max()
    return out


def opts(**kw):
    import sparse_attention_indexer_fp8_amd as ftk

    o = ftk.Options()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def sample_rows(T, n_mid=24, edge=8, seed=0):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(edge, max(edge + 1, T - edge)), size=min(n_mid, max(0, T - 2 * edge)),
                     replace=False)
    rows = np.unique(np.concatenate([np.arange(min(edge, T)), np.arange(max(0, T - edge), T), mid]))
    return rows.astype(np.int64)
