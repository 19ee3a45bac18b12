"""Loader for the hand-worked examples in tests/golden/hand_examples.json."""
import json
import os

import numpy as np

import workloads

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def load():
    with open(PATH) as f:
        return json.load(f)["examples"]


def _val(v):
    return -np.inf if v == "-inf" else float(v)


def build(ex, case, dtype):
    """Full-shape operands (H=32, d=128) for one example case, one query row."""
    qf = np.zeros((1, workloads.HEADS, workloads.DIM), np.float32)
    for h, d, v in ex["q"]:
        qf[0, h, d] = v
    w = np.zeros((1, workloads.HEADS), np.float32)
    for h, v in ex["weights"]:
        w[0, h] = v
    kf = np.zeros((ex["num_kv"], workloads.DIM), np.float32)
    for s, d, v in ex["kv"]:
        kf[s, d] = v
    q = workloads._quantize(qf, dtype)
    kv = workloads._quantize(kf, dtype)
    sc = np.asarray(ex["kv_scales"], np.float32)
    ks = np.array([case["ks"]], np.int32)
    ke = np.array([case["ke"]], np.int32)
    exp_idx = np.array([case["idx"]], np.int32)
    exp_val = np.array([[_val(v) for v in case["val"]]], np.float32)
    return dict(q=q, kv=kv, dtype=dtype, kv_scales=sc, weights=w, ks=ks, ke=ke,
                topk=case["topk"], name=ex["name"]), exp_idx, exp_val


def all_cases():
    for ex in load():
        for ci, case in enumerate(ex["cases"]):
            for dtype in ("fp8", "bf16"):
                yield f"{ex['name']}-{ci}-{dtype}", ex, case, dtype
