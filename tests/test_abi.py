"""The C-ABI library loads and exports every entry point include/flashtopk.h
declares; argument checks that need no device memory (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_attention_indexer_fp8_amd as ftk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashtopk.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flashtopk_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ftk.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return ftk.load_library()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(ftk.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings_and_version(lib):
    assert ftk.flashtopk_status_string(0) == "ok"
    assert ftk.flashtopk_status_string(1) == "invalid argument"
    assert ftk.flashtopk_status_string(2) == "unsupported dtype"
    assert ftk.flashtopk_status_string(999) == "unknown status"
    assert ftk.flashtopk_version() >= 100


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (FLASHTOPK_\w+) (-?\d+)", text))
    assert int(consts["FLASHTOPK_FP8_E4M3"]) == ftk.FLASHTOPK_FP8_E4M3
    assert int(consts["FLASHTOPK_BF16"]) == ftk.FLASHTOPK_BF16
    assert int(consts["FLASHTOPK_MAX_TOPK"]) == ftk.MAX_TOPK
    assert int(consts["FLASHTOPK_PATH_RECOVER"]) == ftk.PATH_RECOVER
    assert int(consts["FLASHTOPK_PATH_FUSED"]) == ftk.PATH_FUSED
    assert int(consts["FLASHTOPK_SCORES_F32"]) == ftk.FLASHTOPK_SCORES_F32
    assert int(consts["FLASHTOPK_SCORES_BF16"]) == ftk.FLASHTOPK_SCORES_BF16
    assert int(consts["FLASHTOPK_OUT_INDEX_ORDER"]) == ftk.FLASHTOPK_OUT_INDEX_ORDER
    assert int(consts["FLASHTOPK_OUT_INT64"]) == ftk.FLASHTOPK_OUT_INT64
    for name in ("WINDOW", "Q", "KV", "WEIGHT", "SCALE", "PAGE"):
        assert int(consts["FLASHTOPK_INVALID_" + name]) == getattr(ftk, "FLASHTOPK_INVALID_" + name)


def test_options_and_info_layout_match_header():
    # sizes of the C structs as laid out by the platform ABI
    assert ctypes.sizeof(ftk.Options) == 40
    assert ctypes.sizeof(ftk.Info) == 4 + 4 + 8 * 10 + 4 + 4 + 6 * 4 + 4 + 4 + 8  # invalid, padding, candidates


def test_struct_layout_matches_the_c_compiler(tmp_path):
    # The binding's ctypes structs against the header as a C compiler lays
    # it out: sizes and the offset of every field.
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "flashtopk.h"', "int main(void) {"]
    for cname, py in (("flashtopk_options", ftk.Options), ("flashtopk_info", ftk.Info)):
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in (("flashtopk_options", ftk.Options), ("flashtopk_info", ftk.Info)):
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def _call(lib, **kw):
    args = dict(q=None, kv=None, kv_scales=None, weights=None, ks=None, ke=None, num_q=0, num_kv=0,
                dtype=0, topk=1, out_idx=None, out_val=None, stream=None)
    args.update(kw)
    return lib.flashtopk_select(*[args[k] for k in ("q", "kv", "kv_scales", "weights", "ks", "ke", "num_q",
                                                    "num_kv", "dtype", "topk", "out_idx", "out_val",
                                                    "stream")])


def test_argument_errors_without_device(lib):
    # these return before any device work
    assert _call(lib, dtype=7) == 2
    assert _call(lib, topk=0) == 1
    assert _call(lib, topk=4097) == 1
    assert _call(lib, num_q=-1) == 1
    assert _call(lib, num_kv=1 << 31) == 1
    assert _call(lib, num_q=0, topk=5) == 0                  # empty call is a no-op
    assert _call(lib, num_q=3, topk=5) == 1                  # null required pointers
    assert lib.flashtopk_reserve(-1, 0, 1, 0, None) == 1
    assert lib.flashtopk_reserve(1, 1, 1, 3, None) == 2
    assert lib.flashtopk_reserve(1, 1 << 31, 1, 0, None) == 1
    assert lib.flashtopk_get_last_info(None, None) == 1
    assert lib.flashtopk_get_last_recovered(None, None, 0, None) == 1     # no count pointer
    n = ctypes.c_int64(0)
    assert lib.flashtopk_get_last_recovered(None, None, 5, ctypes.byref(n)) == 1  # rows missing
    tf = ctypes.c_double(1.0)
    assert lib.flashtopk_probe_mfma(7, 10, None, ctypes.byref(tf)) == 1          # no such dtype
    assert lib.flashtopk_probe_mfma(0, 0, None, ctypes.byref(tf)) == 1           # no rounds
    assert lib.flashtopk_probe_mfma(0, 10, None, None) == 1                      # no output


def test_misaligned_operands_rejected(lib):
    buf = (ctypes.c_uint8 * 64)()
    base = ctypes.addressof(buf)
    odd = base + (1 if base % 16 else 1)
    p = ctypes.c_void_p(odd)
    ok = ctypes.c_void_p(base + (-base) % 16)
    assert _call(lib, q=p, kv=ok, weights=ok, ks=ok, ke=ok, out_idx=ok, num_q=1, num_kv=1) == 1


def _rows(lib, **kw):
    args = dict(x=None, dtype=1, rows=0, cols=0, stride=0, ends=None, topk=1, out_idx=None, out_val=None,
                nan_flag=None, flags=0, stream=None)
    args.update(kw)
    return lib.flashtopk_topk_rows(*[args[k] for k in ("x", "dtype", "rows", "cols", "stride", "ends", "topk",
                                                       "out_idx", "out_val", "nan_flag", "flags", "stream")])


def test_topk_rows_argument_errors_without_device(lib):
    buf = (ctypes.c_uint8 * 64)()
    base = ctypes.addressof(buf)
    ok = ctypes.c_void_p(base + (-base) % 16)
    odd = ctypes.c_void_p(base + (-base) % 16 + 2)
    assert _rows(lib, dtype=2) == 2
    assert _rows(lib, topk=0) == 1
    assert _rows(lib, topk=4097) == 1
    assert _rows(lib, rows=-1) == 1
    assert _rows(lib, cols=1 << 31) == 1
    assert _rows(lib, rows=0, topk=5) == 0                                   # no-op
    assert _rows(lib, rows=2, cols=8, stride=8, x=ok) == 1                  # null out_idx
    assert _rows(lib, rows=2, cols=8, stride=8, out_idx=ok) == 1            # null x
    assert _rows(lib, rows=2, cols=8, stride=8, x=odd, out_idx=ok) == 1     # misaligned x
    assert _rows(lib, rows=2, cols=8, stride=4, x=ok, out_idx=ok) == 1      # stride < cols
    assert _rows(lib, rows=2, cols=9, stride=9, x=ok, out_idx=ok) == 1      # 18-byte BF16 stride
    assert _rows(lib, rows=2, cols=6, stride=6, x=ok, out_idx=ok, dtype=0) == 1  # 24-byte f32 stride
    assert _rows(lib, rows=2, cols=8, stride=8, x=ok, out_idx=ok, flags=4) == 1   # unknown output flag


def test_select_paged_argument_errors_without_device(lib):
    buf = (ctypes.c_uint8 * 64)()
    base = ctypes.addressof(buf)
    ok = ctypes.c_void_p(base + (-base) % 16)

    def call(**kw):
        a = dict(q=ok, pages=ok, spages=None, table=ok, page_size=64, num_pages=4, w=ok, ks=ok, ke=ok, num_q=1,
                 num_kv=100, dtype=0, topk=1, oi=ok, ov=None, stream=None, opt=None)
        a.update(kw)
        return lib.flashtopk_select_paged(*a.values())

    assert call(dtype=5) == 2
    assert call(page_size=0) == 1
    assert call(num_pages=-1) == 1
    assert call(topk=0) == 1
    assert call(num_q=0) == 0                  # no-op
    assert call(table=None) == 1               # keys without a block table
    assert call(num_pages=0) == 1              # keys without pages
    assert call(pages=ctypes.c_void_p(ok.value + 2)) == 1  # misaligned pool


# ------------------------------------------------- windows_from_cu_seqlens ---

def _windows_by_definition(cu_q, cu_k):
    """Bottom-right aligned causal windows, row by row (README "Usage"
    windows_from_cu_seqlens; query i of document j, Lq queries and Lk keys,
    sees [cu_k[j], cu_k[j] + Lk - Lq + i + 1), clipped to the document)."""
    ks, ke = [], []
    for j in range(len(cu_q) - 1):
        lq, lk = cu_q[j + 1] - cu_q[j], cu_k[j + 1] - cu_k[j]
        for i in range(lq):
            e = cu_k[j] + lk - lq + i + 1
            ks.append(cu_k[j])
            ke.append(min(max(e, cu_k[j]), cu_k[j + 1]))
    return np.asarray(ks, np.int32), np.asarray(ke, np.int32)


@pytest.mark.parametrize("cu_q,cu_k", [
    ([0, 8192, 24576, 49152, 65536], [0, 8192, 24576, 49152, 65536]),   # the packed BF16 sequence
    ([0, 2, 2, 5], [0, 4, 6, 9]),                                        # an empty document, Lq < Lk
    ([0, 4], [0, 2]),                                                    # Lq > Lk: leading empty windows
    ([0, 0, 3], [0, 5, 5]),                                              # a document without keys
    ([0, 1, 2, 3], [0, 100, 200, 300]),                                  # decode: one query per document
])
def test_windows_from_cu_seqlens(cu_q, cu_k):
    import torch

    import workloads

    ks, ke = ftk.windows_from_cu_seqlens(torch.tensor(cu_q, dtype=torch.int32), torch.tensor(cu_k, dtype=torch.int32))
    assert ks.dtype == torch.int32 and ke.dtype == torch.int32
    dks, dke = _windows_by_definition(cu_q, cu_k)
    assert np.array_equal(ks.numpy(), dks) and np.array_equal(ke.numpy(), dke)
    wks, wke = workloads.packed_windows(cu_q, cu_k)
    assert np.array_equal(ks.numpy(), wks) and np.array_equal(ke.numpy(), wke)


def test_windows_from_cu_seqlens_hand_values():
    import torch

    ks, ke = ftk.windows_from_cu_seqlens(torch.tensor([0, 2, 2, 5]), torch.tensor([0, 4, 6, 9]))
    assert ks.tolist() == [0, 0, 6, 6, 6]
    assert ke.tolist() == [3, 4, 7, 8, 9]
    ks, ke = ftk.windows_from_cu_seqlens(torch.tensor([0, 4]), torch.tensor([0, 2]))
    assert ks.tolist() == [0, 0, 0, 0]
    assert ke.tolist() == [0, 0, 1, 2]
