"""The C-ABI library loads, exports every symbol include/ddt.h declares, agrees
with the binding's struct layouts, and rejects bad arguments on the host.

No call here reaches a kernel launch: every call either only computes sizes or
pointers, or fails argument validation, which happens before any HIP call.
"""
import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

from dynamic_draft_tree_row_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddt.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from dynamic_draft_tree_row_amd import build_lib
        build_lib.build()
    return L.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddt_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ddt.h but not exported"
        assert n in L.SIGNATURES, f"{n} has no binding signature"
    assert set(L.SIGNATURES) == set(names)


def test_struct_layouts_match_the_header():
    """Compile a probe with the host C compiler and compare sizeof/offsetof."""
    fields = {
        "ddt_tree": L.Tree, "ddt_flat": L.Flat, "ddt_logits": L.Logits,
        "ddt_cast": L.Cast, "ddt_graft_gate": L.Gate, "ddt_attn": L.Attn, "ddt_kv_cache": L.KVCache,
    }
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){"]
    for cname, cls in fields.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-o", exe, src], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(l.split() for l in out.strip().splitlines())
    for cname, cls in fields.items():
        assert int(got[cname]) == C.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, f"{cname}.{f}"


def test_sizes_and_binding_are_host_only(lib):
    B, cap, D, R = 8, 710, 8, 10
    n = lib.ddt_tree_bytes(B, cap, D, R)
    assert n > B * cap * 4 * 7
    buf = (C.c_uint8 * (n + 256))()
    base = (C.addressof(buf) + 255) & ~255
    t = L.Tree()
    assert lib.ddt_tree_bind(C.byref(t), C.c_void_p(base), n, B, cap, D, R) == L.DDT_OK
    assert (t.B, t.cap, t.D_max, t.R_max) == (B, cap, D, R)
    ptrs = [getattr(t, f) for f, _ in L.Tree._fields_[4:]]
    assert all(p % 256 == 0 and base <= p < base + n for p in ptrs)
    assert len(set(ptrs)) == len(ptrs)
    assert lib.ddt_tree_bind(C.byref(t), C.c_void_p(base), n - 1, B, cap, D, R) == L.DDT_EWORKSPACE
    assert lib.ddt_tree_bind(C.byref(t), C.c_void_p(base + 4), n, B, cap, D, R) == L.DDT_EINVAL
    assert lib.ddt_tree_bind(C.byref(t), None, n, B, cap, D, R) == L.DDT_EINVAL
    assert lib.ddt_tree_bind(C.byref(t), C.c_void_p(base), n, B, 5000, D, R) == L.DDT_ECAPACITY
    fbytes = lib.ddt_flat_bytes(B, 60, 8)
    fb = (C.c_uint8 * (fbytes + 256))()
    fbase = (C.addressof(fb) + 255) & ~255
    f = L.Flat()
    assert lib.ddt_flat_bind(C.byref(f), C.c_void_p(fbase), fbytes, B, 60, 8) == L.DDT_OK
    assert (f.P, f.W, f.Dp, f.L) == (61, 2, 8, 60)
    assert lib.ddt_flat_bind(C.byref(f), C.c_void_p(fbase), fbytes, B, 300, 8) == L.DDT_ECAPACITY


def test_workspace_and_chunk_sizes(lib):
    assert lib.ddt_chunk_elems(L.DDT_BF16) == 8192
    assert lib.ddt_chunk_elems(L.DDT_F32) == 4096
    assert lib.ddt_chunk_elems(7) == -1
    # 80 rows x 16 chunks x (2 + 2*10) words
    assert lib.ddt_workspace_bytes(80, 128256, L.DDT_BF16, 10) == 80 * 16 * 22 * 4
    assert lib.ddt_workspace_bytes(10, 32000, L.DDT_F32, 10) == 10 * 8 * 22 * 4
    assert lib.ddt_workspace_bytes(1, 0, L.DDT_BF16, 10) == 0


def test_calls_reject_bad_arguments_before_launch(lib):
    n = lib.ddt_tree_bytes(2, 64, 3, 4)
    buf = (C.c_uint8 * (n + 256))()
    base = (C.addressof(buf) + 255) & ~255
    t = L.Tree()
    assert lib.ddt_tree_bind(C.byref(t), C.c_void_p(base), n, 2, 64, 3, 4) == L.DDT_OK
    dummy = C.c_void_p(base)
    lg = L.Logits(dummy, L.DDT_BF16, 1000, 4000, 1000)
    ws = C.c_void_p(base)
    e = lib.ddt_tree_expand
    assert e(None, 1, dummy, C.byref(lg), 4, 4, None, None, ws, 1 << 20, None) == L.DDT_EINVAL
    assert e(C.byref(t), 0, dummy, C.byref(lg), 4, 4, None, None, ws, 1 << 20, None) == L.DDT_EINVAL
    assert e(C.byref(t), 1, None, C.byref(lg), 4, 4, None, None, ws, 1 << 20, None) == L.DDT_EINVAL
    assert e(C.byref(t), 1, dummy, C.byref(lg), 33, 4, None, None, ws, 1 << 20, None) == L.DDT_ECAPACITY
    assert e(C.byref(t), 1, dummy, C.byref(lg), 4, 5, None, None, ws, 1 << 20, None) == L.DDT_ECAPACITY
    assert e(C.byref(t), 1, dummy, C.byref(lg), 4, 4, None, None, ws, 16, None) == L.DDT_EWORKSPACE
    bad = L.Logits(dummy, 9, 1000, 4000, 1000)
    assert e(C.byref(t), 1, dummy, C.byref(bad), 4, 4, None, None, ws, 1 << 20, None) == L.DDT_EDTYPE
    # a tree too small for the requested budgets
    assert e(C.byref(t), 1, dummy, C.byref(lg), 8, 4, None, None, ws, 1 << 20, None) == L.DDT_ECAPACITY
    cs = L.Cast(dummy, dummy, 256, 16, 128, dummy, 0.1, dummy, 9, 0)
    gate = L.Gate()
    assert e(C.byref(t), 1, dummy, C.byref(lg), 4, 4, C.byref(cs), None, ws, 1 << 20, None) == L.DDT_EINVAL
    assert e(C.byref(t), 1, dummy, C.byref(lg), 4, 4, C.byref(cs), C.byref(gate), ws, 1 << 20,
             None) == L.DDT_EINVAL
    assert lib.ddt_tree_rerank(C.byref(t), 300, None, 0, dummy, dummy, None) == L.DDT_ECAPACITY
    assert lib.ddt_tree_rerank(C.byref(t), 10, None, 0, None, dummy, None) == L.DDT_EINVAL
    assert lib.ddt_succ_gather(C.byref(t), dummy, 0, 1000, 8, 8, 9, 60, 60, dummy, dummy,
                               None) == L.DDT_EINVAL
    assert lib.ddt_succ_gather(C.byref(t), dummy, 0, 1000, 8, 8, 8, 60, 59, dummy, dummy,
                               None) == L.DDT_EINVAL
    f = L.Flat()
    assert lib.ddt_tree_build_mask(C.byref(t), dummy, dummy, 0, C.byref(f), None, None) == L.DDT_EINVAL
    sl = lib.ddt_tree_select
    assert sl(C.byref(t), 300, None, 0, dummy, dummy, 0, C.byref(f), None, None) == L.DDT_ECAPACITY
    assert sl(C.byref(t), 10, None, 0, None, dummy, 0, C.byref(f), None, None) == L.DDT_EINVAL
    assert sl(C.byref(t), 10, None, 0, dummy, dummy, 0, C.byref(f), None, None) == L.DDT_EINVAL
    assert lib.ddt_row_topk(C.byref(lg), 2, 3, 0, None, None, None, None, ws, 1 << 20, None) == L.DDT_EINVAL
    assert lib.ddt_row_topk(C.byref(lg), 2, 3, 40, None, None, None, None, ws, 1 << 20,
                            None) == L.DDT_ECAPACITY
    huge = L.Logits(dummy, L.DDT_BF16, 64 * 8192 + 1, 0, 0)
    assert lib.ddt_row_topk(C.byref(huge), 1, 1, 4, None, None, None, None, ws, 1 << 30,
                            None) == L.DDT_ECAPACITY
    assert lib.ddt_strerror(L.DDT_EWORKSPACE).decode() == "workspace too small"
    # tree attention with key splits: sizes are host arithmetic; a split
    # count above 1 needs an aligned workspace of the stated size
    sp, wsb = lib.ddt_tree_attention_splits, lib.ddt_tree_attention_ws_bytes
    assert sp(64, 129, 32, 8, 4096, 0) == 1 and wsb(64, 129, 32, 8, 4096, 0) == 0
    # 8 requests x 8 heads x 2 tiles = 128 workgroups: 4 splits (512 in all)
    # of 17 of the 65 key blocks; partials of 4 x 8 x 61 x 32 rows, 128
    # outputs + 2 statistics each
    assert sp(8, 61, 32, 8, 4096, 0) == 4
    assert wsb(8, 61, 32, 8, 4096, 0) == 4 * 8 * 61 * 32 * (128 * 4 + 8)
    assert sp(8, 1, 32, 8, 4096, 0) == 8 and sp(16, 61, 32, 8, 4096, 0) == 2
    assert sp(2, 20, 2, 1, 300, 5) == 3                     # 6 blocks, 2 per split
    assert sp(2, 20, 2, 1, 300, 99) == 6 and sp(2, 20, 2, 1, 0, 4) == 1
    assert sp(2, 20, 3, 2, 300, 0) == 0 and wsb(0, 20, 2, 1, 300, 0) == 0
    nf = lib.ddt_flat_bytes(2, 19, 4)
    fbuf = (C.c_uint8 * (nf + 256))()
    fbase = (C.addressof(fbuf) + 255) & ~255
    fl = L.Flat()
    assert lib.ddt_flat_bind(C.byref(fl), C.c_void_p(fbase), nf, 2, 19, 4) == L.DDT_OK
    at = L.Attn(dummy, dummy, dummy, dummy, dummy, 2, 20, 2, 1, 128, 300, 0.1)
    asp = lib.ddt_tree_attention_split
    need = wsb(2, 20, 2, 1, 300, 5)
    assert asp(C.byref(fl), C.byref(at), dummy, -1, ws, need, None) == L.DDT_EINVAL
    assert asp(C.byref(fl), C.byref(at), dummy, 5, None, need, None) == L.DDT_EWORKSPACE
    assert asp(C.byref(fl), C.byref(at), dummy, 5, ws, need - 1, None) == L.DDT_EWORKSPACE
    assert asp(C.byref(fl), C.byref(at), dummy, 5, C.c_void_p(base + 8), need, None) == L.DDT_EWORKSPACE
    bad_at = L.Attn(dummy, dummy, dummy, dummy, dummy, 2, 20, 2, 1, 128, 300, 0.0)
    assert asp(C.byref(fl), C.byref(bad_at), dummy, 5, ws, need, None) == L.DDT_EINVAL
    # paged KV cache
    kv = L.KVCache(dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 4, 8, 64, 16, 8, 128)
    c = lib.ddt_kv_commit
    assert c(None, dummy, dummy, 8, dummy, dummy, 61, dummy, None) == L.DDT_EINVAL
    assert c(C.byref(kv), None, dummy, 8, dummy, dummy, 61, dummy, None) == L.DDT_EINVAL
    assert c(C.byref(kv), dummy, dummy, -1, dummy, dummy, 61, dummy, None) == L.DDT_EINVAL
    assert c(C.byref(kv), dummy, dummy, 8, dummy, C.c_void_p(base + 8), 61, dummy, None) == L.DDT_EINVAL
    odd = L.KVCache(dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 4, 8, 64, 16, 3, 5)
    assert c(C.byref(odd), dummy, dummy, 8, dummy, dummy, 61, dummy, None) == L.DDT_EINVAL
    big = L.KVCache(dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 2000, 8, 64, 16, 8, 128)
    assert c(C.byref(big), dummy, dummy, 8, dummy, dummy, 61, dummy, None) == L.DDT_ECAPACITY
    wide = L.KVCache(dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 4, 5000, 64, 16, 8, 128)
    assert lib.ddt_kv_release(C.byref(wide), dummy, 1, None) == L.DDT_ECAPACITY
    assert lib.ddt_kv_fork(C.byref(kv), None, dummy, 1, dummy, None) == L.DDT_EINVAL
    assert lib.ddt_kv_fork(C.byref(kv), dummy, dummy, -1, dummy, None) == L.DDT_EINVAL
    assert lib.ddt_kv_release(C.byref(kv), None, 2, None) == L.DDT_EINVAL
    # nothing to do: no launch, no device touched
    assert lib.ddt_kv_fork(C.byref(kv), None, None, 0, None, None) == L.DDT_OK
    assert lib.ddt_kv_release(C.byref(kv), None, 0, None) == L.DDT_OK
