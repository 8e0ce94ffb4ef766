"""The C-ABI library without a GPU: it loads, exports what include/*.h declare,
and rejects bad arguments synchronously, before any device work.

Pointers passed here are never dereferenced: each call fails validation first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "exact_tiled_softmax_fa_amd")


def _declared_functions():
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(fa_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    import exact_tiled_softmax_fa_amd as fa
    return fa.lib()


def test_header_declares_the_entry_points():
    assert _declared_functions() == ["fa_bwd", "fa_bwd_blocksparse", "fa_bwd_masked", "fa_fwd", "fa_fwd_blocksparse",
                                     "fa_fwd_cpu", "fa_fwd_ex", "fa_fwd_masked", "fa_fwd_splitkv",
                                     "fa_fwd_splitkv_blocksparse", "fa_fwd_splitkv_heuristic",
                                     "fa_fwd_splitkv_masked", "fa_fwd_splitkv_noalloc",
                                     "fa_fwd_splitkv_workspace_size", "fa_status_string",
                                     "fa_version"]


def test_every_declared_symbol_is_exported(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_exported_symbols_match_with_nm():
    import subprocess
    import exact_tiled_softmax_fa_amd as fa
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported


def test_status_codes_are_pinned():
    """The numeric values of fa_dtype and fa_status are part of the ABI: FA_OK .. FA_ERR_LAUNCH
    are 0 .. 7 in the order of the interface's definition, then the codes this library adds."""
    text = open(os.path.join(INCLUDE, "fa_types.h")).read()
    vals = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(FA_\w+)\s*=\s*(\d+)", text)}
    assert vals == {"FA_F16": 0, "FA_BF16": 1, "FA_OK": 0, "FA_ERR_NULL": 1, "FA_ERR_SHAPE": 2,
                    "FA_ERR_HEAD_DIM": 3, "FA_ERR_DTYPE": 4, "FA_ERR_ALIGN": 5, "FA_ERR_SCALE": 6,
                    "FA_ERR_LAUNCH": 7, "FA_ERR_ALIAS": 8, "FA_ERR_OPTION": 9, "FA_ERR_WORKSPACE": 10,
                    "FA_ERR_SCRATCH": 11}


def test_status_strings_match_codes(L):
    assert L.fa_status_string(7) == b"kernel launch failed"
    assert b"overlap" in L.fa_status_string(8)
    assert b"option" in L.fa_status_string(9)
    assert b"workspace" in L.fa_status_string(10)
    assert b"scratch" in L.fa_status_string(11)


def test_entry_points_take_fa_dtype():
    """Every entry point with an element type declares it as fa_dtype, never a bare int."""
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            assert not re.search(r"\bint\s+dtype\b", text), f
            if f != "fa_types.h":
                assert "fa_dtype dtype" in text, f


def test_status_strings(L):
    for st in range(0, 12):
        s = L.fa_status_string(st)
        assert s and s != b"unknown status"
    assert L.fa_status_string(99) == b"unknown status"
    assert L.fa_status_string(0) == b"ok"
    assert L.fa_version() >= 100


# Fake, well-aligned device addresses; validation fails before any of them is used.
QA, KA, VA, OA, LA = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
GOOD = dict(q=QA, k=KA, v=VA, o=OA, lse=LA, B=1, H=2, N=64, d=64, scale=0.125, causal=0, stream=None, dtype=0)


def _call(L, **kw):
    a = dict(GOOD)
    a.update(kw)
    import exact_tiled_softmax_fa_amd as fa
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                     a["causal"], a["stream"], a["dtype"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(N=0), 2), (dict(N=-5), 2), (dict(N=(1 << 24), d=128), 2), (dict(N=(1 << 25), d=64), 2),
    (dict(B=1 << 20, H=1 << 20, N=1 << 20), 2),
    (dict(d=0), 3), (dict(d=32), 3), (dict(d=96), 3), (dict(d=256), 3),
    (dict(dtype=2), 4), (dict(dtype=-1), 4),
    (dict(q=QA + 8), 5), (dict(k=KA + 2), 5), (dict(v=VA + 4), 5), (dict(o=OA + 12), 5), (dict(lse=LA + 2), 5),
    (dict(scale=0.0), 6), (dict(scale=-0.125), 6), (dict(scale=float("inf")), 6), (dict(scale=float("nan")), 6),
    (dict(o=QA), 8), (dict(o=KA + 16), 8), (dict(lse=VA + 64), 8), (dict(lse=OA), 8),
])
def test_argument_errors(L, kw, code):
    assert _call(L, **kw) == code


def test_product_path_never_touches_the_oracle():
    """The GPU library and its binding share no code with the oracle and never load it."""
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp", ".c")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f"{f} mentions the oracle"
    for f in os.listdir(os.path.join(ROOT, "include")):
        assert "oracle" not in open(os.path.join(ROOT, "include", f)).read()
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "exact_tiled_softmax_fa_amd" not in text and "fa_fwd.h" not in text, f


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    import exact_tiled_softmax_fa_amd as fa
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


@pytest.mark.parametrize("thr,variant", [(-1.0, 0), (15.5, 0), (float("nan"), 0), (float("inf"), 0), (8.0, 2), (8.0, 3), (8.0, -1)])
def test_option_errors(L, thr, variant):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(GOOD)
    st = fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                   a["causal"], a["stream"], a["dtype"], fa.FaOptions(thr, variant))
    assert st == 9


def test_argument_errors_precede_option_errors(L):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(GOOD)
    st = fa.fa_fwd(None, a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                   a["causal"], a["stream"], a["dtype"], fa.FaOptions(-1.0, 0))
    assert st == 1


# fa_bwd: fake, well-aligned, non-overlapping addresses (validation fails before any is used)
BWD = dict(q=0x100000, k=0x200000, v=0x300000, o=0x400000, dout=0x500000, lse=0x600000, dq=0x700000,
           dk=0x800000, dv=0x900000, delta=0xA00000, B=1, H=2, N=64, d=64, scale=0.125, causal=0, stream=None,
           dtype=0)


def _bwd(**kw):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(BWD)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"], a["delta"],
                     a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["stream"], a["dtype"])


@pytest.mark.parametrize("kw,code", [
    *[(dict(**{p: None}), 1) for p in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta")],
    (dict(B=0), 2), (dict(N=0), 2), (dict(N=(1 << 24), d=128), 2), (dict(B=1 << 20, H=1 << 20, N=1 << 20), 2),
    (dict(d=96), 3), (dict(dtype=2), 4),
    (dict(q=0x100008), 5), (dict(dout=0x500004), 5), (dict(dq=0x700002), 5), (dict(lse=0x600002), 5),
    (dict(delta=0xA00001), 5),
    (dict(scale=0.0), 6), (dict(scale=float("nan")), 6),
    (dict(dq=0x100000), 8), (dict(dk=0x500000 + 64), 8), (dict(dv=0x700000), 8), (dict(delta=0x600000), 8),
    (dict(delta=0x900000), 8), (dict(dk=0x700000 + 16), 8),
])
def test_backward_argument_errors(L, kw, code):
    assert _bwd(**kw) == code


def test_backward_binding_fails_loudly_without_gpu_tensors():
    import torch
    import exact_tiled_softmax_fa_amd as fa
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q)


def _split(num_splits, ws, ws_bytes, **kw):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                             a["causal"], a["stream"], a["dtype"], num_splits, ws, ws_bytes)


def test_splitkv_workspace_size_and_heuristic(L):
    import exact_tiled_softmax_fa_amd as fa
    assert fa.splitkv_workspace_size(1, 2, 64, 64, 4) == 4 * 2 * 64 * 66 * 4
    assert fa.splitkv_workspace_size(1, 2, 64, 64, 1) == 0
    assert fa.splitkv_workspace_size(1, 2, 64, 64, 65) == 0
    assert fa.splitkv_workspace_size(1, 2, 64, 96, 4) == 0
    # cost model: rounds of ceil(G S / 256) workgroups of 1/S of the key tiles plus a start-up cost,
    # and a merge that grows with S
    assert fa.splitkv_heuristic(1, 32, 8192, 128, 0) == 1      # G = 1024: 4 full rounds already
    assert fa.splitkv_heuristic(1, 2, 16384, 128, 0) == 2      # G = 128: 2 splits fill one round
    assert fa.splitkv_heuristic(1, 1, 25600, 128, 0) == 5      # G = 100: 5 splits, 500 in 2 rounds
    assert fa.splitkv_heuristic(1, 1, 2048, 128, 0) == 8       # G = 8: capped at 32 key tiles / 4
    assert fa.splitkv_heuristic(1, 100, 512, 64, 0) == 1       # G = 200: splitting cannot shorten it
    assert fa.splitkv_heuristic(1, 1, 256, 64, 1) == 1         # too few key tiles to split
    assert 1 <= fa.splitkv_heuristic(1, 1, 1 << 22, 128, 0) <= 64


WS = 0xB00000


@pytest.mark.parametrize("num_splits,ws,ws_bytes,kw,code", [
    (0, WS, 1 << 20, {}, 9), (65, WS, 1 << 30, {}, 9), (-1, WS, 1 << 20, {}, 9),
    (4, None, 1 << 20, {}, 10), (4, WS, 100, {}, 10), (4, WS + 8, 1 << 20, {}, 10),
    (4, QA, 1 << 20, {}, 10), (4, OA - 64, 1 << 20, {}, 10), (4, LA, 1 << 20, {}, 10),
    (4, WS, 1 << 20, dict(q=None), 1), (4, WS, 1 << 20, dict(d=96), 3), (4, WS, 1 << 20, dict(o=QA), 8),
    (0, WS, 1 << 20, dict(q=None), 1),
])
def test_splitkv_argument_errors(L, num_splits, ws, ws_bytes, kw, code):
    assert _split(num_splits, ws, ws_bytes, **kw) == code


@pytest.mark.parametrize("mask,kw,code", [
    (None, {}, 1), ((-2, 0, None), {}, 9), ((0, -2, None), {}, 9), ((1 << 31, 0, None), {}, 9),
    ((4, 0, 0x600002), {}, 5), ((4, 0, None), dict(q=None), 1), ((4, 0, None), dict(d=96), 3),
    ((4, 0, None), dict(o=QA), 8),
])
def test_masked_argument_errors(L, mask, kw, code):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(GOOD)
    a.update(kw)
    m = None if mask is None else fa.FaMask(*mask)
    assert fa.fa_fwd_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                            a["stream"], a["dtype"], m) == code


FAR = dict(q=0x10000000, k=0x20000000, v=0x30000000, o=0x40000000, lse=0x50000000)  # far apart: large N


@pytest.mark.parametrize("blocks,mask,kw,code", [
    (None, None, {}, 1), ((None, 64, 64, 0, 0), None, {}, 1),
    ((0xC00000, 32, 64, 0, 0), None, {}, 9), ((0xC00000, 64, 96, 0, 0), None, {}, 9),
    ((0xC00000, 0, 64, 0, 0), None, {}, 9), ((0xC00000, 64, 64, -1, 0), None, {}, 9),
    ((0xC00000, 64, 64, 0, -8), None, {}, 9), ((0xC00000, 1 << 31, 64, 0, 0), None, {}, 9),
    ((0xC00000, 64, 64, 0, 0), (-2, 0, None), {}, 9), ((0xC00000, 64, 64, 0, 0), (4, 0, 0x600002), {}, 5),
    ((0xC00000, 64, 64, 0, 0), None, dict(q=None), 1), ((0xC00000, 64, 64, 0, 0), None, dict(d=96), 3),
    ((0xC00000, 64, 64, 0, 0), None, dict(o=QA), 8), ((0xC00000, 64, 64, 0, 0), None, dict(N=1 << 24, **FAR), 2),
])
def test_blocksparse_argument_errors(L, blocks, mask, kw, code):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(GOOD)
    a.update(kw)
    b = None if blocks is None else fa.FaBlockMask(*blocks)
    m = None if mask is None else fa.FaMask(*mask)
    assert fa.fa_fwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                 a["scale"], a["stream"], a["dtype"], m, b) == code


def _bwd_masked(mask, **kw):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(BWD)
    a.update(kw)
    m = None if mask is None else fa.FaMask(*mask)
    return fa.fa_bwd_masked(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                            a["delta"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["stream"], a["dtype"], m)


@pytest.mark.parametrize("mask,kw,code", [
    (None, {}, 1), ((-2, 0, None), {}, 9), ((0, -2, None), {}, 9), ((1 << 31, 0, None), {}, 9),
    ((4, 0, 0x600002), {}, 5), ((4, 0, None), dict(q=None), 1), ((4, 0, None), dict(delta=None), 1),
    ((4, 0, None), dict(d=96), 3), ((4, 0, None), dict(dq=0x100000), 8), ((4, 0, None), dict(scale=0.0), 6),
])
def test_bwd_masked_argument_errors(L, mask, kw, code):
    assert _bwd_masked(mask, **kw) == code


BWD_FAR = {name: (i + 1) << 28 for i, name in enumerate(("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv",
                                                           "delta"))}  # far apart: large N


@pytest.mark.parametrize("blocks,mask,kw,code", [
    (None, None, {}, 1), ((None, 64, 64, 0, 0), None, {}, 1),
    ((0xC00000, 32, 64, 0, 0), None, {}, 9), ((0xC00000, 64, 96, 0, 0), None, {}, 9),
    ((0xC00000, 64, 0, 0, 0), None, {}, 9), ((0xC00000, 64, 64, -1, 0), None, {}, 9),
    ((0xC00000, 64, 64, 0, -8), None, {}, 9), ((0xC00000, 64, 1 << 31, 0, 0), None, {}, 9),
    ((0xC00000, 64, 64, 0, 0), (-2, 0, None), {}, 9), ((0xC00000, 64, 64, 0, 0), (4, 0, 0x600002), {}, 5),
    ((0xC00000, 64, 64, 0, 0), None, dict(q=None), 1), ((0xC00000, 64, 64, 0, 0), None, dict(delta=None), 1),
    ((0xC00000, 64, 64, 0, 0), None, dict(d=96), 3), ((0xC00000, 64, 64, 0, 0), None, dict(dk=0x100000), 8),
    ((0xC00000, 64, 64, 0, 0), None, dict(scale=-1.0), 6),
    ((0xC00000, 64, 64, 0, 0), None, dict(N=1 << 24, **BWD_FAR), 2),
])
def test_bwd_blocksparse_argument_errors(L, blocks, mask, kw, code):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(BWD)
    a.update(kw)
    b = None if blocks is None else fa.FaBlockMask(*blocks)
    m = None if mask is None else fa.FaMask(*mask)
    assert fa.fa_bwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                                 a["delta"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["stream"], a["dtype"], m,
                                 b) == code


@pytest.mark.parametrize("num_splits,ws,ws_bytes,mask,kw,code", [
    (4, WS, 1 << 20, None, {}, 1), (0, WS, 1 << 20, (8, 0, None), {}, 9), (65, WS, 1 << 30, (8, 0, None), {}, 9),
    (4, WS, 1 << 20, (-2, 0, None), {}, 9), (4, WS, 1 << 20, (8, 1 << 31, None), {}, 9),
    (4, WS, 1 << 20, (8, 0, 0x600002), {}, 5),
    (4, None, 1 << 20, (8, 0, None), {}, 10), (4, WS, 100, (8, 0, None), {}, 10),
    (4, WS + 8, 1 << 20, (8, 0, None), {}, 10), (4, QA, 1 << 20, (8, 0, None), {}, 10),
    (4, WS, 1 << 20, (8, 0, None), dict(q=None), 1), (4, WS, 1 << 20, (8, 0, None), dict(d=96), 3),
    (4, WS, 1 << 20, (8, 0, None), dict(o=QA), 8),
    # the trivial masks go to fa_fwd_splitkv, which checks the same workspace
    (4, None, 1 << 20, (-1, -1, None), {}, 10),
])
def test_splitkv_masked_argument_errors(L, num_splits, ws, ws_bytes, mask, kw, code):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(GOOD)
    a.update(kw)
    m = None if mask is None else fa.FaMask(*mask)
    assert fa.fa_fwd_splitkv_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                    a["scale"], a["stream"], a["dtype"], m, num_splits, ws, ws_bytes) == code


@pytest.mark.parametrize("num_splits,ws,ws_bytes,blocks,mask,kw,code", [
    (4, WS, 1 << 20, None, None, {}, 1), (4, WS, 1 << 20, (None, 64, 64, 0, 0), None, {}, 1),
    (0, WS, 1 << 20, (0xC00000, 64, 64, 0, 0), None, {}, 9), (65, WS, 1 << 30, (0xC00000, 64, 64, 0, 0), None, {}, 9),
    (4, WS, 1 << 20, (0xC00000, 32, 64, 0, 0), None, {}, 9), (4, WS, 1 << 20, (0xC00000, 64, 64, 0, -8), None, {}, 9),
    (4, WS, 1 << 20, (0xC00000, 64, 64, 0, 0), (-2, 0, None), {}, 9),
    (4, WS, 1 << 20, (0xC00000, 64, 64, 0, 0), (8, 0, 0x600002), {}, 5),
    (4, None, 1 << 20, (0xC00000, 64, 64, 0, 0), None, {}, 10), (4, WS, 100, (0xC00000, 64, 64, 0, 0), None, {}, 10),
    (4, WS + 8, 1 << 20, (0xC00000, 64, 64, 0, 0), None, {}, 10),
    (4, QA, 1 << 20, (0xC00000, 64, 64, 0, 0), None, {}, 10),
    (4, WS, 1 << 20, (0xC00000, 64, 64, 0, 0), None, dict(q=None), 1),
    (4, WS, 1 << 20, (0xC00000, 64, 64, 0, 0), None, dict(d=96), 3),
    (4, WS, 1 << 20, (0xC00000, 64, 64, 0, 0), None, dict(o=QA), 8),
])
def test_splitkv_blocksparse_argument_errors(L, num_splits, ws, ws_bytes, blocks, mask, kw, code):
    import exact_tiled_softmax_fa_amd as fa
    a = dict(GOOD)
    a.update(kw)
    b = None if blocks is None else fa.FaBlockMask(*blocks)
    m = None if mask is None else fa.FaMask(*mask)
    assert fa.fa_fwd_splitkv_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                         a["scale"], a["stream"], a["dtype"], m, b, num_splits, ws, ws_bytes) == code


def test_noalloc_rejects_before_device_work():
    """fa_fwd_splitkv_noalloc checks its arguments and the scratch limit on the host, before any
    device call (the pointers here are never dereferenced)."""
    import exact_tiled_softmax_fa_amd as fa
    q, k, v, o, lse = (i << 32 for i in range(1, 6))  # far apart: no overlap
    # 2 splits of B*H*N = 65536 rows of d = 128 need 2 * 65536 * 130 * 4 bytes > 64 MiB
    assert fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 8, 8192, 128, 0.088, 0, 0, 0, 2) == 11
    assert fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 8, 8192, 128, 0.088, 0, 0, 0, 0) == 9
    assert fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 8, 8192, 128, 0.088, 0, 0, 0, 65) == 9
    assert fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 8, 8192, 96, 0.088, 0, 0, 0, 2) == 3
    assert fa.fa_fwd_splitkv_noalloc(None, k, v, o, lse, 1, 8, 8192, 128, 0.088, 0, 0, 0, 2) == 1
    assert fa.fa_fwd_splitkv_noalloc(q, k, v, q, lse, 1, 8, 8192, 128, 0.088, 0, 0, 0, 2) == 8
    # the largest problem that fits: B*H*N*(d+2)*splits <= 2^24
    assert fa.splitkv_workspace_size(1, 1, 64527, 128, 2) <= 64 << 20 < fa.splitkv_workspace_size(1, 1, 64528, 128, 2)
