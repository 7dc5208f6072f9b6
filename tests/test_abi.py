"""C ABI checks that need no GPU: the library loads, exports every entry point declared in
include/jattn.h, include/jattn_adaln.h, include/jattn_mlp.h and include/jattn_diag.h, and rejects invalid arguments on the host before any HIP call.

Every call here is constructed to fail validation: the fake device addresses are never
dereferenced, because a call that passed validation would enqueue kernels."""
import ctypes
import math
import os
import re

import pytest

from diffusion_transformer_joint_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libjattn.so not built (run __graft_entry__.build())")

A = 0x10000  # 256-byte aligned fake addresses, distinct ranges
TB = 1 << 24


def fake(i):
    return A + i * TB


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    header = "".join(open(os.path.join(ROOT, "include", h)).read() for h in ("jattn.h", "jattn_adaln.h", "jattn_mlp.h", "jattn_diag.h"))
    declared = set(re.findall(r"\b(jattn_[a-z_]+)\s*\(", header))
    assert declared == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.jattn_status_string(code).decode() == name
    assert lib.jattn_status_string(99).decode() == "JATTN_UNKNOWN_STATUS"
    assert lib.jattn_abi_version() == _lib.ABI_VERSION


def fwd(lib, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gains=fake(3), valid_len=None, B=2, L=100, H=3, D=64,
             scale=0.125, eps=1e-6, out=fake(4), lse=fake(5), ws=fake(6), ws_bytes=None, stream=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.jattn_fwd_workspace_bytes(a["B"], a["L"], a["H"], a["D"])
    return lib.jattn_fwd(a["q"], a["k"], a["v"], a["gains"], a["valid_len"], a["B"], a["L"], a["H"], a["D"],
                         ctypes.c_float(a["scale"]), ctypes.c_float(a["eps"]), a["out"], a["lse"], a["ws"],
                         a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), _lib.INVALID_VALUE),
    (dict(k=None), _lib.INVALID_VALUE),
    (dict(v=None), _lib.INVALID_VALUE),
    (dict(gains=None), _lib.INVALID_VALUE),
    (dict(out=None), _lib.INVALID_VALUE),
    (dict(lse=None), _lib.INVALID_VALUE),
    (dict(B=0), _lib.INVALID_VALUE),
    (dict(L=0), _lib.INVALID_VALUE),
    (dict(H=-1), _lib.INVALID_VALUE),
    (dict(D=44), _lib.NOT_SUPPORTED),
    (dict(D=256), _lib.NOT_SUPPORTED),
    (dict(B=1, L=1 << 20, H=64, D=128), _lib.NOT_SUPPORTED),
    (dict(scale=math.inf), _lib.INVALID_VALUE),
    (dict(scale=math.nan), _lib.INVALID_VALUE),
    (dict(eps=-1e-6), _lib.INVALID_VALUE),
    (dict(eps=math.nan), _lib.INVALID_VALUE),
    (dict(q=fake(0) + 8), _lib.INVALID_VALUE),          # misaligned bf16 tensor
    (dict(lse=fake(5) + 2), _lib.INVALID_VALUE),        # misaligned fp32 array
    (dict(out=fake(0)), _lib.INVALID_VALUE),            # out aliases q
    (dict(lse=fake(4) + 4096), _lib.INVALID_VALUE),     # lse overlaps out
    (dict(out=fake(3) - 16), _lib.INVALID_VALUE),       # out overlaps gains
    (dict(ws=None), _lib.WORKSPACE),                    # no workspace
    (dict(ws_bytes=1024), _lib.WORKSPACE),              # workspace too small
    (dict(ws=fake(6) + 64), _lib.INVALID_VALUE),        # workspace must be 256-byte aligned
    (dict(ws=fake(1)), _lib.INVALID_VALUE),             # workspace aliases k
    (dict(ws=fake(4)), _lib.INVALID_VALUE),             # workspace aliases out
])
def test_fwd_rejects(lib, kw, expect):
    assert fwd(lib, **kw) == expect


def bwd(lib, ws_bytes=None, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gains=fake(3), valid_len=None, out=fake(4), lse=fake(5),
             dout=fake(6), B=2, L=100, H=3, D=64, scale=0.125, eps=1e-6, dq=fake(7), dk=fake(8), dv=fake(9),
             dgains=fake(10), ws=fake(11), fws=None, stream=None)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.jattn_bwd_workspace_bytes(a["B"], a["L"], a["H"], a["D"])
    return lib.jattn_bwd(a["q"], a["k"], a["v"], a["gains"], a["valid_len"], a["out"], a["lse"], a["dout"],
                         a["B"], a["L"], a["H"], a["D"], ctypes.c_float(a["scale"]), ctypes.c_float(a["eps"]),
                         a["dq"], a["dk"], a["dv"], a["dgains"], a["ws"], ws_bytes, a["fws"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(dout=None), _lib.INVALID_VALUE),
    (dict(dq=None), _lib.INVALID_VALUE),
    (dict(dgains=None), _lib.INVALID_VALUE),
    (dict(lse=None), _lib.INVALID_VALUE),
    (dict(B=0), _lib.INVALID_VALUE),
    (dict(D=16), _lib.NOT_SUPPORTED),
    (dict(scale=-math.inf), _lib.INVALID_VALUE),
    (dict(eps=-0.5), _lib.INVALID_VALUE),
    (dict(ws=None), _lib.WORKSPACE),
    (dict(dk=fake(8) + 4), _lib.INVALID_VALUE),
    (dict(ws=fake(11) + 64), _lib.INVALID_VALUE),       # workspace must be 256-byte aligned
    (dict(dq=fake(6)), _lib.INVALID_VALUE),             # dq aliases dout
    (dict(dv=fake(7) + 4096), _lib.INVALID_VALUE),      # dv overlaps dq
    (dict(ws=fake(0)), _lib.INVALID_VALUE),             # workspace aliases q
    (dict(fws=fake(12) + 64), _lib.INVALID_VALUE),      # forward workspace must be 256-byte aligned
    (dict(fws=fake(11)), _lib.INVALID_VALUE),           # workspace aliases the forward workspace
    (dict(fws=fake(8)), _lib.INVALID_VALUE),            # dk aliases the forward workspace
])
def test_bwd_rejects(lib, kw, expect):
    assert bwd(lib, **kw) == expect


def test_bwd_ex_rejects_bad_event_arguments(lib):
    need = lib.jattn_bwd_workspace_bytes(2, 100, 3, 64)
    base = [fake(0), fake(1), fake(2), fake(3), None, fake(4), fake(5), fake(6), 2, 100, 3, 64,
            ctypes.c_float(0.125), ctypes.c_float(1e-6), fake(7), fake(8), fake(9), fake(10), fake(11), need, None]
    assert lib.jattn_bwd_ex(*base, None, 1, None) == _lib.INVALID_VALUE
    assert lib.jattn_bwd_ex(*base, fake(12), -1, None) == _lib.INVALID_VALUE
    assert lib.jattn_bwd_ex(*base, fake(12), len(_lib.BWD_STAGES) + 1, None) == _lib.INVALID_VALUE
    # valid event arguments still fail on the invalid tensor arguments, before any HIP call
    bad = list(base)
    bad[0] = None
    assert lib.jattn_bwd_ex(*bad, fake(12), len(_lib.BWD_STAGES), None) == _lib.INVALID_VALUE


def test_bwd_rejects_small_workspace(lib):
    need = lib.jattn_bwd_workspace_bytes(2, 100, 3, 64)
    assert need > 0
    assert bwd(lib, ws_bytes=need - 1) == _lib.WORKSPACE


def test_fwd_workspace_bytes(lib):
    assert lib.jattn_fwd_workspace_bytes(0, 10, 1, 64) == 0
    assert lib.jattn_fwd_workspace_bytes(1, 10, 1, 44) == 0
    w = lib.jattn_fwd_workspace_bytes(16, 1101, 12, 64)
    assert w >= 16 * 1101 * 12 * 64 * 2 and w % 256 == 0


def test_workspace_bytes(lib):
    assert lib.jattn_bwd_workspace_bytes(0, 10, 1, 64) == 0
    assert lib.jattn_bwd_workspace_bytes(1, 10, 1, 44) == 0
    w = lib.jattn_bwd_workspace_bytes(16, 1101, 12, 64)
    # normalised K and Q rows (bf16), two statistics per padded query row (9 blocks of 128 rows per
    # pair) and one set of per-workgroup gain-gradient partials
    assert w >= 2 * 16 * 12 * 1101 * 64 * 2 + 2 * 16 * 12 * 9 * 128 * 4 + 16 * 12 * 9 * 64 * 4
    assert w % 256 == 0


def test_fwd_ex_rejects_bad_event_arguments(lib):
    base = [fake(0), fake(1), fake(2), fake(3), None, 2, 100, 3, 64, ctypes.c_float(0.125), ctypes.c_float(1e-6),
            fake(4), fake(5), fake(6), lib.jattn_fwd_workspace_bytes(2, 100, 3, 64)]
    assert lib.jattn_fwd_ex(*base, None, 1, None) == _lib.INVALID_VALUE
    assert lib.jattn_fwd_ex(*base, fake(12), -1, None) == _lib.INVALID_VALUE
    assert lib.jattn_fwd_ex(*base, fake(12), len(_lib.FWD_STAGES) + 1, None) == _lib.INVALID_VALUE
    bad = list(base)
    bad[0] = None
    assert lib.jattn_fwd_ex(*bad, fake(12), len(_lib.FWD_STAGES), None) == _lib.INVALID_VALUE


def test_stage_names_match_header():
    hdr = open(os.path.join(ROOT, "include", "jattn.h")).read()
    assert int(re.search(r"#define JATTN_BWD_STAGES (\d+)", hdr).group(1)) == len(_lib.BWD_STAGES)
    assert int(re.search(r"#define JATTN_FWD_STAGES (\d+)", hdr).group(1)) == len(_lib.FWD_STAGES)


# ------------------------------------------------------------------------------------------------
# Two-stream entry points: tensors are host arrays {image part, text part} of device pointers.
def pair(i, j):
    return _lib.PtrPair(fake(i), fake(j))


def fwd_streams(lib, **kw):
    a = dict(q=(0, 1), k=(2, 3), v=(4, 5), gains=fake(6), valid_len=None, B=2, n_img=100, n_txt=37, H=3, D=64,
             scale=0.125, eps=1e-6, out=(7, 8), lse=fake(9), ws=fake(10), ws_bytes=None, events=None, n_events=0)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.jattn_fwd_workspace_bytes(a["B"], max(a["n_img"] + a["n_txt"], 0), a["H"], a["D"])
    keep = {}
    def arg(name):
        t = a[name]
        if t is None or isinstance(t, _lib.PtrPair):
            keep[name] = t
        else:
            keep[name] = _lib.PtrPair(*[None if x is None else (fake(x) if isinstance(x, int) and x < 64 else x)
                                        for x in t])
        return None if keep[name] is None else keep[name].arg
    return lib.jattn_fwd_streams(arg("q"), arg("k"), arg("v"), a["gains"], a["valid_len"], a["B"], a["n_img"],
                                 a["n_txt"], a["H"], a["D"], ctypes.c_float(a["scale"]), ctypes.c_float(a["eps"]),
                                 arg("out"), a["lse"], a["ws"], a["ws_bytes"], a["events"], a["n_events"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), _lib.INVALID_VALUE),                       # no host array
    (dict(q=(None, 1)), _lib.INVALID_VALUE),                  # image part missing
    (dict(v=(4, None)), _lib.INVALID_VALUE),                  # text part missing
    (dict(out=(7, None)), _lib.INVALID_VALUE),
    (dict(k=(fake(2) + 8, 3)), _lib.INVALID_VALUE),           # misaligned image part
    (dict(n_img=-1), _lib.INVALID_VALUE),
    (dict(n_img=0, n_txt=0), _lib.INVALID_VALUE),
    (dict(D=44), _lib.NOT_SUPPORTED),
    (dict(gains=None), _lib.INVALID_VALUE),
    (dict(eps=math.nan), _lib.INVALID_VALUE),
    (dict(out=(1, 8)), _lib.INVALID_VALUE),                   # image output aliases the text query part
    (dict(out=(7, fake(6) - 16)), _lib.INVALID_VALUE),        # text output overlaps the gains
    (dict(lse=fake(7) + 4096), _lib.INVALID_VALUE),           # lse overlaps the image output
    (dict(ws=None), _lib.WORKSPACE),
    (dict(ws_bytes=1024), _lib.WORKSPACE),
    (dict(ws=fake(0)), _lib.INVALID_VALUE),                   # workspace aliases the image queries
    (dict(n_events=1), _lib.INVALID_VALUE),                   # events count without an array
    # the pointers of an empty stream are ignored: these reach the workspace check
    (dict(n_txt=0, q=(0, None), k=(2, None), v=(4, None), out=(7, None), ws_bytes=1024), _lib.WORKSPACE),
    (dict(n_img=0, q=(None, 1), k=(None, 3), v=(None, 5), out=(None, 8), ws_bytes=1024), _lib.WORKSPACE),
])
def test_fwd_streams_rejects(lib, kw, expect):
    assert fwd_streams(lib, **kw) == expect


def bwd_streams(lib, **kw):
    a = dict(q=(0, 1), k=(2, 3), v=(4, 5), gains=fake(6), valid_len=None, out=(7, 8), lse=fake(9), dout=(10, 11),
             B=2, n_img=100, n_txt=37, H=3, D=64, scale=0.125, eps=1e-6, dq=(12, 13), dk=(14, 15), dv=(16, 17),
             dgains=fake(18), ws=fake(19), ws_bytes=None, fws=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.jattn_bwd_workspace_bytes(a["B"], a["n_img"] + a["n_txt"], a["H"], a["D"])
    keep = []
    def arg(name):
        t = a[name]
        if t is None:
            return None
        p = _lib.PtrPair(*[None if x is None else (fake(x) if x < 64 else x) for x in t])
        keep.append(p)
        return p.arg
    return lib.jattn_bwd_streams(arg("q"), arg("k"), arg("v"), a["gains"], a["valid_len"], arg("out"), a["lse"],
                                 arg("dout"), a["B"], a["n_img"], a["n_txt"], a["H"], a["D"],
                                 ctypes.c_float(a["scale"]), ctypes.c_float(a["eps"]), arg("dq"), arg("dk"),
                                 arg("dv"), a["dgains"], a["ws"], a["ws_bytes"], a["fws"], None, 0, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dout=None), _lib.INVALID_VALUE),
    (dict(dq=(12, None)), _lib.INVALID_VALUE),
    (dict(dgains=None), _lib.INVALID_VALUE),
    (dict(n_txt=-5), _lib.INVALID_VALUE),
    (dict(dk=(14, fake(15) + 4)), _lib.INVALID_VALUE),       # misaligned text part
    (dict(dq=(12, 10)), _lib.INVALID_VALUE),                  # text dq aliases the image dout
    (dict(dv=(fake(13) + 4096, 17)), _lib.INVALID_VALUE),     # image dv overlaps the text dq
    (dict(dgains=fake(6)), _lib.INVALID_VALUE),               # dgains aliases the gains
    (dict(ws=None), _lib.WORKSPACE),
    (dict(ws=fake(19) + 64), _lib.INVALID_VALUE),
    (dict(fws=fake(19)), _lib.INVALID_VALUE),                 # workspace aliases the forward workspace
    (dict(fws=fake(20) + 64), _lib.INVALID_VALUE),
    (dict(n_txt=0, q=(0, None), k=(2, None), v=(4, None), out=(7, None), dout=(10, None), dq=(12, None),
          dk=(14, None), dv=(16, None), ws_bytes=1024), _lib.WORKSPACE),
])
def test_bwd_streams_rejects(lib, kw, expect):
    assert bwd_streams(lib, **kw) == expect


# ------------------------------------------------------------------------------------------------
# Packed variable-length entry points
def fwd_varlen(lib, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gains=fake(3), cu=fake(4), B=3, maxlen=100, total=250, H=3, D=64,
             scale=0.125, eps=1e-6, out=fake(5), lse=fake(6), ws=fake(7), ws_bytes=None, events=None, n_events=0)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.jattn_varlen_fwd_workspace_bytes(a["B"], a["maxlen"], a["total"], a["H"], a["D"])
    return lib.jattn_fwd_varlen(a["q"], a["k"], a["v"], a["gains"], a["cu"], a["B"], a["maxlen"], a["total"], a["H"],
                                a["D"], ctypes.c_float(a["scale"]), ctypes.c_float(a["eps"]), a["out"], a["lse"],
                                a["ws"], a["ws_bytes"], a["events"], a["n_events"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(cu=None), _lib.INVALID_VALUE),
    (dict(q=None), _lib.INVALID_VALUE),
    (dict(total=0), _lib.INVALID_VALUE),
    (dict(maxlen=0), _lib.INVALID_VALUE),
    (dict(B=0), _lib.INVALID_VALUE),
    (dict(D=36), _lib.NOT_SUPPORTED),
    (dict(B=70000), _lib.NOT_SUPPORTED),
    (dict(cu=fake(4) + 2), _lib.INVALID_VALUE),           # misaligned offsets
    (dict(out=fake(0)), _lib.INVALID_VALUE),              # out aliases q
    (dict(lse=fake(4)), _lib.INVALID_VALUE),              # lse aliases cu_seqlens
    (dict(ws=None), _lib.WORKSPACE),
    (dict(ws_bytes=100), _lib.WORKSPACE),
    (dict(ws=fake(7) + 32), _lib.INVALID_VALUE),
    (dict(n_events=3), _lib.INVALID_VALUE),
])
def test_fwd_varlen_rejects(lib, kw, expect):
    assert fwd_varlen(lib, **kw) == expect


def test_bwd_varlen_rejects(lib):
    need = lib.jattn_varlen_bwd_workspace_bytes(3, 100, 250, 3, 64)
    base = dict(q=fake(0), k=fake(1), v=fake(2), gains=fake(3), cu=fake(4), out=fake(5), lse=fake(6), dout=fake(7),
                dq=fake(8), dk=fake(9), dv=fake(10), dgains=fake(11), ws=fake(12), ws_bytes=need, fws=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.jattn_bwd_varlen(a["q"], a["k"], a["v"], a["gains"], a["cu"], a["out"], a["lse"], a["dout"], 3, 100,
                                    250, 3, 64, ctypes.c_float(0.125), ctypes.c_float(1e-6), a["dq"], a["dk"], a["dv"],
                                    a["dgains"], a["ws"], a["ws_bytes"], a["fws"], None, 0, None)
    assert call(cu=None) == _lib.INVALID_VALUE
    assert call(dgains=None) == _lib.INVALID_VALUE
    assert call(dq=fake(7)) == _lib.INVALID_VALUE       # dq aliases dout
    assert call(dk=fake(4)) == _lib.INVALID_VALUE       # dk aliases cu_seqlens
    assert call(ws_bytes=need - 1) == _lib.WORKSPACE
    assert call(fws=fake(12)) == _lib.INVALID_VALUE     # workspace aliases the forward workspace


def test_varlen_workspace_bytes(lib):
    assert lib.jattn_varlen_fwd_workspace_bytes(2, 10, 0, 1, 64) == 0
    assert lib.jattn_varlen_fwd_workspace_bytes(2, 10, 15, 1, 44) == 0
    f = lib.jattn_varlen_fwd_workspace_bytes(16, 2370, 22682, 12, 64)
    assert f >= 22682 * 12 * 64 * 2 and f % 256 == 0
    w = lib.jattn_varlen_bwd_workspace_bytes(16, 2370, 22682, 12, 64)
    # two bf16 row copies, two statistics per (row, head) with 128 rows of slack per sequence, gain partials
    assert w >= 2 * 22682 * 12 * 64 * 2 + 2 * (22682 + 128 * 16) * 12 * 4 + 16 * 12 * 19 * 64 * 4


# ------------------------------------------------------------------------------------------------
# Local-window entry points: the joint entry points' validation with two extra bounds
def test_window_entry_points_reject(lib):
    fwb = lib.jattn_fwd_workspace_bytes(2, 100, 3, 64)
    def fwdw(**kw):
        a = dict(q=fake(0), out=fake(4), ws=fake(6), ws_bytes=fwb, D=64, left=16, right=-1)
        a.update(kw)
        return lib.jattn_fwd_window(a["q"], fake(1), fake(2), fake(3), None, 2, 100, 3, a["D"], ctypes.c_float(0.125),
                                    ctypes.c_float(1e-6), a["left"], a["right"], a["out"], fake(5), a["ws"],
                                    a["ws_bytes"], None, 0, None)
    assert fwdw(q=None) == _lib.INVALID_VALUE
    assert fwdw(out=fake(1)) == _lib.INVALID_VALUE
    assert fwdw(D=44) == _lib.NOT_SUPPORTED
    assert fwdw(ws_bytes=16) == _lib.WORKSPACE
    assert fwdw(left=-5, right=10**9, ws_bytes=16) == _lib.WORKSPACE   # any bounds are accepted
    need = lib.jattn_bwd_workspace_bytes(2, 100, 3, 64)
    def bwdw(**kw):
        a = dict(dq=fake(7), ws=fake(11), ws_bytes=need)
        a.update(kw)
        return lib.jattn_bwd_window(fake(0), fake(1), fake(2), fake(3), None, fake(4), fake(5), fake(6), 2, 100, 3, 64,
                                    ctypes.c_float(0.125), ctypes.c_float(1e-6), 4, 4, a["dq"], fake(8), fake(9),
                                    fake(10), a["ws"], a["ws_bytes"], None, None, 0, None)
    assert bwdw(dq=fake(6)) == _lib.INVALID_VALUE
    assert bwdw(ws_bytes=need - 1) == _lib.WORKSPACE


@pytest.mark.parametrize("which,blocks,iters,out", [
    (2, 8, 4, fake(0)),            # unknown probe
    (-1, 8, 4, fake(0)),
    (0, 0, 4, fake(0)),            # no workgroups
    (1, 8, 0, fake(0)),            # no iterations
    (0, 1 << 23, 4, fake(0)),      # blocks * 256 reaches 2^31
    (0, 8, 4, None),               # no output
    (1, 8, 4, fake(0) + 2),        # misaligned output
])
def test_probe_rejects_invalid_arguments(lib, which, blocks, iters, out):
    assert lib.jattn_probe_saturate(which, blocks, iters, ctypes.c_float(1.0), out, None) == _lib.INVALID_VALUE


def fwd_noalloc(lib, **kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gains=fake(3), valid_len=None, B=2, L=100, H=3, D=64,
             scale=0.125, eps=1e-6, out=fake(4), lse=fake(5), stream=None)
    a.update(kw)
    return lib.jattn_fwd_noalloc(a["q"], a["k"], a["v"], a["gains"], a["valid_len"], a["B"], a["L"], a["H"], a["D"],
                                 ctypes.c_float(a["scale"]), ctypes.c_float(a["eps"]), a["out"], a["lse"], a["stream"])


def test_noalloc_scratch_size(lib):
    assert lib.jattn_fwd_noalloc_max_scratch_bytes() == 64 << 20


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), _lib.INVALID_VALUE),
    (dict(lse=None), _lib.INVALID_VALUE),
    (dict(D=44), _lib.NOT_SUPPORTED),
    (dict(eps=-1.0), _lib.INVALID_VALUE),
    (dict(out=fake(1)), _lib.INVALID_VALUE),        # out aliases k
    (dict(q=fake(0) + 8), _lib.INVALID_VALUE),      # misaligned
    # normalised keys (B L H D bf16) one 256-byte chunk past the 64 MiB scratch array; tensors that
    # big at fake addresses 2^32 apart, so only the scratch limit can refuse the call
    (dict(B=1, L=(64 << 20) // (16 * 64 * 2) + 1, H=16, D=64, q=1 << 32, k=2 << 32, v=3 << 32, gains=4 << 32,
          out=5 << 32, lse=6 << 32), _lib.WORKSPACE),
])
def test_noalloc_validation(lib, kw, expect):
    assert fwd_noalloc(lib, **kw) == expect


def test_noalloc_largest_accepted_size_is_the_scratch(lib):
    # exactly 64 MiB of normalised keys passes the size check: the call is then refused by the next
    # check (out aliasing q), still before any HIP call
    L = (64 << 20) // (16 * 64 * 2)
    assert fwd_noalloc(lib, B=1, L=L, H=16, D=64, q=1 << 32, k=2 << 32, v=3 << 32, gains=4 << 32, out=1 << 32,
                       lse=6 << 32) == _lib.INVALID_VALUE


@pytest.mark.parametrize("args", [
    (3, 192, 1101, 64, 9),      # unknown mode
    (0, 0, 1101, 64, 9),        # no pairs
    (0, 192, 1101, 66, 9),      # D not a multiple of 4
    (0, 192, 1101, 132, 9),     # D past 128
    (0, 192, 1101, 64, 65),     # too many key blocks
    (1, 4096, 4096, 128, 9),    # element count past 2^31
])
def test_probe_dq_accumulation_validation(lib, args):
    mode, pairs, L, D, nkb = args
    assert lib.jattn_probe_dq_accumulation(mode, pairs, L, D, nkb, fake(0), 1 << 40, None) == _lib.INVALID_VALUE


def test_probe_dq_accumulation_buffer_size(lib):
    pairs, L, D, nkb = 2, 100, 64, 3
    n = pairs * L * D * 4
    for mode, need in ((0, n), (1, nkb * n), (2, (nkb + 1) * n)):
        assert lib.jattn_probe_dq_accumulation(mode, pairs, L, D, nkb, fake(0), need - 4, None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_dq_accumulation(0, pairs, L, D, nkb, None, n, None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_dq_accumulation(0, pairs, L, D, nkb, fake(0) + 4, n, None) == _lib.INVALID_VALUE


@pytest.mark.parametrize("args", [
    (8, 4, 10),    # unknown mode
    (-1, 4, 10),
    (0, 0, 10),    # no workgroups
    (0, 4, 0),     # no iterations
    (0, 1 << 23, 10),  # blocks * 256 >= 2^31
])
def test_probe_tile_validation(lib, args):
    mode, blocks, iters = args
    assert lib.jattn_probe_tile(mode, blocks, iters, ctypes.c_float(1.0), fake(0), fake(1), None) == _lib.INVALID_VALUE


def test_probe_tile_pointers(lib):
    assert lib.jattn_probe_tile(0, 4, 10, ctypes.c_float(1.0), None, fake(1), None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_tile(0, 4, 10, ctypes.c_float(1.0), fake(0), None, None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_tile(0, 4, 10, ctypes.c_float(1.0), fake(0) + 2, fake(1), None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_tile(0, 4, 10, ctypes.c_float(1.0), fake(0), fake(1) + 4, None) == _lib.INVALID_VALUE


@pytest.mark.parametrize("args", [(3, 4, 10), (-1, 4, 10), (0, 0, 10), (0, 4, 0), (0, 1 << 23, 10)])
def test_probe_lds_read_validation(lib, args):
    mode, blocks, iters = args
    assert lib.jattn_probe_lds_read(mode, blocks, iters, fake(1), None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_lds_read(0, 4, 10, None, None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_lds_read(0, 4, 10, fake(1) + 4, None) == _lib.INVALID_VALUE


@pytest.mark.parametrize("args", [(7, 4, 10), (-1, 4, 10), (0, 0, 10), (0, 4, 0), (0, 1 << 22, 10)])
def test_probe_issue_validation(lib, args):
    mode, blocks, iters = args
    assert lib.jattn_probe_issue(mode, blocks, iters, ctypes.c_float(1.0), fake(0), fake(1), None) == _lib.INVALID_VALUE


def test_probe_issue_pointers(lib):
    assert lib.jattn_probe_issue(0, 4, 10, ctypes.c_float(1.0), None, fake(1), None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_issue(0, 4, 10, ctypes.c_float(1.0), fake(0), None, None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_issue(0, 4, 10, ctypes.c_float(1.0), fake(0) + 2, fake(1), None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_issue(0, 4, 10, ctypes.c_float(1.0), fake(0), fake(1) + 4, None) == _lib.INVALID_VALUE


@pytest.mark.parametrize("args", [(3, 0, 4, 10), (-1, 0, 4, 10), (0, 2, 4, 10), (0, -1, 4, 10), (0, 0, 0, 10),
                                  (0, 1, 4, 0), (2, 1, 1 << 22, 10)])
def test_probe_pingpong_validation(lib, args):
    mode, lds, blocks, iters = args
    assert lib.jattn_probe_pingpong(mode, lds, blocks, iters, ctypes.c_float(1.0), fake(0), fake(1),
                                    None) == _lib.INVALID_VALUE


def test_probe_pingpong_pointers(lib):
    f = ctypes.c_float(1.0)
    assert lib.jattn_probe_pingpong(0, 0, 4, 10, f, None, fake(1), None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_pingpong(0, 0, 4, 10, f, fake(0), None, None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_pingpong(0, 0, 4, 10, f, fake(0) + 2, fake(1), None) == _lib.INVALID_VALUE
    assert lib.jattn_probe_pingpong(0, 0, 4, 10, f, fake(0), fake(1) + 4, None) == _lib.INVALID_VALUE
