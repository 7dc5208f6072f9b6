"""Host-side validation of the adaLN-modulated QKV projection entry points (include/jattn_adaln.h):
every call here fails validation before any HIP call, so the fake device addresses are never used."""
import ctypes
import os
import re

import pytest

from diffusion_transformer_joint_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libjattn.so not built (run __graft_entry__.build())")

A, TB = 0x10000, 1 << 26


def fake(i):
    return A + i * TB


def pair(i, j):
    return _lib.PtrPair(None if i is None else fake(i), None if j is None else fake(j))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def fwd(lib, **kw):
    a = dict(x=pair(0, 1), mod=pair(2, 3), w=pair(4, 5), bias=pair(6, 7), B=2, n_img=64, n_txt=10, C=128, eps=1e-6,
             q=pair(8, 9), k=pair(10, 11), v=pair(12, 13), ws=fake(14), ws_bytes=None, events=None, n_events=0)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.jattn_adaln_qkv_fwd_workspace_bytes(a["B"], a["n_img"], a["n_txt"], a["C"])
    arg = lambda p: None if p is None else p.arg
    return lib.jattn_adaln_qkv_fwd(arg(a["x"]), arg(a["mod"]), arg(a["w"]), arg(a["bias"]), a["B"], a["n_img"],
                                   a["n_txt"], a["C"], ctypes.c_float(a["eps"]), arg(a["q"]), arg(a["k"]),
                                   arg(a["v"]), a["ws"], a["ws_bytes"], a["events"], a["n_events"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), _lib.INVALID_VALUE),
    (dict(x=pair(None, 1)), _lib.INVALID_VALUE),             # null pointer of a non-empty stream
    (dict(w=_lib.PtrPair(fake(4) + 2, fake(5))), _lib.INVALID_VALUE),  # misaligned
    (dict(B=0), _lib.INVALID_VALUE),
    (dict(n_img=-1), _lib.INVALID_VALUE),
    (dict(n_img=0, n_txt=0), _lib.INVALID_VALUE),
    (dict(C=96), _lib.INVALID_VALUE),                      # not a multiple of 64
    (dict(C=0), _lib.INVALID_VALUE),
    (dict(C=8192), _lib.NOT_SUPPORTED),
    (dict(B=1 << 20, n_img=1 << 12), _lib.NOT_SUPPORTED),  # rows * 3C past 2^31
    (dict(eps=-1.0), _lib.INVALID_VALUE),
    (dict(eps=float("nan")), _lib.INVALID_VALUE),
    (dict(ws=None), _lib.WORKSPACE),
    (dict(ws=fake(14) + 16), _lib.WORKSPACE),              # workspace not 256-byte aligned
    (dict(ws_bytes=1024), _lib.WORKSPACE),
    (dict(q=pair(0, 9)), _lib.INVALID_VALUE),              # q aliases x
    (dict(k=pair(8, 11)), _lib.INVALID_VALUE),             # k aliases q
    (dict(v=_lib.PtrPair(fake(14), fake(13))), _lib.INVALID_VALUE),  # v aliases the workspace
    (dict(n_events=-1), _lib.INVALID_VALUE),
    (dict(n_events=1), _lib.INVALID_VALUE),                # events NULL
    (dict(events=fake(20), n_events=3), _lib.INVALID_VALUE),
])
def test_fwd_rejects(lib, kw, expect):
    assert fwd(lib, **kw) == expect


def test_fwd_empty_text_stream_needs_no_text_pointers(lib):
    """With n_txt = 0 the text pointers may be NULL: the call then fails only on the (deliberately
    missing) workspace, after the pointer checks."""
    kw = dict(n_txt=0, x=pair(0, None), mod=pair(2, None), w=pair(4, None), bias=pair(6, None), q=pair(8, None),
              k=pair(10, None), v=pair(12, None))
    assert fwd(lib, ws=None, **kw) == _lib.WORKSPACE
    assert fwd(lib, x=pair(0, None), ws=None) == _lib.WORKSPACE  # (the workspace is checked first)
    assert fwd(lib, **dict(kw, x=pair(None, None))) == _lib.INVALID_VALUE


def bwd(lib, **kw):
    a = dict(x=pair(0, 1), mod=pair(2, 3), w=pair(4, 5), dq=pair(6, 7), dk=pair(8, 9), dv=pair(10, 11), B=2,
             n_img=64, n_txt=10, C=128, dx=pair(12, 13), dmod=pair(14, 15), dw=pair(16, 17), dbias=pair(18, 19),
             fws=fake(20), fws_bytes=None, ws=fake(21), ws_bytes=None, events=None, n_events=0)
    a.update(kw)
    if a["fws_bytes"] is None:
        a["fws_bytes"] = lib.jattn_adaln_qkv_fwd_workspace_bytes(a["B"], a["n_img"], a["n_txt"], a["C"])
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.jattn_adaln_qkv_bwd_workspace_bytes(a["B"], a["n_img"], a["n_txt"], a["C"])
    arg = lambda p: None if p is None else p.arg
    return lib.jattn_adaln_qkv_bwd(*(arg(a[k]) for k in ("x", "mod", "w", "dq", "dk", "dv")), a["B"], a["n_img"],
                                   a["n_txt"], a["C"], *(arg(a[k]) for k in ("dx", "dmod", "dw", "dbias")), a["fws"],
                                   a["fws_bytes"], a["ws"], a["ws_bytes"], a["events"], a["n_events"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dq=None), _lib.INVALID_VALUE),
    (dict(dbias=None), _lib.INVALID_VALUE),               # the pair itself is required (its entries may be NULL)
    (dict(dx=pair(12, None)), _lib.INVALID_VALUE),
    (dict(C=100), _lib.INVALID_VALUE),
    (dict(fws=None), _lib.WORKSPACE),
    (dict(fws_bytes=256), _lib.WORKSPACE),
    (dict(ws=None), _lib.WORKSPACE),
    (dict(ws_bytes=256), _lib.WORKSPACE),
    (dict(dx=pair(0, 13)), _lib.INVALID_VALUE),           # dx aliases x
    (dict(dw=pair(16, 16)), _lib.INVALID_VALUE),          # the two weight gradients alias
    (dict(dmod=_lib.PtrPair(fake(20), fake(15))), _lib.INVALID_VALUE),  # dmod aliases the forward workspace
    (dict(events=fake(30), n_events=6), _lib.INVALID_VALUE),
])
def test_bwd_rejects(lib, kw, expect):
    assert bwd(lib, **kw) == expect


def test_bwd_dbias_may_be_skipped(lib):
    """NULL dbias entries are allowed: such a call passes the pointer checks and fails here only on
    the deliberately small workspace."""
    assert bwd(lib, dbias=pair(None, None), ws_bytes=256) == _lib.WORKSPACE


def test_workspace_bytes(lib):
    f = lib.jattn_adaln_qkv_fwd_workspace_bytes
    b = lib.jattn_adaln_qkv_bwd_workspace_bytes
    assert f(16, 1024, 77, 768) == 16 * 1024 * 768 * 2 + (16 * 77 * 768 * 2 + 255) // 256 * 256 + \
        16 * 1024 * 8 + (16 * 77 * 8 + 255) // 256 * 256
    assert f(0, 10, 10, 128) == 0 and b(2, 10, 10, 100) == 0 and f(2, 0, 0, 128) == 0
    assert b(16, 1024, 77, 768) > 16 * 1101 * 768 * 4  # at least the fp32 input gradient of h
    assert b(2, 64, 0, 128) < b(2, 64, 10, 128)


def test_stage_counts_match_header():
    hdr = open(os.path.join(ROOT, "include", "jattn_adaln.h")).read()
    assert int(re.search(r"#define JATTN_ADALN_FWD_STAGES (\d+)", hdr).group(1)) == len(_lib.ADALN_FWD_STAGES)
    assert int(re.search(r"#define JATTN_ADALN_BWD_STAGES (\d+)", hdr).group(1)) == len(_lib.ADALN_BWD_STAGES)
