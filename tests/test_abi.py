"""The C ABI without a GPU: the library loads, exports every function include/attn.h
declares, and rejects bad arguments with the documented status before touching
HIP.  Fake (non-NULL) pointers are only passed when no GPU is visible, so a
validation bug can never turn into a kernel launch on bad memory.
"""
import ctypes
import os
import re

import pytest
import torch

import attention_forward_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NO_GPU = torch.cuda.device_count() == 0
cpu_only = pytest.mark.skipif(not NO_GPU, reason="passes fake device pointers; CPU hosts only")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(A.LIB_PATH):
        from attention_forward_amd import build

        build.build()
    return A.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_bound_functions():
    assert declared_functions() == sorted(A.EXPORTED)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_null_pointers(L):
    assert L.attn_fwd(None, None, None, None, None, 1, 1, 1, 1, 1, 128, 0, 1.0, 0, None) == A.ATTN_ERR_NULL
    assert "non-NULL" in A.last_error()
    assert L.attn_splitkv_combine(None, None, None, None, 1, 1, 128, 1, 0, None) == A.ATTN_ERR_NULL
    assert L.attn_fwd_decode(None, None, None, None, None, 1, 1, 1, 1, 128, 1.0, 0, 1, None, 0,
                             None) == A.ATTN_ERR_NULL


P = ctypes.c_void_p(1 << 20)  # aligned, non-NULL, never dereferenced


def fwd(L, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Sq=8, Sk=8, d=128, causal=0,
             scale=0.1, dtype=0)
    a.update(kw)
    return L.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                      a["Sk"], a["d"], a["causal"], a["scale"], a["dtype"], None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), A.ATTN_ERR_SHAPE), (dict(Sq=-1), A.ATTN_ERR_SHAPE), (dict(Sk=0), A.ATTN_ERR_SHAPE),
    (dict(Hq=3, Hkv=2), A.ATTN_ERR_SHAPE), (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(d=32), A.ATTN_ERR_UNSUPPORTED), (dict(d=64), A.ATTN_ERR_NO_DEVICE),
    (dict(dtype=2), A.ATTN_ERR_UNSUPPORTED), (dict(causal=2), A.ATTN_ERR_VALUE),
    (dict(scale=-1.0), A.ATTN_ERR_VALUE), (dict(scale=float("nan")), A.ATTN_ERR_VALUE),
    (dict(scale=float("inf")), A.ATTN_ERR_VALUE),
    (dict(q=ctypes.c_void_p((1 << 20) + 8)), A.ATTN_ERR_ALIGN),
    (dict(lse=ctypes.c_void_p((1 << 20) + 2)), A.ATTN_ERR_ALIGN),
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, Sq=1 << 20), A.ATTN_ERR_SHAPE),
    (dict(Sk=1 << 24), A.ATTN_ERR_SHAPE), (dict(Sq=1 << 24), A.ATTN_ERR_SHAPE),
    (dict(), A.ATTN_ERR_NO_DEVICE),
])
def test_fwd_validation(L, kw, status):
    assert fwd(L, **kw) == status
    assert A.last_error() != ""


def dec(L, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=2, Hq=8, Hkv=2, Sk=100, d=128, scale=0.1, dtype=1,
             ns=4, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.attn_fwd_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                             a["Sk"], a["d"], a["scale"], a["dtype"], a["ns"], a["ws"], a["wsb"],
                             None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(Hq=7), A.ATTN_ERR_SHAPE), (dict(Hq=66, Hkv=2), A.ATTN_ERR_UNSUPPORTED),
    (dict(ns=0), A.ATTN_ERR_VALUE), (dict(ns=101), A.ATTN_ERR_VALUE),
    (dict(wsb=16), A.ATTN_ERR_WORKSPACE), (dict(ws=None), A.ATTN_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 4)), A.ATTN_ERR_ALIGN), (dict(d=256), A.ATTN_ERR_UNSUPPORTED),
    (dict(d=64), A.ATTN_ERR_NO_DEVICE),
    (dict(scale=-0.5), A.ATTN_ERR_VALUE), (dict(Sk=1 << 24, ns=4), A.ATTN_ERR_SHAPE),
    (dict(), A.ATTN_ERR_NO_DEVICE),
])
def test_decode_validation(L, kw, status):
    assert dec(L, **kw) == status


def f8(L, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Sq=8, Sk=8, d=128, causal=0,
             scale=0.1, qd=1.0, kd=1.0, vd=1.0, dtype=1)
    a.update(kw)
    return L.attn_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["qd"], a["kd"],
                          a["vd"], a["dtype"], None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), A.ATTN_ERR_NULL), (dict(B=0), A.ATTN_ERR_SHAPE),
    (dict(Hq=3, Hkv=2), A.ATTN_ERR_SHAPE), (dict(d=64), A.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=2), A.ATTN_ERR_UNSUPPORTED), (dict(causal=3), A.ATTN_ERR_VALUE),
    (dict(scale=-1.0), A.ATTN_ERR_VALUE), (dict(qd=0.0), A.ATTN_ERR_VALUE),
    (dict(kd=-2.0), A.ATTN_ERR_VALUE), (dict(vd=float("inf")), A.ATTN_ERR_VALUE),
    (dict(qd=1e30, kd=1e30), A.ATTN_ERR_VALUE),
    (dict(v=ctypes.c_void_p((1 << 20) + 4)), A.ATTN_ERR_ALIGN),
    (dict(Sk=1 << 24), A.ATTN_ERR_SHAPE), (dict(dtype=0), A.ATTN_ERR_NO_DEVICE),
    (dict(causal=1), A.ATTN_ERR_NO_DEVICE), (dict(), A.ATTN_ERR_NO_DEVICE),
])
def test_fp8_validation(L, kw, status):
    assert f8(L, **kw) == status
    assert A.last_error() != ""


def spl(L, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Sq=300, Sk=500, d=128, causal=0,
             scale=0.1, dtype=0, ns=4, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.attn_fwd_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["dtype"], a["ns"],
                            a["ws"], a["wsb"], None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), A.ATTN_ERR_NULL), (dict(B=0), A.ATTN_ERR_SHAPE),
    (dict(Hq=3, Hkv=2), A.ATTN_ERR_SHAPE), (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=3), A.ATTN_ERR_UNSUPPORTED), (dict(causal=-1), A.ATTN_ERR_VALUE),
    (dict(scale=float("nan")), A.ATTN_ERR_VALUE),
    # 500 keys are 8 tiles of 64: 1..8 splits are valid
    (dict(ns=0), A.ATTN_ERR_VALUE), (dict(ns=9), A.ATTN_ERR_VALUE), (dict(ns=8), A.ATTN_ERR_NO_DEVICE),
    (dict(wsb=16), A.ATTN_ERR_WORKSPACE), (dict(ws=None), A.ATTN_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 4)), A.ATTN_ERR_ALIGN),
    (dict(o=ctypes.c_void_p((1 << 20) + 8)), A.ATTN_ERR_ALIGN),
    (dict(Sk=1 << 24, ns=4), A.ATTN_ERR_SHAPE), (dict(d=64), A.ATTN_ERR_NO_DEVICE),
    (dict(causal=1), A.ATTN_ERR_NO_DEVICE), (dict(), A.ATTN_ERR_NO_DEVICE),
])
def test_split_validation(L, kw, status):
    assert spl(L, **kw) == status
    assert A.last_error() != ""


def test_split_workspace_and_recommendation(L):
    # fp32 partial O [B,Hq,Sq,S,d] then fp32 partial LSE [B,Hq,Sq,S], each 256-byte aligned
    assert A.attn_fwd_split_workspace_bytes(1, 1, 512, 128, 8) == 512 * 8 * 128 * 4 + 512 * 8 * 4
    assert A.attn_fwd_split_workspace_bytes(1, 1, 3, 64, 1) == 768 + 256
    assert A.attn_fwd_split_workspace_bytes(1, 0, 3, 64, 1) == 0
    # 2 blocks of 256 rows, 8 tiles of keys: 128 splits wanted, two tiles per split -> 4
    assert A.attn_fwd_num_splits(1, 1, 512, 512, 128) == 4
    # 1 block, 128 tiles: 256 splits wanted -> 64 (two tiles each)
    assert A.attn_fwd_num_splits(1, 1, 100, 8192, 128) == 64
    # 16 blocks, 32 tiles: 16 splits wanted, 16 allowed
    assert A.attn_fwd_num_splits(1, 2, 2048, 2048, 128) == 16
    # a single tile cannot be split
    assert A.attn_fwd_num_splits(1, 1, 64, 64, 128) == 1
    assert A.attn_fwd_num_splits(1, 1, 64, 100, 128) == 1
    # already 256 items or more: no split
    assert A.attn_fwd_num_splits(4, 16, 1024, 1024, 128) == 1
    assert A.attn_fwd_num_splits(2, 16, 2048, 2048, 64) == 1
    assert A.attn_fwd_num_splits(1, 16, 2048, 2048, 64) == 2
    assert A.attn_fwd_num_splits(0, 16, 2048, 2048, 64) == 1


@cpu_only
def test_combine_validation(L):
    assert L.attn_splitkv_combine(P, P, P, None, 1, 1, 128, 0, 0, None) == A.ATTN_ERR_VALUE
    assert L.attn_splitkv_combine(P, P, P, None, 1, 1, 128, 2, 5, None) == A.ATTN_ERR_UNSUPPORTED
    assert L.attn_splitkv_combine(P, P, P, None, 0, 1, 128, 2, 0, None) == A.ATTN_ERR_SHAPE
    assert L.attn_splitkv_combine(P, P, P, None, 1, 1, 128, 2, 0, None) == A.ATTN_ERR_NO_DEVICE
    assert L.attn_splitkv_combine(P, P, P, None, 1, 1, 64, 2, 0, None) == A.ATTN_ERR_NO_DEVICE
    assert L.attn_splitkv_combine(P, P, P, None, 1, 1, 80, 2, 0, None) == A.ATTN_ERR_UNSUPPORTED


def test_workspace_size(L):
    # fp32 partial O [B,Hq,S,d] then fp32 partial LSE [B,Hq,S], each 256-byte aligned
    n = A.attn_decode_workspace_bytes(64, 32, 128, 16)
    assert n == 64 * 32 * 16 * 128 * 4 + 64 * 32 * 16 * 4
    assert A.attn_decode_workspace_bytes(1, 1, 128, 3) == 1536 + 256
    assert A.attn_decode_workspace_bytes(0, 1, 128, 3) == 0


def test_binding_rejects_host_tensors():
    q = torch.zeros(1, 1, 4, 128, dtype=torch.float16)
    with pytest.raises(A.AttnError):
        A.attn_fwd(q, q, q)


@cpu_only
def test_noalloc_decode_validation(L):
    """The no-allocation decode validates as attn_fwd_decode does, and rejects
    partials larger than its fixed scratch before any HIP call."""
    def na(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=None, B=2, Hq=8, Hkv=2, Sk=100, d=128, scale=0.1,
                 dtype=1, ns=4)
        a.update(kw)
        return L.attn_fwd_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                         a["Hq"], a["Hkv"], a["Sk"], a["d"], a["scale"],
                                         a["dtype"], a["ns"], None)
    assert A.attn_decode_scratch_bytes() == 32 << 20
    assert na(q=None) == A.ATTN_ERR_NULL
    assert na(Hq=7) == A.ATTN_ERR_SHAPE
    assert na(ns=101) == A.ATTN_ERR_VALUE
    assert na(d=96) == A.ATTN_ERR_UNSUPPORTED
    # 64 x 64 rows x 32 splits x 128 fp32 = 64 MiB of partials > 32 MiB
    assert na(B=64, Hq=64, Hkv=8, Sk=8192, ns=32) == A.ATTN_ERR_WORKSPACE
    assert "scratch" in A.last_error()
    assert na() == A.ATTN_ERR_NO_DEVICE
