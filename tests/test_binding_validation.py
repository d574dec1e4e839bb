"""The Python binding rejects mismatched tensors before anything is launched.

The C ABI sees only pointers and sizes, so a k with another batch or head
dimension than q, a v of another shape, an output buffer of the wrong size or
dtype would make the kernels read or write past the caller's buffers.  Each
wrapper checks shapes, dtypes, devices and contiguity first; these tests use
host tensors (the shape and dtype checks run before the device check) and a
stand-in library that fails the test if any launching entry point is reached.
"""
import pytest
import torch

import attention_forward_amd as A

LAUNCHING = ("attn_fwd", "attn_fwd_fp8", "attn_fwd_split", "attn_fwd_decode",
             "attn_splitkv_combine")


class _NoLaunch:
    """Sizing helpers answer; launching entry points fail the test."""

    def __getattr__(self, name):
        if name in LAUNCHING:
            def launch(*args):
                raise AssertionError("%s was called" % name)
            return launch
        if name == "attn_fwd_num_splits":
            return lambda *a: 2
        if name in ("attn_fwd_split_workspace_bytes", "attn_decode_workspace_bytes"):
            return lambda *a: 4096
        if name == "attn_last_error":
            return lambda: b""
        raise AttributeError(name)


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    monkeypatch.setattr(A, "_lib", _NoLaunch())


F16, BF16, F32 = torch.float16, torch.bfloat16, torch.float32


def t(*shape, dtype=F16):
    return torch.zeros(*shape, dtype=dtype)


def status_of(fn, *args, **kw):
    with pytest.raises(A.AttnError) as e:
        fn(*args, **kw)
    return e.value.status


Q = (2, 4, 8, 128)
KV = (2, 2, 16, 128)


@pytest.mark.parametrize("q,k,v,kw,status", [
    (t(*Q), t(1, 2, 16, 128), t(1, 2, 16, 128), {}, A.ATTN_ERR_SHAPE),      # batch
    (t(*Q), t(2, 2, 16, 64), t(2, 2, 16, 64), {}, A.ATTN_ERR_SHAPE),        # head dim
    (t(*Q), t(*KV), t(2, 2, 17, 128), {}, A.ATTN_ERR_SHAPE),                # v vs k
    (t(*Q), t(*KV), t(2, 1, 16, 128), {}, A.ATTN_ERR_SHAPE),
    (t(2, 4, 128), t(*KV), t(*KV), {}, A.ATTN_ERR_SHAPE),                   # rank
    (t(*Q), t(*KV, dtype=BF16), t(*KV), {}, A.ATTN_ERR_UNSUPPORTED),        # k dtype
    (t(*Q), t(*KV), t(*KV, dtype=torch.uint8), {}, A.ATTN_ERR_UNSUPPORTED),  # 1-byte v
    (t(*Q, dtype=F32), t(*KV, dtype=F32), t(*KV, dtype=F32), {}, A.ATTN_ERR_UNSUPPORTED),
    (t(*Q), t(*KV), t(*KV), dict(out=t(2, 4, 9, 128)), A.ATTN_ERR_SHAPE),   # out shape
    (t(*Q), t(*KV), t(*KV), dict(out=t(*Q, dtype=BF16)), A.ATTN_ERR_UNSUPPORTED),
    (t(*Q), t(*KV), t(*KV), dict(lse=t(2, 4, 7, dtype=F32)), A.ATTN_ERR_SHAPE),
    (t(*Q), t(*KV), t(*KV), dict(lse=t(2, 4, 8)), A.ATTN_ERR_UNSUPPORTED),  # fp16 lse
    (t(*Q), t(*KV), t(*KV), {}, A.ATTN_ERR_VALUE),                          # host tensors
])
@pytest.mark.parametrize("entry", ["fwd", "split"])
def test_prefill_rejects(entry, q, k, v, kw, status):
    fn = A.attn_fwd if entry == "fwd" else A.attn_fwd_split
    assert status_of(fn, q, k, v, **kw) == status


def test_split_rejects_a_wrong_out_before_the_workspace():
    q, k = t(*Q), t(*KV)
    ws = t(100, dtype=torch.uint8)
    assert status_of(A.attn_fwd_split, q, k, k, out=t(2, 4, 8, 64), workspace=ws) \
        == A.ATTN_ERR_SHAPE


def test_non_contiguous_is_rejected_after_shape_checks():
    q = t(2, 4, 128, 8).transpose(2, 3)          # right shape, wrong strides
    assert status_of(A.attn_fwd, q, t(*KV), t(*KV)) == A.ATTN_ERR_VALUE


DQ = (2, 8, 1, 128)
DKV = (2, 2, 100, 128)


@pytest.mark.parametrize("q,k,v,kw,status", [
    (t(*DQ), t(3, 2, 100, 128), t(3, 2, 100, 128), {}, A.ATTN_ERR_SHAPE),   # batch
    (t(*DQ), t(2, 2, 100, 64), t(2, 2, 100, 64), {}, A.ATTN_ERR_SHAPE),     # head dim
    (t(*DQ), t(*DKV), t(2, 2, 99, 128), {}, A.ATTN_ERR_SHAPE),             # v vs k (Sk)
    (t(*DQ), t(*DKV), t(2, 1, 100, 128), {}, A.ATTN_ERR_SHAPE),            # v vs k (Hkv)
    (t(2, 8, 2, 128), t(*DKV), t(*DKV), {}, A.ATTN_ERR_SHAPE),             # Sq != 1
    (t(*DQ), t(*DKV, dtype=torch.uint8), t(*DKV, dtype=torch.uint8), {}, A.ATTN_ERR_UNSUPPORTED),
    (t(*DQ, dtype=BF16), t(*DKV), t(*DKV), {}, A.ATTN_ERR_UNSUPPORTED),
    (t(*DQ), t(*DKV), t(*DKV), dict(out=t(2, 8, 128)), A.ATTN_ERR_SHAPE),
    (t(*DQ), t(*DKV), t(*DKV), dict(out=t(*DQ, dtype=BF16)), A.ATTN_ERR_UNSUPPORTED),
    (t(*DQ), t(*DKV), t(*DKV), dict(lse=t(2, 8, 1, dtype=F32)), A.ATTN_ERR_SHAPE),
    (t(*DQ), t(*DKV), t(*DKV), dict(lse=t(2, 8, dtype=torch.float64)), A.ATTN_ERR_UNSUPPORTED),
    (t(*DQ), t(*DKV), t(*DKV), {}, A.ATTN_ERR_VALUE),                      # host tensors
])
def test_decode_rejects(q, k, v, kw, status):
    assert status_of(A.attn_fwd_decode, q, k, v, 4, **kw) == status


E8 = torch.float8_e4m3fn


@pytest.mark.parametrize("q,k,v,kw,status", [
    (t(*Q, dtype=E8), t(1, 2, 16, 128, dtype=E8), t(1, 2, 16, 128, dtype=E8), {},
     A.ATTN_ERR_SHAPE),
    (t(*Q, dtype=E8), t(*KV, dtype=E8), t(2, 2, 15, 128, dtype=E8), {}, A.ATTN_ERR_SHAPE),
    (t(*Q, dtype=E8), t(*KV), t(*KV, dtype=E8), {}, A.ATTN_ERR_UNSUPPORTED),       # 2-byte k
    (t(*Q, dtype=torch.float8_e5m2), t(*KV, dtype=E8), t(*KV, dtype=E8), {},
     A.ATTN_ERR_UNSUPPORTED),                                                     # E5M2 q
    (t(*Q, dtype=E8), t(*KV, dtype=E8), t(*KV, dtype=E8), dict(out=t(2, 4, 8, 64)),
     A.ATTN_ERR_SHAPE),
    (t(*Q, dtype=E8), t(*KV, dtype=E8), t(*KV, dtype=E8), dict(out_dtype=F32),
     A.ATTN_ERR_UNSUPPORTED),
    (t(*Q, dtype=E8), t(*KV, dtype=E8), t(*KV, dtype=E8), dict(lse=t(2, 4, 8)),
     A.ATTN_ERR_UNSUPPORTED),
    (t(*Q, dtype=E8), t(*KV, dtype=E8), t(*KV, dtype=E8), {}, A.ATTN_ERR_VALUE),
])
def test_fp8_rejects(q, k, v, kw, status):
    assert status_of(A.attn_fwd_fp8, q, k, v, **kw) == status


@pytest.mark.parametrize("op,lp,kw,status", [
    (t(2, 3, 5, 128, dtype=F16), t(2, 3, 5, dtype=F32), {}, A.ATTN_ERR_UNSUPPORTED),
    (t(2, 3, 5, 128, dtype=F32), t(2, 3, 5, dtype=F16), {}, A.ATTN_ERR_UNSUPPORTED),
    (t(2, 3, 5, 128, dtype=F32), t(2, 3, 4, dtype=F32), {}, A.ATTN_ERR_SHAPE),
    (t(2, 3, 5, 128, dtype=F32), t(2, 3, dtype=F32), {}, A.ATTN_ERR_SHAPE),
    (t(2, 3, 5, 128, dtype=F32), t(2, 3, 5, dtype=F32), dict(out=t(2, 3, 64)), A.ATTN_ERR_SHAPE),
    (t(2, 3, 5, 128, dtype=F32), t(2, 3, 5, dtype=F32), dict(lse=t(2, 3, 5, dtype=F32)),
     A.ATTN_ERR_SHAPE),
    (t(2, 3, 5, 128, dtype=F32), t(2, 3, 5, dtype=F32), {}, A.ATTN_ERR_VALUE),
])
def test_combine_rejects(op, lp, kw, status):
    assert status_of(A.attn_splitkv_combine, op, lp, F16, **kw) == status


def test_combine_rejects_output_dtype():
    op, lp = t(2, 3, 5, 128, dtype=F32), t(2, 3, 5, dtype=F32)
    assert status_of(A.attn_splitkv_combine, op, lp, F32) == A.ATTN_ERR_UNSUPPORTED
