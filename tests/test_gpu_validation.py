"""On the GPU, a call with mismatched tensors raises before anything is enqueued:
its NaN-poisoned outputs are untouched after the stream has drained, and a
correct call made afterwards still produces the right result.
"""
import pytest
import torch

import attention_forward_amd as A
from tests.test_gpu_parity import say

pytestmark = pytest.mark.gpu


def poisoned(shape, dtype):
    return torch.full(shape, float("nan"), device="cuda", dtype=dtype)


def untouched(*ts):
    torch.cuda.synchronize()
    return all(bool(torch.isnan(t.float()).all()) for t in ts)


def test_prefill_mismatch_enqueues_nothing():
    say("case validation prefill")
    q = torch.randn(1, 2, 64, 128, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(1, 2, 64, 128, device="cuda", dtype=torch.bfloat16)
    o = poisoned(q.shape, torch.bfloat16)
    lse = poisoned((1, 2, 64), torch.float32)
    bad = [
        dict(k=k[..., :64].contiguous()),                 # head dim
        dict(v=k[:, :, :32].contiguous()),                # v shorter than k
        dict(k=k.half()),                                 # dtype
        dict(out=poisoned((1, 2, 32, 128), torch.bfloat16)),  # short out
        dict(lse=poisoned((1, 2, 32), torch.float32)),    # short lse
        dict(out=poisoned(q.shape, torch.float16)),       # out dtype
    ]
    for kw in bad:
        args = dict(k=k, v=k, out=o, lse=lse)
        args.update(kw)
        with pytest.raises(A.AttnError):
            A.attn_fwd(q, args["k"], args["v"], out=args["out"], lse=args["lse"])
        assert untouched(o, lse), kw
    A.attn_fwd(q, k, k, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any() and not torch.isnan(lse).any()


def test_decode_mismatch_enqueues_nothing():
    say("case validation decode")
    q = torch.randn(2, 8, 1, 128, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(2, 2, 300, 128, device="cuda", dtype=torch.bfloat16)
    o = poisoned(q.shape, torch.bfloat16)
    lse = poisoned((2, 8), torch.float32)
    need = A.attn_decode_workspace_bytes(2, 8, 128, 4)
    bad = [
        dict(k=k[:1].contiguous(), v=k[:1].contiguous()),     # batch
        dict(v=k[:, :, :200].contiguous()),                    # v shorter than k
        dict(k=k.view(torch.uint8)[..., :128].contiguous()),   # 1-byte k
        dict(out=poisoned((2, 4, 1, 128), torch.bfloat16)),
        dict(lse=poisoned((2, 4), torch.float32)),
        dict(workspace=torch.empty(need - 256, dtype=torch.uint8, device="cuda")),
    ]
    for kw in bad:
        args = dict(k=k, v=k, out=o, lse=lse, workspace=None)
        args.update(kw)
        with pytest.raises(A.AttnError):
            A.attn_fwd_decode(q, args["k"], args["v"], 4, out=args["out"], lse=args["lse"],
                              workspace=args["workspace"])
        assert untouched(o, lse), kw
    A.attn_fwd_decode(q, k, k, 4, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any() and not torch.isnan(lse).any()


def test_combine_mismatch_enqueues_nothing():
    say("case validation combine")
    op = torch.randn(2, 3, 5, 128, device="cuda")
    lp = torch.randn(2, 3, 5, device="cuda")
    o = poisoned((2, 3, 128), torch.float16)
    lse = poisoned((2, 3), torch.float32)
    for kw in (dict(lp=lp[:, :, :4].contiguous()), dict(lp=lp.half()), dict(op=op.half())):
        a_op, a_lp = kw.get("op", op), kw.get("lp", lp)
        with pytest.raises(A.AttnError):
            A.attn_splitkv_combine(a_op, a_lp, torch.float16, out=o, lse=lse)
        assert untouched(o, lse), kw
