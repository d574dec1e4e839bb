"""attn_fwd_decode_noalloc, the decode entry point that allocates nothing, against
attn_fwd_decode (the same kernels with a caller-supplied workspace) and the
oracle: two calls in a row on the library's per-GPU scratch, the second with a
smaller input, each bitwise equal to attn_fwd_decode and inside the parity
gate; and a call whose partials would not fit the scratch is rejected with
nothing launched.
"""
import numpy as np
import pytest
import torch

import attention_forward_amd as A
import oracle
from attention_forward_amd.synthetic import BF16, F16, TORCH_DTYPE, bits, make_qkv
from tests.test_gpu_parity import check_lse, gate, say

pytestmark = pytest.mark.gpu


def run_both(B, Hq, Hkv, Sk, d, dtype, ns, seed):
    q, k, v = make_qkv(B, Hq, Hkv, 1, Sk, d, dtype, seed)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    t = TORCH_DTYPE[dtype]
    o_ws = torch.full((B, Hq, 1, d), float("nan"), device="cuda", dtype=t)
    l_ws = torch.full((B, Hq), float("nan"), device="cuda")
    A.attn_fwd_decode(qd, kd, vd, ns, out=o_ws, lse=l_ws)
    o_na = torch.full_like(o_ws, float("nan"))
    l_na = torch.full_like(l_ws, float("nan"))
    A.attn_fwd_decode_noalloc(qd, kd, vd, ns, out=o_na, lse=l_na)
    torch.cuda.synchronize()
    return (q, k, v), (o_ws.cpu(), l_ws.cpu()), (o_na.cpu(), l_na.cpu())


def test_two_calls_then_a_smaller_one_match_the_workspace_entry_point():
    assert A.attn_decode_scratch_bytes() == 32 << 20
    cases = [
        # the decode workload's shape (16.9 MB of partials), then a smaller call
        (64, 32, 8, 8192, 128, BF16, 16, 5),
        (2, 8, 2, 1000, 128, F16, 8, 12),
        (1, 4, 1, 300, 64, BF16, 3, 13),
    ]
    for B, Hq, Hkv, Sk, d, dtype, ns, seed in cases:
        say("case noalloc", B, Hq, Hkv, Sk, d, dtype, ns)
        (q, k, v), (o_ws, l_ws), (o_na, l_na) = run_both(B, Hq, Hkv, Sk, d, dtype, ns, seed)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), (B, Hq, Sk, d)
        rows = np.arange(B * Hq) if B * Hq <= 64 else np.sort(
            np.random.default_rng(seed).choice(B * Hq, 64, replace=False))
        o, lse, o_ref = oracle.attention_rows(bits(q), bits(k), bits(v), dtype, False,
                                              1.0 / np.sqrt(d), rows.astype(np.int64),
                                              want_ref=True)
        og = o_na.reshape(-1, d)[torch.from_numpy(rows)].double().numpy()
        gate(og, o, o_ref, np.ones(len(rows), bool), name="noalloc %s" % ((B, Hq, Sk, d),))
        check_lse(l_na.reshape(-1)[torch.from_numpy(rows)].double().numpy(), lse,
                  "noalloc lse")


def test_partials_larger_than_the_scratch_are_rejected():
    say("case noalloc too large")
    q = torch.zeros(64, 64, 1, 128, device="cuda", dtype=torch.bfloat16)
    k = torch.zeros(64, 8, 64, 128, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, float("nan"))
    assert A.attn_decode_workspace_bytes(64, 64, 128, 32) > A.attn_decode_scratch_bytes()
    with pytest.raises(A.AttnError) as e:
        A.attn_fwd_decode_noalloc(q, k, k, 32, out=o)
    assert e.value.status == A.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()
