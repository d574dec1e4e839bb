"""Long single heads against the FP64 oracle: a decode, and prefill (plain,
causal and split-KV) of 300 queries, over about 131 thousand keys, every length
ragged against the 64-key tile.

These reach four times past the longest workload (32768 keys): 2048 tiles feed
one running sum and one accumulator per row, one head's K and V are addressed
through one buffer descriptor, and the split paths merge 64 partials.  Every
output row is compared; the gate is the parity tests' gate A with the 4e-3
cap and the LSE bound.  (The oracle decodes a head's K and V to FP64 in each
thread, which is what bounds the length here.)
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_forward_amd import attn_fwd, attn_fwd_decode, attn_fwd_split
from attention_forward_amd.synthetic import BF16, F16, TORCH_DTYPE, bits, make_qkv
from tests.test_gpu_parity import check_lse, gate, say

pytestmark = pytest.mark.gpu

SK_DECODE = (1 << 17) - 1  # 2047 full tiles and one of 63 keys
SK_PREFILL = (1 << 17) + 3  # 2048 full tiles and one of 3 keys
SQ_PREFILL = 300


def test_decode_long():
    B, Hq, Hkv, ns, d = 1, 4, 1, 64, 128
    say("case decode long", (B, Hq, Hkv, SK_DECODE, ns))
    q, k, v = make_qkv(B, Hq, Hkv, 1, SK_DECODE, d, BF16, seed=901)
    scale = 1.0 / math.sqrt(d)
    o = torch.full((B, Hq, 1, d), float("nan"), device="cuda", dtype=TORCH_DTYPE[BF16])
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    attn_fwd_decode(q.cuda(), k.cuda(), v.cuda(), ns, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_, lse_, o_ref = oracle.attention(bits(q), bits(k), bits(v), BF16, False, scale)
    n = B * Hq
    gate(o.cpu().double().numpy().reshape(n, d), o_.reshape(n, d), o_ref.reshape(n, d),
         np.ones(n, bool), name="decode %d keys" % SK_DECODE)
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), "decode long")


_PREFILL = {}


def _prefill_case(causal):
    """Inputs and oracle of the long prefill, computed once per causal flag."""
    if causal not in _PREFILL:
        q, k, v = make_qkv(1, 1, 1, SQ_PREFILL, SK_PREFILL, 128, F16, seed=902 + causal)
        say("oracle for the long prefill, causal=%s" % causal)
        ref = oracle.attention(bits(q), bits(k), bits(v), F16, causal, 1.0 / math.sqrt(128))
        _PREFILL[causal] = (q, k, v) + tuple(ref)
    return _PREFILL[causal]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("split", [0, 64], ids=["fwd", "split64"])
def test_prefill_long(causal, split):
    B, H, d = 1, 1, 128
    say("case prefill long", (B, H, SQ_PREFILL, SK_PREFILL, causal, split))
    q, k, v, o_, lse_, o_ref = _prefill_case(causal)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda")
    if split:
        attn_fwd_split(qd, kd, vd, split, causal=causal, scale=scale, out=o, lse=lse)
    else:
        attn_fwd(qd, kd, vd, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    n = B * H * SQ_PREFILL
    gate(o.cpu().double().numpy().reshape(n, d), o_.reshape(n, d), o_ref.reshape(n, d),
         np.ones(n, bool), name="prefill %d x %d keys" % (SQ_PREFILL, SK_PREFILL))
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), "prefill long")
