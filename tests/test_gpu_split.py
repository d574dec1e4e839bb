"""Parity of the split-KV prefill (attn_fwd_split, through the C ABI) with the
FP64 oracle, on an MI355X, under the same gate as attn_fwd (see
test_gpu_parity.py): every row of small shapes, split counts from 1 to one per
64-key tile (so ranges hold one tile, several, a ragged tail, or nothing
visible under the causal mask), both head dimensions, a moving reference max
inside a split, and the under-filled workload (B=1, H=1, S=512) with the
recommended split count.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_forward_amd import attn_fwd_num_splits, attn_fwd_split
from attention_forward_amd.synthetic import ALL_WORKLOADS, BF16, F16, TORCH_DTYPE, bits, make_qkv
from tests.test_gpu_parity import check_lse, gate, say

pytestmark = pytest.mark.gpu


def gpu_split(q, k, v, causal, scale, ns):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    attn_fwd_split(qd, kd, vd, ns, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(q, k, v, dtype, causal, scale, ns, name, cap=False):
    B, Hq, Sq, d = q.shape
    Sk = k.shape[2]
    o_gpu, lse_gpu = gpu_split(q, k, v, causal, scale, ns)
    o, lse, o_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, causal, scale)
    n = B * Hq * Sq
    gate(o_gpu.to(torch.float64).numpy().reshape(n, d), o.reshape(n, d), o_ref.reshape(n, d),
         np.ones(n, bool) if cap else None, name=name)
    check_lse(lse_gpu.to(torch.float64).numpy().reshape(-1), lse.reshape(-1), name)
    if causal and Sq > Sk:
        assert torch.all(o_gpu[:, :, : Sq - Sk] == 0), "fully masked rows must be exactly zero"


SPLIT_SMALL = [
    # B, Hq, Hkv, Sq, Sk, dtype, causal, d, splits
    (1, 1, 1, 1, 1, F16, False, 128, (1,)),
    (1, 2, 2, 64, 64, BF16, False, 128, (1,)),
    (1, 2, 2, 200, 200, F16, False, 128, (1, 2, 4)),
    (1, 2, 2, 333, 333, BF16, True, 128, (2, 3, 6)),
    (2, 8, 2, 130, 257, BF16, False, 128, (2, 5)),
    (1, 4, 1, 100, 300, F16, True, 128, (3, 5)),
    (1, 2, 2, 300, 100, BF16, True, 128, (2,)),
    (1, 2, 2, 1, 700, BF16, False, 128, (4, 11)),
    (1, 3, 3, 129, 63, F16, True, 128, (1,)),
    (2, 4, 4, 640, 640, F16, True, 128, (3, 10)),
    (1, 2, 1, 513, 1000, BF16, False, 128, (7, 16)),
    (1, 2, 2, 333, 333, F16, True, 64, (2, 6)),
    (2, 8, 2, 130, 257, BF16, False, 64, (3, 5)),
    (1, 2, 2, 300, 100, F16, True, 64, (2,)),
    (2, 4, 4, 640, 640, BF16, True, 64, (4, 10)),
]


@pytest.mark.parametrize("shape", [s[:8] + (ns,) for s in SPLIT_SMALL for ns in s[8]],
                         ids=lambda s: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s_d%d_ns%d" % (
    s[0], s[1], s[2], s[3], s[4], "bf16" if s[5] else "f16", "causal" if s[6] else "full",
    s[7], s[8]))
def test_split_small_all_rows(shape):
    B, Hq, Hkv, Sq, Sk, dtype, causal, d, ns = shape
    name = "split %s" % (shape,)
    say("case", name)
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype, seed=300 + Sq + Sk + d + ns)
    check(q, k, v, dtype, causal, 1.0 / math.sqrt(d), ns, name)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_split_growing_scores(causal, d):
    """Key norms grow along the sequence: the reference max of every split moves
    inside it, and the merge has to reconcile very different partial LSEs."""
    B, H, S, dtype, ns = 1, 2, 1000, BF16, 3
    name = "split growing scores %s d%d" % ("causal" if causal else "full", d)
    say("case", name)
    q, k, v = make_qkv(B, H, H, S, S, d, dtype, seed=78)
    ramp = torch.linspace(1.0, 6.0, S).view(1, 1, S, 1)
    k = (k.float() * ramp).to(TORCH_DTYPE[dtype])
    check(q, k, v, dtype, causal, 1.0 / math.sqrt(d), ns, name)


def test_split_underfilled_workload():
    w = ALL_WORKLOADS["fwd_f16_b1_h1_s512"]
    ns = attn_fwd_num_splits(w.B, w.Hq, w.Sq, w.Sk, w.d)
    say("case workload", w.name, "splits", ns)
    assert ns > 1
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.dtype, w.seed)
    check(q, k, v, w.dtype, w.causal, w.scale, ns, w.name + " split", cap=True)
