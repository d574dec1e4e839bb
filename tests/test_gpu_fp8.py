"""Parity of the FP8 prefill (attn_fwd_fp8, through the C ABI) with the FP64
oracle, on an MI355X.

The FP8 gate, the 16-bit gate's form with the FP8 reference in place of the
same-dtype one: a result passes iff

    max_abs(gpu - oracle) <= 2 * max_abs(ref_fp8 - oracle) + 1e-5

where the oracle is exact attention over the real (descaled) inputs and
ref_fp8 rounds the unnormalised softmax weights to E4M3 before P.V and O to
the output dtype.  LSE: |lse_gpu - lse| <= 1e-4 + 1e-6 |lse| + 2^-11 W, the
16-bit tests' bound plus the error of the scores themselves.  The FP8 matrix
unit's dot products are not correctly rounded fp32 sums: measured on random
E4M3 vectors (tests/test_gpu_mfma_precision.py, which keeps checking it), a
64-term product is off by up to 2^-11.6 of its largest single term, and two
chained ones (the 128 terms of a score) by up to 2^-12.6 of sum_i |q_i k_i|.  The LSE moves by at most the softmax-weighted mean of its
scores' errors, so W is sum_j softmax_j * |scale q_descale k_descale| *
sum_i |q_i k_ji| over the row's visible keys, and 2^-11 leaves a factor of 3
over that worst case.  (The kernel's LSE on the peaked rows below stays within
2^-16.3 W.)  Small shapes compare every row; the full-size workload sampled
rows.  Outputs are poisoned with NaN before each call.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_forward_amd import attn_fwd_fp8
from attention_forward_amd.synthetic import BF16, F16, FP8_WORKLOADS, TORCH_DTYPE, bytes_u8, make_qkv_fp8
from tests.test_gpu_parity import gate, sample_rows, say

pytestmark = pytest.mark.gpu


def gpu_fp8(q8, k8, v8, causal, scale, ds, out_dtype):
    qd, kd, vd = q8.cuda(), k8.cuda(), v8.cuda()
    B, Hq, Sq, d = q8.shape
    o = torch.full((B, Hq, Sq, d), float("nan"), device="cuda", dtype=TORCH_DTYPE[out_dtype])
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda", dtype=torch.float32)
    attn_fwd_fp8(qd, kd, vd, causal=causal, scale=scale, q_descale=ds[0], k_descale=ds[1],
                 v_descale=ds[2], out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SCORE_ERR = 2.0 ** -11  # FP8 score error allowed, relative to sum_i |q_i k_i|


def decode(t):
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def score_weight(q8, k8, ds, causal, scale, rows):
    """W per row: sum_j softmax_j |scale qd kd| sum_i |q_i k_ji| over the row's
    visible keys (0 for a row that sees none), in float64."""
    B, Hq, Sq, d = q8.shape
    Hkv, Sk = k8.shape[1], k8.shape[2]
    q = decode(q8).reshape(-1, d)
    k = decode(k8).reshape(B * Hkv, Sk, d)
    c = scale * ds[0] * ds[1]
    bh, i = rows // Sq, rows % Sq
    kvh = (bh // Hq) * Hkv + (bh % Hq) // (Hq // Hkv)
    w = np.zeros(len(rows))
    for hk in np.unique(kvh):
        sel = np.nonzero(kvh == hk)[0]
        qr = q[rows[sel]]
        s = c * (qr @ k[hk].T)
        a = abs(c) * (np.abs(qr) @ np.abs(k[hk]).T)
        if causal:
            s = np.where(np.arange(Sk)[None, :] > i[sel][:, None] + (Sk - Sq), -np.inf, s)
        mx = s.max(axis=1, keepdims=True)
        seen = np.isfinite(mx[:, 0])
        p = np.exp(s - np.where(np.isfinite(mx), mx, 0.0))
        p /= np.maximum(p.sum(axis=1, keepdims=True), 1e-300)
        w[sel] = np.where(seen, (p * a).sum(axis=1), 0.0)
    return w


def check_lse_fp8(lse_gpu, lse, w, name):
    fin = np.isfinite(lse)
    assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(lse)), "%s: -inf LSE rows differ" % name
    d = np.abs(lse_gpu[fin] - lse[fin])
    tol = 1e-4 + 1e-6 * np.abs(lse[fin]) + SCORE_ERR * w[fin]
    say("%s: lse max diff %.3e, max diff / tolerance %.3f" % (
        name, d.max() if d.size else 0.0, (d / tol).max() if d.size else 0.0))
    assert (d <= tol).all(), "%s: LSE off by %.3e" % (name, d.max())


FP8_SMALL = [
    # B, Hq, Hkv, Sq, Sk, out dtype, causal
    (1, 1, 1, 1, 1, BF16, False),
    (1, 2, 2, 64, 64, BF16, False),
    (1, 2, 2, 200, 200, F16, False),
    (1, 2, 2, 333, 333, BF16, True),
    (2, 8, 2, 130, 257, BF16, False),
    (1, 4, 1, 100, 300, F16, True),
    (1, 2, 2, 300, 100, BF16, True),
    (1, 2, 2, 1, 700, BF16, False),
    (1, 3, 3, 129, 63, F16, True),
    (2, 4, 4, 640, 640, BF16, True),
    (1, 2, 1, 513, 1000, F16, False),
    (1, 16, 8, 2200, 2200, BF16, True),  # more items than a 256-CU grid, XCD-grouped order
]


def check(q8, k8, v8, ds, causal, scale, out_dtype, name, rows=None):
    B, Hq, Sq, d = q8.shape
    o_gpu, lse_gpu = gpu_fp8(q8, k8, v8, causal, scale, ds, out_dtype)
    assert not torch.isnan(o_gpu).any(), "unwritten output elements"
    assert not torch.isnan(lse_gpu).any(), "unwritten LSE elements"
    if rows is None:
        rows = np.arange(B * Hq * Sq, dtype=np.int64)
    o, lse, o_ref = oracle.attention_fp8_rows(bytes_u8(q8), bytes_u8(k8), bytes_u8(v8), causal,
                                              scale, ds[0], ds[1], ds[2], out_dtype, rows)
    og = o_gpu.reshape(-1, d)[torch.from_numpy(rows)].double().numpy()
    gate(og, o, o_ref, name=name)
    check_lse_fp8(lse_gpu.reshape(-1)[torch.from_numpy(rows)].double().numpy(), lse,
                  score_weight(q8, k8, ds, causal, scale, rows), name)
    return o_gpu


@pytest.mark.parametrize("shape", FP8_SMALL, ids=lambda s: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s" % (
    s[0], s[1], s[2], s[3], s[4], "bf16" if s[5] else "f16", "causal" if s[6] else "full"))
def test_fp8_small_all_rows(shape):
    B, Hq, Hkv, Sq, Sk, out_dtype, causal = shape
    name = "fp8 %s" % (shape,)
    say("case", name)
    (q8, k8, v8), ds = make_qkv_fp8(B, Hq, Hkv, Sq, Sk, 128, seed=400 + Sq + Sk)
    o_gpu = check(q8, k8, v8, ds, causal, 1.0 / math.sqrt(128), out_dtype, name)
    if causal and Sq > Sk:
        assert torch.all(o_gpu[:, :, : Sq - Sk] == 0), "fully masked rows must be exactly zero"


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fp8_growing_scores_and_descales(causal):
    """Key norms grow along the sequence (the reference max moves mid-loop), and
    the descales are far from 1 on both sides."""
    B, H, S = 1, 2, 1000
    name = "fp8 growing scores %s" % ("causal" if causal else "full")
    say("case", name)
    gen = torch.Generator().manual_seed(79)
    x = [torch.randn((B, H, S, 128), generator=gen) for _ in range(3)]
    x[1] = x[1] * torch.linspace(1.0, 6.0, S).view(1, 1, S, 1)
    from attention_forward_amd.synthetic import _quantise_e4m3

    (q8, qd), (k8, kd), (v8, vd) = [_quantise_e4m3(t * f) for t, f in zip(x, (0.01, 30.0, 500.0))]
    check(q8, k8, v8, (qd, kd, vd), causal, 1.0 / math.sqrt(128), BF16, name)


@pytest.mark.parametrize("out_dtype", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fp8_peaked_rows(causal, out_dtype):
    """Scores spread over about 38 exponent steps per row, with the top keys in
    the last tiles: a row's result rests on a few weights, so a weight taken
    against a reference below the row max, and rounded to E4M3 there, would
    show (see the gate calibration's peaked inputs)."""
    from tests.test_gate_fp8 import inputs

    name = "fp8 peaked rows %s" % ("causal" if causal else "full")
    say("case", name)
    (q8, k8, v8), ds = inputs(True, 41)
    check(q8, k8, v8, ds, causal, 1.0 / math.sqrt(128), out_dtype, name)


@pytest.mark.parametrize("wname", list(FP8_WORKLOADS))
def test_fp8_workload(wname):
    w = FP8_WORKLOADS[wname]
    say("case workload", wname)
    (q8, k8, v8), ds = make_qkv_fp8(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.seed)
    rows = sample_rows(w.B, w.Hq, w.Sq, np.random.default_rng(w.seed), 1024)
    check(q8, k8, v8, ds, w.causal, w.scale, w.dtype, wname, rows)


def test_fp8_repeat_runs_are_bitwise_identical():
    say("case fp8 determinism")
    (q8, k8, v8), ds = make_qkv_fp8(2, 4, 4, 1024, 1024, 128, seed=9)
    outs = [gpu_fp8(q8, k8, v8, True, 0.088, ds, BF16) for _ in range(3)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
