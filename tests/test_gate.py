"""Calibration of the correctness gate (CPU only).

A numpy model of the kernels' numerics -- 64-key tiles, scores and sums in
fp32, exp2 domain with scale*log2(e) folded into one multiply, the threshold
rescale (tau = 8), P rounded to the input dtype before P.V, O rounded at the
end -- must pass gate A against the FP64 oracle:

    max_abs(model - oracle) <= 2 * max_abs(ref_dtype - oracle) + 1e-5.

Each plausible kernel defect injected into the model must fail it, by a wide
margin (the pages calibrate their gate the same way: an injected bug sits far
outside the bound, "The FA5090 Optimization Journey", sec. 2.1):
the rescale dropped, the causal mask off by one, the GQA head mapping wrong,
P and V permuted differently, the last tile missing, uniform weights instead
of the softmax.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_forward_amd.synthetic import BF16, F16, TORCH_DTYPE, bits, make_qkv

TAU = 8.0
KT = 64


def rnd(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        TORCH_DTYPE[dtype]).to(torch.float32).numpy()


def kernel_model(q, k, v, dtype, causal, scale, defect=None):
    """q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] (float32 holding dtype values) -> O [B,Hq,Sq,d]."""
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sl2 = np.float32(scale * 1.4426950408889634)
    off = Sk - Sq + (1 if defect == "causal_off_by_one" else 0)
    out = np.zeros_like(q)
    n_tiles = (Sk + KT - 1) // KT
    if defect == "last_tile_missing":
        n_tiles -= 1
    rows = np.arange(Sq)
    for b in range(B):
        for h in range(Hq):
            hk = h % Hkv if defect == "gqa_mapping" else h // G
            m = np.full(Sq, -np.inf, np.float32)
            l = np.zeros(Sq, np.float32)
            acc = np.zeros((Sq, d), np.float32)
            for t in range(n_tiles):
                j0, j1 = t * KT, min(Sk, t * KT + KT)
                keys = np.arange(j0, j1)
                s = (q[b, h] @ k[b, hk, j0:j1].T).astype(np.float32)
                hidden = np.zeros(s.shape, bool)
                if causal:
                    hidden = keys[None, :] > rows[:, None] + off
                x = np.where(hidden, -np.inf, s * sl2).astype(np.float32)
                mx = x.max(axis=1)
                jump = mx > m + TAU
                alpha = np.where(jump, np.exp2(np.where(jump, m - mx, 0)), 1).astype(np.float32)
                m = np.where(jump, mx, m)
                m_eff = np.where(np.isneginf(m), 0, m).astype(np.float32)
                p = np.where(hidden, 0, np.exp2(x - m_eff[:, None])).astype(np.float32)
                if defect == "uniform_weights":
                    p = np.where(hidden, 0, 1).astype(np.float32)
                l = (l * alpha + p.sum(axis=1)).astype(np.float32)
                vt = v[b, hk, j0:j1]
                if defect == "pv_permutation":
                    vt = vt[::-1]
                if defect != "rescale_dropped":
                    acc = acc * alpha[:, None]
                acc = (acc + rnd(p, dtype) @ vt).astype(np.float32)
            o = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1)[:, None], 0)
            out[b, h] = rnd(o, dtype)
    return out


def inputs(dtype, growing, seed):
    B, Hq, Hkv, Sq, Sk, d = 1, 4, 2, 200, 300, 64
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype, seed)
    if growing:  # later keys' scores pass the first tile's max by far more than tau
        k = (k.float() * torch.linspace(1.0, 6.0, Sk).view(1, 1, Sk, 1)).to(TORCH_DTYPE[dtype])
    return q, k, v


def gate_ratio(q, k, v, dtype, causal, defect):
    scale = 1.0 / math.sqrt(q.shape[-1])
    o, _, o_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, causal, scale)
    model = kernel_model(q.float().numpy(), k.float().numpy(), v.float().numpy(), dtype, causal,
                         scale, defect)
    err = np.abs(model - o).max()
    bound = 2.0 * np.abs(o_ref - o).max() + 1e-5
    return err / bound


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("growing", [False, True], ids=["random", "growing"])
def test_kernel_model_passes_the_gate(dtype, causal, growing):
    r = gate_ratio(*inputs(dtype, growing, 31), dtype, causal, None)
    assert r <= 1.0, r


DEFECTS = [
    # defect, needs growing scores, needs the causal mask
    ("rescale_dropped", True, False),
    ("causal_off_by_one", False, True),
    ("gqa_mapping", False, False),
    ("pv_permutation", False, False),
    ("last_tile_missing", False, False),
    ("uniform_weights", False, False),
]


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("defect,growing,causal", DEFECTS, ids=[d[0] for d in DEFECTS])
def test_injected_defect_fails_the_gate_by_a_wide_margin(defect, growing, causal, dtype):
    r = gate_ratio(*inputs(dtype, growing, 32), dtype, causal, defect)
    assert r > 5.0, (defect, r)


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_kernel_model_passes_the_gate_on_peaked_rows(dtype, causal):
    """The FP8 calibration's peaked rows (scores spread over ~38 exponent steps,
    top keys in the last tiles), as 16-bit inputs.  There the threshold rule
    leaves a row's top weight up to 2^8 off the exact max, which in E4M3 costs
    up to 1/16 of it and fails the FP8 gate; rounded to 16 bits it costs at most
    2^-9, and the model stays inside the 16-bit gate."""
    from tests.test_gate_fp8 import e4m3, inputs as fp8_inputs

    (q8, k8, v8), (qd, kd, vd) = fp8_inputs(True, 41)
    t = TORCH_DTYPE[dtype]
    q = torch.from_numpy(e4m3(q8) * np.float32(qd * kd)).to(t)
    k = torch.from_numpy(e4m3(k8)).to(t)
    v = torch.from_numpy(e4m3(v8) * np.float32(vd)).to(t)
    assert gate_ratio(q, k, v, dtype, causal, None) <= 1.0
