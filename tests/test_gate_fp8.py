"""Calibration of the FP8 correctness gate (CPU only).

A numpy model of the FP8 kernel's numerics must pass the FP8 gate against the
FP64 oracle, and each plausible defect injected into the model must fail it by
a wide margin (the same calibration as the 16-bit gate; "The FA5090
Optimization Journey", sec. 2.1, checks that an injected bug lands far outside
the bound).  The model:
- E4M3 inputs decoded exactly (through torch's float8_e4m3fn, not the oracle),
- scores in fp32 over 64-key tiles, with scale * q_descale * k_descale * log2(e)
  folded into one fp32 multiplier as the host folds it,
- the exact running max as the reference of the weights (tau = 0: the max
  moves whenever a tile's max exceeds it),
- the weights rounded to E4M3 (unnormalised) for P.V, their unrounded sum in l,
- O = acc * (v_descale / l), rounded to the output dtype.

    FP8 gate: max_abs(model - oracle) <= 2 * max_abs(ref_fp8 - oracle) + 1e-5

The same model with the 16-bit path's lazy reference (tau = 8) fails the gate
on rows dominated by a few keys: their top weight, taken against a reference
that lags the row max by a fraction of an exponent step, lands between E4M3
grid points (up to 1/16 relative error), where against the exact max it is
exactly 1.  That is why the FP8 kernel keeps the exact running max.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_forward_amd.synthetic import BF16, F16, TORCH_DTYPE, bytes_u8, make_qkv_fp8

TAU = 0.0  # the FP8 kernel's threshold (log2 units)
TAU_16BIT = 8.0  # the 16-bit kernels'
KT = 64
E4M3_MAX = 448.0


def e4m3(t):
    """uint8 E4M3 tensor -> float32 numpy values."""
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def round_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).to(
        torch.float32).numpy()


def round_out(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(TORCH_DTYPE[dtype]).to(
        torch.float32).numpy()


def kernel_model(q8, k8, v8, causal, scale, ds, out_dtype, defect=None, tau=None):
    tau = TAU if tau is None else tau
    q, k, v = e4m3(q8), e4m3(k8), e4m3(v8)
    qd, kd, vd = ds
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    folded = scale * (qd * kd if defect != "qk_descale_missing" else 1.0)
    sl2 = np.float32(folded * 1.4426950408889634)
    off = Sk - Sq + (1 if defect == "causal_off_by_one" else 0)
    out = np.zeros((B, Hq, Sq, d), np.float32)
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
                jump = mx > m + tau
                alpha = np.where(jump, np.exp2(np.where(jump, m - mx, 0)), 1).astype(np.float32)
                m = np.where(jump, mx, m)
                m_eff = np.where(np.isneginf(m), 0, m).astype(np.float32)
                p = np.where(hidden, 0, np.exp2(x - m_eff[:, None])).astype(np.float32)
                l = (l * alpha + p.sum(axis=1)).astype(np.float32)
                vt = v[b, hk, j0:j1]
                if defect == "pv_permutation":
                    vt = vt[::-1]
                if defect != "rescale_dropped":
                    acc = acc * alpha[:, None]
                acc = (acc + round_e4m3(p) @ vt).astype(np.float32)
            o_scale = vd if defect != "v_descale_missing" else 1.0
            inv = np.where(l > 0, np.float32(o_scale) / np.where(l > 0, l, 1), 0).astype(np.float32)
            out[b, h] = round_out(acc * inv[:, None], out_dtype)
    return out


def inputs(growing, seed):
    B, Hq, Hkv, Sq, Sk, d = 1, 4, 2, 200, 300, 128
    (q8, k8, v8), ds = make_qkv_fp8(B, Hq, Hkv, Sq, Sk, d, seed)
    if not growing:
        return (q8, k8, v8), ds
    # later keys' scores pass the first tile's max by far more than tau; K re-quantised per tensor
    kf = torch.from_numpy(e4m3(k8)) * ds[1] * torch.linspace(1.0, 6.0, Sk).view(1, 1, Sk, 1)
    kd = float(kf.abs().max()) / E4M3_MAX
    k8 = (kf / kd).to(torch.float8_e4m3fn).view(torch.uint8)
    return (q8, k8, v8), (ds[0], kd, ds[2])


def gate_ratio(growing, seed, causal, out_dtype, defect, tau=None):
    (q8, k8, v8), ds = inputs(growing, seed)
    scale = 1.0 / math.sqrt(q8.shape[-1])
    o, _, o_ref = oracle.attention_fp8(bytes_u8(q8), bytes_u8(k8), bytes_u8(v8), causal, scale,
                                       ds[0], ds[1], ds[2], out_dtype)
    model = kernel_model(q8, k8, v8, causal, scale, ds, out_dtype, defect, tau)
    err = np.abs(model - o).max()
    bound = 2.0 * np.abs(o_ref - o).max() + 1e-5
    return err / bound


@pytest.mark.parametrize("out_dtype", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("growing", [False, True], ids=["random", "growing"])
def test_fp8_kernel_model_passes_the_gate(growing, causal, out_dtype):
    r = gate_ratio(growing, 41, causal, out_dtype, None)
    assert r <= 1.0, r


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fp8_threshold_rescale_exceeds_the_gate_on_peaked_rows(causal):
    assert gate_ratio(False, 41, causal, BF16, None, TAU_16BIT) < 1.0
    assert gate_ratio(True, 41, causal, BF16, None, TAU_16BIT) > 1.2


DEFECTS = [
    # defect, needs growing scores, needs the causal mask
    ("v_descale_missing", False, False),
    ("qk_descale_missing", False, False),
    ("rescale_dropped", True, False),
    ("causal_off_by_one", False, True),
    ("gqa_mapping", False, False),
    ("pv_permutation", False, False),
    ("last_tile_missing", False, False),
]


@pytest.mark.parametrize("defect,growing,causal", DEFECTS, ids=[d[0] for d in DEFECTS])
def test_fp8_injected_defect_fails_the_gate_by_a_wide_margin(defect, growing, causal):
    r = gate_ratio(growing, 42, causal, BF16, defect)
    assert r > 5.0, (defect, r)


def test_score_weight_closed_forms():
    """The FP8 LSE tolerance's W on rows with closed forms: a row that sees one
    key (W = |scale qd kd| sum_i |q_i k_i|), a row whose scores are all equal
    (the plain mean over its keys), and a row that sees none (0)."""
    from tests.test_gpu_fp8 import score_weight

    e = lambda x: torch.tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    # Sq = 3 > Sk = 2, causal: row 0 sees nothing, row 1 key 0, row 2 keys 0 and 1
    q = [[[[1.0, -2.0], [0.5, 4.0], [1.0, 0.0]]]]
    k = [[[[3.0, 1.0], [-2.0, 8.0]]]]
    q8, k8 = e(q), e(k)
    scale, qd, kd = 0.5, 2.0, -0.25
    c = abs(scale * qd * kd)
    w = score_weight(q8, k8, (qd, kd, 1.0), True, scale, np.arange(3, dtype=np.int64))
    assert w[0] == 0.0
    assert w[1] == pytest.approx(c * (0.5 * 3.0 + 4.0 * 1.0))
    # row 2: q = (1, 0) scores 3c' and -2c' differ; take the softmax by hand
    s = np.array([3.0, -2.0]) * scale * qd * kd
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    assert w[2] == pytest.approx(c * (p[0] * 3.0 + p[1] * 2.0))
    # equal scores (q orthogonal to the difference of the keys): the plain mean
    k8b = e([[[[2.0, 1.0], [2.0, -1.0]]]])
    q8b = e([[[[1.0, 0.0]]]])
    wb = score_weight(q8b, k8b, (1.0, 1.0, 1.0), False, 1.0, np.arange(1, dtype=np.int64))
    assert wb[0] == pytest.approx((2.0 + 2.0) / 2)
