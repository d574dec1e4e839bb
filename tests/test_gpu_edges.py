"""Edge cases of every entry point on an MI355X, against the FP64 oracle under
the same gates as the other GPU tests:

* scale = 0 (uniform weights over the visible keys; the masked ones must stay
  exactly zero, not NaN from -inf * 0), for prefill, split prefill, decode and
  FP8;
* very large scores (|scale * q.k| up to ~2e3): every weight but the row max
  underflows, LSE is large;
* the max-free form of the threshold rule at its bound: tile maxima placed
  just below and just above the bound on the weights (2^7) and the rescale
  threshold (2^8) above the running reference, so that some tiles are accepted
  by the fast form, some redone by the full step, and some move the reference.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_forward_amd import attn_fwd, attn_fwd_decode, attn_fwd_fp8, attn_fwd_split
from attention_forward_amd.synthetic import (BF16, F16, TORCH_DTYPE, _quantise_e4m3, bits,
                                             bytes_u8, make_qkv, make_qkv_fp8)
from tests.test_gpu_parity import check_lse, gate, say

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, causal, scale, split=0):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    if split:
        attn_fwd_split(qd, kd, vd, split, causal=causal, scale=scale, out=o, lse=lse)
    else:
        attn_fwd(qd, kd, vd, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_fwd(q, k, v, dtype, causal, scale, name, split=0):
    B, Hq, Sq, d = q.shape
    o_gpu, lse_gpu = run_fwd(q, k, v, causal, scale, split)
    assert not torch.isnan(o_gpu).any() and not torch.isnan(lse_gpu).any(), name
    o, lse, o_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, causal, scale)
    n = B * Hq * Sq
    gate(o_gpu.double().numpy().reshape(n, d), o.reshape(n, d), o_ref.reshape(n, d), name=name)
    check_lse(lse_gpu.double().numpy().reshape(-1), lse.reshape(-1), name)
    return o_gpu


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("split", [0, 3], ids=["fwd", "split3"])
def test_scale_zero(split, causal, d):
    name = "scale 0 %s %s d%d" % ("split" if split else "fwd", "causal" if causal else "full", d)
    say("case", name)
    q, k, v = make_qkv(1, 2, 1, 300, 260, d, BF16, seed=501)
    o_gpu = check_fwd(q, k, v, BF16, causal, 0.0, name, split)
    if causal:  # rows 0..39 see no key at all (Sq - Sk = 40)
        assert torch.all(o_gpu[:, :, :40] == 0)


def test_scale_zero_decode_and_fp8():
    say("case scale 0 decode / fp8")
    q, k, v = make_qkv(2, 8, 2, 1, 333, 128, F16, seed=502)
    o = torch.full((2, 8, 1, 128), float("nan"), device="cuda", dtype=torch.float16)
    lse = torch.full((2, 8), float("nan"), device="cuda")
    attn_fwd_decode(q.cuda(), k.cuda(), v.cuda(), 5, scale=0.0, out=o, lse=lse)
    torch.cuda.synchronize()
    o_, lse_, o_ref = oracle.attention(bits(q), bits(k), bits(v), F16, False, 0.0)
    gate(o.cpu().double().numpy().reshape(16, 128), o_.reshape(16, 128), o_ref.reshape(16, 128),
         name="decode scale 0")
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), "decode scale 0")
    (q8, k8, v8), ds = make_qkv_fp8(1, 2, 2, 200, 150, 128, seed=503)
    o = torch.full((1, 2, 200, 128), float("nan"), device="cuda", dtype=torch.bfloat16)
    lse = torch.full((1, 2, 200), float("nan"), device="cuda")
    attn_fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), causal=True, scale=0.0, q_descale=ds[0],
                 k_descale=ds[1], v_descale=ds[2], out=o, lse=lse)
    torch.cuda.synchronize()
    o_, lse_, o_ref = oracle.attention_fp8(bytes_u8(q8), bytes_u8(k8), bytes_u8(v8), True, 0.0,
                                           ds[0], ds[1], ds[2], BF16)
    og = o.cpu()
    assert torch.all(og[:, :, :50] == 0)
    gate(og.double().numpy().reshape(400, 128), o_.reshape(400, 128), o_ref.reshape(400, 128),
         name="fp8 scale 0")
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), "fp8 scale 0")


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_large_scores(dtype, causal):
    """Q and K of magnitude ~12 (fp16 and bf16 hold them exactly enough): scores
    spread over thousands of natural-log units."""
    name = "large scores %s %s" % ("bf16" if dtype else "f16", "causal" if causal else "full")
    say("case", name)
    q, k, v = make_qkv(1, 2, 2, 260, 330, 128, dtype, seed=504)
    q = (q.float() * 12).to(TORCH_DTYPE[dtype])
    k = (k.float() * 12).to(TORCH_DTYPE[dtype])
    check_fwd(q, k, v, dtype, causal, 1.0 / math.sqrt(128), name)
    check_fwd(q, k, v, dtype, causal, 1.0 / math.sqrt(128), name + " split4", split=4)
    o = torch.full((1, 2, 1, 128), float("nan"), device="cuda", dtype=TORCH_DTYPE[dtype])
    lse = torch.full((1, 2), float("nan"), device="cuda")
    qd = q[:, :, -1:].contiguous()
    attn_fwd_decode(qd.cuda(), k.cuda(), v.cuda(), 6, out=o, lse=lse)
    torch.cuda.synchronize()
    o_, lse_, o_ref = oracle.attention(bits(qd), bits(k), bits(v), dtype, False,
                                       1.0 / math.sqrt(128))
    gate(o.cpu().double().numpy().reshape(2, 128), o_.reshape(2, 128), o_ref.reshape(2, 128),
         name=name + " decode")
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), name + " decode")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_threshold_bound(dtype, d):
    """Each query row's scores are scale * a * b_j (log2 units: the target
    offsets below) plus small noise; 64-key tile t holds one key at offset
    t_off[t] above the first tile's maximum, the rest near 0.  Offsets straddle
    7 (the fast form's bound on the weights, 2^7) and 8 (the rescale
    threshold), first rising slowly, then jumping, then falling back."""
    name = "threshold bound %s d%d" % ("bf16" if dtype else "f16", d)
    say("case", name)
    offs = [0.0, 6.9, 6.95, 7.0, 7.05, 7.2, 7.9, 7.99, 8.01, 8.3, 12.0, 15.2, 15.3, 19.0, 3.0, 0.5]
    S = 64 * len(offs)
    gen = torch.Generator().manual_seed(505)
    scale = 1.0 / math.sqrt(d)
    c = scale / math.log(2.0)  # score units -> log2 units per unit of q0 * k0
    q = torch.randn((1, 2, 96, d), generator=gen) * 0.05
    k = torch.randn((1, 2, S, d), generator=gen) * 0.05
    v = torch.randn((1, 2, S, d), generator=gen)
    q[..., 0] = 4.0
    for t, off in enumerate(offs):
        k[:, :, 64 * t + 17, 0] = off / (4.0 * c)
    q, k, v = [x.to(TORCH_DTYPE[dtype]) for x in (q, k, v)]
    check_fwd(q, k, v, dtype, False, scale, name)
    check_fwd(q, k, v, dtype, True, scale, name + " causal")


@pytest.mark.parametrize("split", [0, 4], ids=["fwd", "split4"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_peaked_rows(dtype, causal, split):
    """16-bit inputs with the FP8 calibration's peaked rows: scores spread over
    ~38 exponent steps, top keys in the last tiles, so the threshold rule's
    reference lags the row max on most rows; the 16-bit rounding of P keeps
    that inside the gate (the CPU model measures about 0.5-0.6 of it)."""
    from tests.test_gate_fp8 import e4m3, inputs

    (q8, k8, v8), (qd, kd, vd) = inputs(True, 41)
    t = TORCH_DTYPE[dtype]
    q = torch.from_numpy(e4m3(q8) * np.float32(qd * kd)).to(t)
    k = torch.from_numpy(e4m3(k8)).to(t)
    v = torch.from_numpy(e4m3(v8) * np.float32(vd)).to(t)
    name = "peaked rows dtype %d causal %s split %d" % (dtype, causal, split)
    say("case", name)
    check_fwd(q, k, v, dtype, causal, 1.0 / math.sqrt(128), name, split)
    if causal or split:
        return
    # the split-KV decode of each head's last query (6 key ranges, GQA 2)
    B, Hq, _, d = q.shape
    qd = q[:, :, -1:].contiguous()
    o = torch.full((B, Hq, 1, d), float("nan"), device="cuda", dtype=t)
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    attn_fwd_decode(qd.cuda(), k.cuda(), v.cuda(), 6, scale=1.0 / math.sqrt(128), out=o, lse=lse)
    torch.cuda.synchronize()
    o_, lse_, o_ref = oracle.attention(bits(qd), bits(k), bits(v), dtype, False, 1.0 / math.sqrt(128))
    n = B * Hq
    gate(o.cpu().double().numpy().reshape(n, d), o_.reshape(n, d), o_ref.reshape(n, d),
         name=name + " decode")
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), name + " decode")
