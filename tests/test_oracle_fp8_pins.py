"""Pins of the FP8 part of the oracle (E4M3 format and FP8 attention) to
things other than itself:

* the E4M3 code points the OCP 8-bit format specification prints
  (tests/golden/e4m3_points.txt);
* torch's float8_e4m3fn conversions, an independent implementation of the
  same format, over all 256 codes and many values (round to nearest even);
* the already pinned 16-bit oracle: every E4M3 value is exact in binary16, so
  FP8 attention with unit descales must equal binary16 attention on the same
  values, and the descales must act as the definition says (q and k only
  through the score scale, v linearly on O);
* a brute-force FP8 reference for tiny shapes written here with numpy and
  torch's float8 and bfloat16 casts.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_points():
    pts = []
    for line in open(os.path.join(HERE, "golden", "e4m3_points.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        pts.append((int(code, 16), float(val)))
    return pts


def test_e4m3_decode_matches_the_specification_table():
    pts = golden_points()
    codes = np.array([c for c, _ in pts], dtype=np.uint8)
    got = oracle.decode_e4m3(codes)
    for (c, want), g in zip(pts, got):
        if math.isnan(want):
            assert math.isnan(g), hex(c)
        else:
            assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), hex(c)


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(11)
    # float32-representable values (so torch's float32 -> float8 path sees the
    # same number), across subnormals, normals and the top binade, plus every
    # exact code value, every midpoint between neighbours and their neighbours
    parts = [rng.uniform(-460, 460, 20000), rng.uniform(-0.02, 0.02, 20000),
             np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000)]
    vals = oracle.decode_e4m3(np.arange(256, dtype=np.uint8))
    fin = np.sort(vals[np.isfinite(vals)])
    mids = (fin[1:] + fin[:-1]) / 2
    parts += [fin, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)]
    x = np.concatenate(parts).astype(np.float32).astype(np.float64)
    x = x[np.abs(x) < 464]  # torch turns larger magnitudes into NaN; the oracle saturates
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.round_e4m3(x)
    bad = np.nonzero(got != ref)[0]
    # signed zeros may differ only in encoding of -0 vs +0 for values that round to zero
    assert bad.size == 0, [(x[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_e4m3_saturation_and_nan():
    got = oracle.round_e4m3(np.array([448.0, 464.0, 1e6, -1e6, np.inf, np.nan]))
    assert list(got[:5]) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    assert got[5] & 0x7F == 0x7F


def random_e4m3(shape, rng, spread=1.0):
    """E4M3 patterns of N(0, spread) values (what a caller quantising real data holds)."""
    return oracle.round_e4m3(rng.standard_normal(shape) * spread)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_equals_binary16_attention_on_the_same_values(causal):
    rng = np.random.default_rng(12)
    B, Hq, Hkv, Sq, Sk, d = 2, 4, 2, 37, 53, 64
    q8 = random_e4m3((B, Hq, Sq, d), rng)
    k8 = random_e4m3((B, Hkv, Sk, d), rng)
    v8 = random_e4m3((B, Hkv, Sk, d), rng)
    scale = 1.0 / math.sqrt(d)
    o8, lse8, _ = oracle.attention_fp8(q8, k8, v8, causal, scale, 1.0, 1.0, 1.0, 1, want_ref=False)
    as16 = lambda a: oracle.round_to(oracle.decode_e4m3(a), oracle.F16)  # exact
    for a in (q8, k8, v8):
        assert np.array_equal(oracle.decode(as16(a), oracle.F16), oracle.decode_e4m3(a))
    o16, lse16, _ = oracle.attention(as16(q8), as16(k8), as16(v8), oracle.F16, causal, scale,
                                     want_ref=False)
    assert np.array_equal(o8, o16)
    assert np.array_equal(lse8, lse16)


def test_fp8_descales_act_as_defined():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, Sq, Sk, d = 1, 2, 1, 20, 70, 128
    q8 = random_e4m3((B, Hq, Sq, d), rng)
    k8 = random_e4m3((B, Hkv, Sk, d), rng)
    v8 = random_e4m3((B, Hkv, Sk, d), rng)
    scale = 1.0 / math.sqrt(d)
    o1, l1, _ = oracle.attention_fp8(q8, k8, v8, True, scale * 0.75 * 2.5, 1.0, 1.0, 1.0, 1,
                                     want_ref=False)
    o2, l2, _ = oracle.attention_fp8(q8, k8, v8, True, scale, 0.75, 2.5, 1.0, 1, want_ref=False)
    o3, l3, _ = oracle.attention_fp8(q8, k8, v8, True, scale, 2.5, 0.75, 3.0, 1, want_ref=False)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-15) and np.allclose(l1, l2, rtol=1e-13)
    assert np.allclose(3.0 * o2, o3, rtol=1e-13, atol=1e-15) and np.allclose(l2, l3, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_reference_brute_force(causal):
    rng = np.random.default_rng(14)
    B, H, Sq, Sk, d = 1, 2, 9, 40, 16
    qds, kds, vds = 0.5, 1.25, 2.0
    q8 = random_e4m3((B, H, Sq, d), rng, 2.0)
    k8 = random_e4m3((B, H, Sk, d), rng, 2.0)
    v8 = random_e4m3((B, H, Sk, d), rng)
    scale = 0.3
    o, lse, o_ref = oracle.attention_fp8(q8, k8, v8, causal, scale, qds, kds, vds, 1)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    q, k, v = dec(q8) * qds, dec(k8) * kds, dec(v8) * vds
    for h in range(H):
        for i in range(Sq):
            nvis = min(Sk, i + Sk - Sq + 1) if causal else Sk
            s = scale * (k[0, h, :nvis] @ q[0, h, i])
            m = s.max()
            p = np.exp(s - m)
            pr = torch.from_numpy(p.astype(np.float32)).to(torch.float8_e4m3fn).to(
                torch.float64).numpy()
            want = (pr @ v[0, h, :nvis]) / p.sum()
            want = torch.from_numpy(want).to(torch.bfloat16).to(torch.float64).numpy()
            assert np.allclose(o_ref[0, h, i], want, rtol=2.0 ** -8, atol=1e-12)
            assert np.allclose(o[0, h, i], (p @ v[0, h, :nvis]) / p.sum(), rtol=1e-12, atol=1e-14)
            assert abs(lse[0, h, i] - (m + math.log(p.sum()))) <= 1e-12 * max(1.0, abs(lse[0, h, i]))
