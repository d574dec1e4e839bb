"""Dot-product error of the matrix instructions the prefill kernels use, measured on
the GPU against exact sums (the bound the FP8 LSE tolerance rests on).

The FP8 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4) does not round
its dot products as a chain of fp32 additions would.  The FP8 LSE tolerance
of tests/test_gpu_fp8.py adds SCORE_ERR * W, W being the softmax-weighted mean
of sum_i |scale * q_i k_i| over the row's keys, for the error of the scores
themselves: a score is a 128-term dot product, two chained instructions, and
the LSE moves by at most the weighted mean of its scores' errors.  This test
measures the worst error of such dot products relative to sum |a_i b_i| over
4096 random pairs each of two input distributions (wide exponent range, and
N(0, 100^2)), and requires it to stay below SCORE_ERR / 2, so that a toolchain
or firmware change that widened the error would be caught before the
tolerance silently became too tight.  The bfloat16 instruction
(v_mfma_f32_32x32x16_bf16), measured the same way, must stay within 2^-20 of
sum |a_i b_i| for 16 and 128 terms: close to fp32 rounding, which is why the
16-bit LSE tolerance needs no score term.

Each probe wave puts one pair (a, b) in every row of A and every column of B,
so all 1024 accumulator entries hold the same dot product; the test also
checks that they agree.
"""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

import attention_forward_amd as A
from tests.test_gpu_fp8 import SCORE_ERR

pytestmark = pytest.mark.gpu

N_PAIRS = 4096


def probe_lib():
    path = os.path.join(os.path.dirname(A.__file__), "libattn_bench.so")
    if not os.path.exists(path):
        raise ImportError("libattn_bench.so is not built (python -m attention_forward_amd.build)")
    L = ctypes.CDLL(path)
    L.mfma_dot_probe.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    L.mfma_dot_probe.restype = ctypes.c_int
    return L


def run_probe(a_dev, b_dev, n, steps, fmt):
    out = torch.full((n, 2), float("nan"), device="cuda")
    assert a_dev.numel() * a_dev.element_size() == n * steps * (64 if fmt == 0 else 32)
    assert b_dev.shape == a_dev.shape and a_dev.is_contiguous() and b_dev.is_contiguous()
    st = probe_lib().mfma_dot_probe(ctypes.c_void_p(a_dev.data_ptr()),
                                    ctypes.c_void_p(b_dev.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()), n, steps, fmt,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    assert np.array_equal(out[:, 0], out[:, 1]), "the entries of one dot product differ"
    return out[:, 0]


def fp8_inputs(kind, n, K, gen):
    x = torch.randn(2, n, K, generator=gen)
    if kind == "wide":  # magnitudes spread over 2^-8 .. 2^7
        x = x * torch.exp2(torch.randint(-8, 8, (2, n, K), generator=gen).float())
    else:
        x = x * 100.0
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn)


def relative_errors(got, a, b):
    """|got - sum a_i b_i| / sum |a_i b_i| per row, with the sums in float64
    (each product of two 8-bit or two 16-bit significands is exact there)."""
    prod = a.double() * b.double()
    exact = prod.sum(dim=1).numpy()
    scale = prod.abs().sum(dim=1).numpy()
    return np.abs(got - exact) / np.maximum(scale, 1e-300)


@pytest.mark.parametrize("kind", ["wide", "normal"])
def test_fp8_score_dot_product_error(kind):
    print("case mfma fp8 precision", kind, flush=True)
    gen = torch.Generator().manual_seed(5 if kind == "wide" else 6)
    steps = 2  # a score at head dimension 128: two chained 64-term instructions
    x = fp8_inputs(kind, N_PAIRS, 64 * steps, gen)
    a8, b8 = x[0].contiguous(), x[1].contiguous()
    got = run_probe(a8.view(torch.uint8).cuda(), b8.view(torch.uint8).cuda(), N_PAIRS, steps, 0)
    rel = relative_errors(got, a8.to(torch.float64), b8.to(torch.float64))
    worst = float(rel.max())
    print("fp8 %s: max |err| / sum|ab| = 2^%.2f (SCORE_ERR = 2^%.2f)"
          % (kind, math.log2(max(worst, 1e-300)), math.log2(SCORE_ERR)), flush=True)
    assert worst <= SCORE_ERR / 2


@pytest.mark.parametrize("steps", [1, 8])
def test_bf16_dot_product_error(steps):
    print("case mfma bf16 precision", steps, flush=True)
    gen = torch.Generator().manual_seed(7 + steps)
    K = 16 * steps
    x = torch.randn(2, N_PAIRS, K, generator=gen) * torch.exp2(
        torch.randint(-8, 8, (2, N_PAIRS, K), generator=gen).float())
    x = x.to(torch.bfloat16)
    a, b = x[0].contiguous(), x[1].contiguous()
    got = run_probe(a.view(torch.int16).cuda(), b.view(torch.int16).cuda(), N_PAIRS, steps, 1)
    rel = relative_errors(got, a.to(torch.float64), b.to(torch.float64))
    worst = float(rel.max())
    print("bf16 %d terms: max |err| / sum|ab| = 2^%.2f" % (K, math.log2(max(worst, 1e-300))),
          flush=True)
    assert worst <= 2.0 ** -20
