"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws iid N(0, 1) values
from a seeded torch CPU generator and rounds them to the input dtype, which is
the input recipe of the workloads below.  The pages measure on synthetic
shapes only (no dataset), so nothing stands in for a public benchmark.

Draw order is fixed: Q, then K, then V, each filled one (batch, head) slice at a
time from the same generator, so a seed reproduces the same tensors on any host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

F16, BF16 = 0, 1
TORCH_DTYPE = {F16: torch.float16, BF16: torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    dtype: int
    causal: bool
    seed: int
    num_splits: int = 0  # > 0: single-token decode with split-KV

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> int:
        """4*B*Hq*Sq*Sk*d, halved when causal (the counting convention of the metric)."""
        f = 4 * self.B * self.Hq * self.Sq * self.Sk * self.d
        return f // 2 if self.causal else f

    @property
    def decode(self) -> bool:
        return self.num_splits > 0


# The five workloads the method is measured on (d = 128, scale = 1/sqrt(128)).
WORKLOADS = {
    "fwd_f16_b1_h1_s512": Workload("fwd_f16_b1_h1_s512", 1, 1, 1, 512, 512, 128, F16, False, 1),
    "fwd_f16_b4_h16_s2048": Workload("fwd_f16_b4_h16_s2048", 4, 16, 16, 2048, 2048, 128, F16,
                                     False, 2),
    "fwd_bf16_causal_b2_h16_s8192": Workload("fwd_bf16_causal_b2_h16_s8192", 2, 16, 16, 8192,
                                             8192, 128, BF16, True, 3),
    "fwd_bf16_causal_b1_h16_s32768": Workload("fwd_bf16_causal_b1_h16_s32768", 1, 16, 16, 32768,
                                              32768, 128, BF16, True, 4),
    "decode_bf16_b64_hq32_hkv8_sk8192_split16": Workload(
        "decode_bf16_b64_hq32_hkv8_sk8192_split16", 64, 32, 8, 1, 8192, 128, BF16, False, 5,
        num_splits=16),
}

# The same shapes at head dimension 64 (the pages' other head dimension): the
# headline prefill workload and the decode workload.
HEAD_DIM_64_WORKLOADS = {
    "fwd_bf16_causal_b2_h16_s8192_d64": Workload("fwd_bf16_causal_b2_h16_s8192_d64", 2, 16, 16,
                                                 8192, 8192, 64, BF16, True, 6),
    "decode_bf16_b64_hq32_hkv8_sk8192_split16_d64": Workload(
        "decode_bf16_b64_hq32_hkv8_sk8192_split16_d64", 64, 32, 8, 1, 8192, 64, BF16, False, 7,
        num_splits=16),
}
ALL_WORKLOADS = {**WORKLOADS, **HEAD_DIM_64_WORKLOADS}


def _fill(shape, gen, dtype) -> torch.Tensor:
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype])
    flat = out.view(-1, shape[-2], shape[-1])
    for i in range(flat.shape[0]):
        flat[i].copy_(torch.randn((shape[-2], shape[-1]), generator=gen, dtype=torch.float32))
    return out


def make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype, seed):
    """Q [B,Hq,Sq,d], K and V [B,Hkv,Sk,d] on the CPU, iid N(0,1) rounded to dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    q = _fill((B, Hq, Sq, d), gen, dtype)
    k = _fill((B, Hkv, Sk, d), gen, dtype)
    v = _fill((B, Hkv, Sk, d), gen, dtype)
    return q, k, v


def make_workload_inputs(w: Workload):
    return make_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.dtype, w.seed)


def bits(t: torch.Tensor):
    """A 16-bit float tensor viewed as a numpy uint16 array of its bit patterns."""
    import numpy as np

    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# FP8: the headline prefill shape with OCP E4M3 inputs and bf16 output (the
# FP8 variant of the method; the pages measure no FP8 workload of their own).
FP8_WORKLOADS = {
    "fwd_fp8_causal_b2_h16_s8192": Workload("fwd_fp8_causal_b2_h16_s8192", 2, 16, 16, 8192, 8192,
                                            128, BF16, True, 8),
}


def _quantise_e4m3(x: torch.Tensor):
    """Per-tensor E4M3 quantisation of real inputs x: descale = amax / 448 (the
    format's largest finite value), bytes = x / descale rounded by torch's
    float8_e4m3fn cast.  Returns (uint8 tensor, descale)."""
    amax = float(x.abs().max())
    descale = amax / 448.0 if amax > 0 else 1.0
    q8 = (x / descale).to(torch.float8_e4m3fn)
    return q8.view(torch.uint8), descale


def make_qkv_fp8(B, Hq, Hkv, Sq, Sk, d, seed):
    """E4M3 inputs: Q, K, V drawn as make_qkv draws them (iid N(0,1), fp32), each
    quantised per tensor.  Returns (q8, k8, v8) as CPU uint8 tensors and the
    descales (q_descale, k_descale, v_descale); the real inputs are q8 * q_descale etc."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    out, scales = [], []
    for shape in ((B, Hq, Sq, d), (B, Hkv, Sk, d), (B, Hkv, Sk, d)):
        x = torch.empty(shape, dtype=torch.float32)
        flat = x.view(-1, shape[-2], shape[-1])
        for i in range(flat.shape[0]):
            flat[i].copy_(torch.randn((shape[-2], shape[-1]), generator=gen, dtype=torch.float32))
        t8, ds = _quantise_e4m3(x)
        out.append(t8)
        scales.append(ds)
    return tuple(out), tuple(scales)


def bytes_u8(t: torch.Tensor):
    """A 1-byte tensor viewed as a numpy uint8 array."""
    return t.contiguous().view(torch.uint8).numpy()
