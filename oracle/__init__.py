"""FP64 CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything in here, and the
two share no code.

The arithmetic lives in ``oracle.c`` (plain C, FP64, OpenMP over query rows);
this module only builds and loads it and marshals numpy arrays.  What it
computes, with the passages it follows, is stated in ``oracle.h``:

* ``attention``: O = softmax(scale * Q K^T [causal]) V and the natural-log LSE,
  with the score row materialised and a max-subtracted softmax ("The FA5090
  Optimization Journey", sec. 2.1 and 2.2; "10 rounds of hand-written fused
  attention ...", "The correctness trap").
* the same-dtype reference: the normalised P rounded to the input dtype before
  the P.V product and O rounded to the input dtype (the second reference of the
  correctness gate, "The FA5090 Optimization Journey", sec. 2.1).
* ``split_partials`` / ``combine``: the split-KV decode partials and their
  log-sum-exp merge.
* ``decode_e4m3`` / ``round_e4m3`` / ``attention_fp8``: the OCP E4M3 format
  and attention over per-tensor-scaled E4M3 inputs, with its FP8 reference
  (unnormalised weights rounded to E4M3 before the product with V).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    c_u16p = ctypes.POINTER(ctypes.c_uint16)
    c_dp = ctypes.POINTER(ctypes.c_double)
    c_i64p = ctypes.POINTER(ctypes.c_int64)
    i, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_decode.argtypes = [c_u16p, i64, i, c_dp]
    lib.oracle_round.argtypes = [c_dp, i64, i, c_u16p]
    lib.oracle_attention_rows.argtypes = [c_u16p, c_u16p, c_u16p, i, i, i, i, i, i, i, i, dbl,
                                          c_i64p, i64, c_dp, c_dp, c_dp, i]
    lib.oracle_split_partials.argtypes = [c_u16p, c_u16p, c_u16p, i, i, i, i, i, i, dbl, i,
                                          c_dp, c_dp]
    lib.oracle_combine.argtypes = [c_dp, c_dp, i64, i, i, c_dp, c_dp]
    c_u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_decode_e4m3.argtypes = [c_u8p, i64, c_dp]
    lib.oracle_round_e4m3.argtypes = [c_dp, i64, c_u8p]
    lib.oracle_attention_fp8_rows.argtypes = [c_u8p, c_u8p, c_u8p, i, i, i, i, i, i, i, dbl, dbl,
                                              dbl, dbl, i, c_i64p, i64, c_dp, c_dp, c_dp, i]
    for fn in (lib.oracle_decode, lib.oracle_round, lib.oracle_attention_rows,
               lib.oracle_split_partials, lib.oracle_combine, lib.oracle_decode_e4m3,
               lib.oracle_round_e4m3, lib.oracle_attention_fp8_rows):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are 16-bit patterns (numpy uint16), got %s" % a.dtype)
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def decode(bits, dtype: int) -> np.ndarray:
    """16-bit patterns -> float64 values (exact)."""
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _check(_load().oracle_decode(_ptr(bits, ctypes.c_uint16), bits.size, dtype,
                                 _ptr(out, ctypes.c_double)), "decode")
    return out


def round_to(values, dtype: int) -> np.ndarray:
    """float64 values -> 16-bit patterns, round to nearest even."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=np.uint16)
    _check(_load().oracle_round(_ptr(values, ctypes.c_double), values.size, dtype,
                                _ptr(out, ctypes.c_uint16)), "round")
    return out


def attention_rows(q, k, v, dtype: int, causal: bool, scale: float, rows, want_ref: bool = True,
                   nthreads: int = 0):
    """Oracle rows.  q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] as uint16 bit patterns.

    rows: flattened indices (b*Hq + hq)*Sq + i.  Returns (o [n,d], lse [n],
    o_ref [n,d] or None), all float64.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    o_ref = np.empty((n, d), dtype=np.float64) if want_ref else None
    rc = _load().oracle_attention_rows(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16), dtype,
        B, Hq, Hkv, Sq, Sk, d, 1 if causal else 0, float(scale), _ptr(rows, ctypes.c_int64), n,
        _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
        _ptr(o_ref, ctypes.c_double) if want_ref else None, nthreads)
    _check(rc, "attention_rows")
    return o, lse, o_ref


def attention(q, k, v, dtype: int, causal: bool, scale: float, want_ref: bool = True,
              nthreads: int = 0):
    """All rows: returns (o [B,Hq,Sq,d], lse [B,Hq,Sq], o_ref or None)."""
    B, Hq, Sq, d = q.shape
    rows = np.arange(B * Hq * Sq, dtype=np.int64)
    o, lse, o_ref = attention_rows(q, k, v, dtype, causal, scale, rows, want_ref, nthreads)
    shp = (B, Hq, Sq, d)
    return o.reshape(shp), lse.reshape(B, Hq, Sq), (o_ref.reshape(shp) if want_ref else None)


def split_partials(q, k, v, dtype: int, scale: float, num_splits: int):
    """Decode partials: q [B,Hq,1,d] -> (o_part [B,Hq,ns,d], lse_part [B,Hq,ns])."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Sq, d = q.shape
    if Sq != 1:
        raise ValueError("split partials are defined for a single query row")
    _, Hkv, Sk, _ = k.shape
    o_part = np.empty((B, Hq, num_splits, d), dtype=np.float64)
    lse_part = np.empty((B, Hq, num_splits), dtype=np.float64)
    rc = _load().oracle_split_partials(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16), dtype,
        B, Hq, Hkv, Sk, d, float(scale), num_splits, _ptr(o_part, ctypes.c_double),
        _ptr(lse_part, ctypes.c_double))
    _check(rc, "split_partials")
    return o_part, lse_part


def combine(o_part, lse_part):
    """Merge partials [R..., ns, d] / [R..., ns] -> (o [R..., d], lse [R...])."""
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    ns, d = o_part.shape[-2], o_part.shape[-1]
    lead = o_part.shape[:-2]
    if lse_part.shape != lead + (ns,):
        raise ValueError("lse_part shape mismatch")
    R = int(np.prod(lead)) if lead else 1
    o = np.empty(lead + (d,), dtype=np.float64)
    lse = np.empty(lead, dtype=np.float64)
    rc = _load().oracle_combine(_ptr(o_part, ctypes.c_double), _ptr(lse_part, ctypes.c_double),
                                R, d, ns, _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    _check(rc, "combine")
    return o, lse


def _u8(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("FP8 inputs are 8-bit patterns (numpy uint8), got %s" % a.dtype)
    return a


def decode_e4m3(bits) -> np.ndarray:
    """E4M3 (OCP, no infinities) patterns -> float64 values (exact)."""
    bits = _u8(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _check(_load().oracle_decode_e4m3(_ptr(bits, ctypes.c_uint8), bits.size,
                                      _ptr(out, ctypes.c_double)), "decode_e4m3")
    return out


def round_e4m3(values) -> np.ndarray:
    """float64 -> E4M3 patterns, nearest-even, saturating at 448."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=np.uint8)
    _check(_load().oracle_round_e4m3(_ptr(values, ctypes.c_double), values.size,
                                     _ptr(out, ctypes.c_uint8)), "round_e4m3")
    return out


def attention_fp8_rows(q, k, v, causal: bool, scale: float, q_descale: float, k_descale: float,
                       v_descale: float, out_dtype: int, rows, want_ref: bool = True,
                       nthreads: int = 0):
    """FP8 oracle rows.  q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] as uint8 E4M3 patterns; the
    real inputs are the decoded values times the per-tensor descales.  Returns
    (o [n,d], lse [n], o_ref [n,d] or None), float64; o_ref is the FP8
    reference (unnormalised weights rounded to E4M3, O rounded to out_dtype)."""
    q, k, v = _u8(q), _u8(k), _u8(v)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    o_ref = np.empty((n, d), dtype=np.float64) if want_ref else None
    rc = _load().oracle_attention_fp8_rows(
        _ptr(q, ctypes.c_uint8), _ptr(k, ctypes.c_uint8), _ptr(v, ctypes.c_uint8), B, Hq, Hkv, Sq,
        Sk, d, 1 if causal else 0, float(scale), float(q_descale), float(k_descale),
        float(v_descale), out_dtype, _ptr(rows, ctypes.c_int64), n, _ptr(o, ctypes.c_double),
        _ptr(lse, ctypes.c_double), _ptr(o_ref, ctypes.c_double) if want_ref else None, nthreads)
    _check(rc, "attention_fp8_rows")
    return o, lse, o_ref


def attention_fp8(q, k, v, causal: bool, scale: float, q_descale: float, k_descale: float,
                  v_descale: float, out_dtype: int, want_ref: bool = True, nthreads: int = 0):
    """All rows of the FP8 oracle: (o [B,Hq,Sq,d], lse [B,Hq,Sq], o_ref or None)."""
    B, Hq, Sq, d = q.shape
    rows = np.arange(B * Hq * Sq, dtype=np.int64)
    o, lse, o_ref = attention_fp8_rows(q, k, v, causal, scale, q_descale, k_descale, v_descale,
                                       out_dtype, rows, want_ref, nthreads)
    shp = (B, Hq, Sq, d)
    return o.reshape(shp), lse.reshape(B, Hq, Sq), (o_ref.reshape(shp) if want_ref else None)
