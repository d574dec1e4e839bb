"""Pins for an attention implementation, used to check the oracle against facts
that do not come from the oracle itself.

Every pin takes ``impl(qf, kf, vf, causal, scale, dtype) -> (o, lse)`` with
float64 inputs that are exactly representable in ``dtype`` and shapes
q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d]; it returns None when the fact holds and a
message when it does not.  The facts come from the mathematics of the
definition (closed forms, invariants, special cases that reduce to a library
routine) and from a brute-force evaluation of the definition in high-precision
decimal arithmetic without the max subtraction.

The definition pinned: O = softmax(scale * Q K^T [causal]) V per (batch, head),
with key j visible to query i iff j <= i + (Sk - Sq) when causal, LSE the
natural log of the softmax denominator, kv head = q head // (Hq // Hkv)
("The FA5090 Optimization Journey", sec. 2.2: the naive reference materialises
the score matrix).
"""
from __future__ import annotations

import decimal
import math

import numpy as np
import scipy.special
import torch

F16, BF16 = 0, 1


def representable(x, dtype):
    """Round float64 values to the dtype with library casts (numpy / torch RNE)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == F16:
        return x.astype(np.float16).astype(np.float64)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


def rand_inputs(rng, B, Hq, Hkv, Sq, Sk, d, dtype, spread=1.0):
    q = representable(rng.standard_normal((B, Hq, Sq, d)) * spread, dtype)
    k = representable(rng.standard_normal((B, Hkv, Sk, d)) * spread, dtype)
    v = representable(rng.standard_normal((B, Hkv, Sk, d)), dtype)
    return q, k, v


def _close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return False
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    finite = ~same_inf
    if np.any(~np.isfinite(a[finite])) or np.any(~np.isfinite(b[finite])):
        return False
    return bool(np.all(np.abs(a[finite] - b[finite]) <= tol))


# ---------------------------------------------------------------- brute force

def _dec_exp(x):
    return x.exp()


def brute_force(qf, kf, vf, causal, scale):
    """The definition in 40-digit decimal arithmetic, exp(s_j)/sum exp(s_k) with no
    max subtraction.  Tiny shapes only."""
    ctx = decimal.Context(prec=40)
    D = decimal.Decimal
    B, Hq, Sq, d = qf.shape
    _, Hkv, Sk, _ = kf.shape
    G = Hq // Hkv
    sc = D(float(np.float32(scale)))
    o = np.zeros((B, Hq, Sq, d))
    lse = np.zeros((B, Hq, Sq))
    with decimal.localcontext(ctx):
        for b in range(B):
            for h in range(Hq):
                hk = h // G
                for i in range(Sq):
                    vis = [j for j in range(Sk) if (not causal) or j <= i + (Sk - Sq)]
                    if not vis:
                        lse[b, h, i] = -math.inf
                        continue
                    e = {}
                    for j in vis:
                        s = sum(D(float(qf[b, h, i, c])) * D(float(kf[b, hk, j, c])) for c in range(d))
                        e[j] = _dec_exp(sc * s)
                    den = sum(e.values())
                    for c in range(d):
                        o[b, h, i, c] = float(sum(e[j] / den * D(float(vf[b, hk, j, c])) for j in vis))
                    lse[b, h, i] = float(den.ln())
    return o, lse


def pin_brute_force(impl, dtype):
    rng = np.random.default_rng(1234 + dtype)
    for (B, Hq, Hkv, Sq, Sk, d, causal) in [
        (1, 1, 1, 1, 1, 1, False), (1, 1, 1, 3, 5, 2, False), (1, 2, 1, 4, 4, 4, True),
        (2, 2, 2, 5, 3, 2, True), (1, 4, 2, 6, 6, 4, False), (1, 1, 1, 6, 2, 3, True),
    ]:
        q, k, v = rand_inputs(rng, B, Hq, Hkv, Sq, Sk, d, dtype, spread=1.5)
        scale = 0.7
        o, lse = impl(q, k, v, causal, scale, dtype)
        ob, lseb = brute_force(q, k, v, causal, scale)
        if not _close(o, ob, 1e-12) or not _close(lse, lseb, 1e-12):
            return "brute force mismatch at shape %s causal=%s" % ((B, Hq, Hkv, Sq, Sk, d), causal)
    return None


# ---------------------------------------------------------------- closed forms

def pin_zero_query(impl, dtype):
    """Q = 0: every visible score is 0, so O is the mean of the visible V rows and
    LSE = ln(number of visible keys)."""
    rng = np.random.default_rng(7)
    for causal in (False, True):
        B, H, Sq, Sk, d = 2, 2, 5, 5, 4
        q = np.zeros((B, H, Sq, d))
        _, k, v = rand_inputs(rng, B, H, H, Sq, Sk, d, dtype)
        o, lse = impl(q, k, v, causal, 0.5, dtype)
        for i in range(Sq):
            n = i + 1 if causal else Sk
            if not _close(o[:, :, i], v[:, :, :n].mean(axis=2), 1e-13):
                return "Q=0 mean-of-V fails (causal=%s, row %d)" % (causal, i)
            if not _close(lse[:, :, i], np.full((B, H), math.log(n)), 1e-13):
                return "Q=0 LSE != ln(n) (causal=%s, row %d)" % (causal, i)
    return None


def pin_constant_v(impl, dtype):
    rng = np.random.default_rng(8)
    q, k, _ = rand_inputs(rng, 1, 2, 2, 4, 6, 3, dtype, spread=2.0)
    v = np.empty_like(k)
    v[...] = np.array([1.5, -0.25, 3.0])
    for causal in (False, True):
        o, _ = impl(q, k, v, causal, 0.9, dtype)
        if not _close(o, np.broadcast_to(v[:, :, :1].repeat(4, axis=2), o.shape), 1e-13):
            return "constant V not returned (causal=%s)" % causal
    return None


def pin_causal_row0(impl, dtype):
    """Causal with Sq == Sk: row 0 sees only key 0, so O = V[0] exactly and
    LSE = scale * q0 . k0."""
    rng = np.random.default_rng(9)
    q, k, v = rand_inputs(rng, 2, 2, 2, 4, 4, 4, dtype)
    scale = 0.6
    o, lse = impl(q, k, v, True, scale, dtype)
    if not np.array_equal(o[:, :, 0], v[:, :, 0]):
        return "causal row 0 != V[0]"
    s00 = float(np.float32(scale)) * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0])
    if not _close(lse[:, :, 0], s00, 1e-13):
        return "causal row 0 LSE != scale q0.k0"
    return None


def pin_single_key(impl, dtype):
    rng = np.random.default_rng(10)
    q, k, v = rand_inputs(rng, 1, 3, 3, 5, 1, 4, dtype)
    o, _ = impl(q, k, v, False, 1.3, dtype)
    if not np.array_equal(o, np.broadcast_to(v, o.shape)):
        return "Sk = 1 does not return V[0]"
    return None


def pin_two_keys(impl, dtype):
    """Two keys: O = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1, LSE = logaddexp(s0, s1)."""
    rng = np.random.default_rng(11)
    q, k, v = rand_inputs(rng, 1, 2, 2, 3, 2, 4, dtype, spread=1.5)
    scale = 0.8
    o, lse = impl(q, k, v, False, scale, dtype)
    sc = float(np.float32(scale))
    s = sc * np.einsum("bhic,bhjc->bhij", q, k)
    w0 = scipy.special.expit(s[..., 0] - s[..., 1])
    w1 = scipy.special.expit(s[..., 1] - s[..., 0])
    exp_o = w0[..., None] * v[:, :, None, 0, :] + w1[..., None] * v[:, :, None, 1, :]
    if not _close(o, exp_o, 1e-13):
        return "two-key logistic form fails"
    if not _close(lse, np.logaddexp(s[..., 0], s[..., 1]), 1e-13):
        return "two-key LSE != logaddexp"
    return None


def pin_identity_v_is_softmax(impl, dtype):
    """V = identity (Sk <= d): row i of O is the probability row, which must equal
    scipy.special.softmax of the scaled scores over the visible keys (masked
    entries 0), sum to 1, and LSE must equal scipy.special.logsumexp."""
    rng = np.random.default_rng(12)
    for causal in (False, True):
        for (Hq, Hkv) in ((2, 2), (4, 2)):
            B, Sq, Sk, d = 2, 5, 7, 8
            q = representable(rng.standard_normal((B, Hq, Sq, d)) * 1.7, dtype)
            k = representable(rng.standard_normal((B, Hkv, Sk, d)) * 1.7, dtype)
            v = np.zeros((B, Hkv, Sk, d))
            for j in range(Sk):
                v[:, :, j, j] = 1.0
            scale = 0.45
            o, lse = impl(q, k, v, causal, scale, dtype)
            sc = float(np.float32(scale))
            kr = np.repeat(k, Hq // Hkv, axis=1)
            s = sc * np.matmul(q, np.swapaxes(kr, -1, -2))
            if causal:
                i = np.arange(Sq)[:, None]
                j = np.arange(Sk)[None, :]
                s = np.where(j <= i + (Sk - Sq), s, -np.inf)
            p = scipy.special.softmax(s, axis=-1)
            if not _close(o[..., :Sk], p, 1e-13) or np.any(o[..., Sk:] != 0):
                return "V = I does not give the softmax rows (causal=%s, G=%d)" % (causal, Hq // Hkv)
            if not _close(o.sum(axis=-1), np.ones((B, Hq, Sq)), 1e-13):
                return "probability rows do not sum to 1"
            if not _close(lse, scipy.special.logsumexp(s, axis=-1), 1e-13):
                return "LSE != logsumexp (causal=%s)" % causal
    return None


def pin_dominant_key(impl, dtype):
    """One key with a score far above the rest takes all the weight."""
    rng = np.random.default_rng(13)
    d = 4
    q = np.zeros((1, 1, 3, d))
    q[..., 0] = 16.0
    k = representable(rng.standard_normal((1, 1, 6, d)) * 0.1, dtype)
    k[0, 0, 4, 0] = 16.0
    _, _, v = rand_inputs(rng, 1, 1, 1, 3, 6, d, dtype)
    o, _ = impl(q, k, v, False, 1.0, dtype)
    if not _close(o, np.broadcast_to(v[:, :, 4:5], o.shape), 1e-13):
        return "dominant key does not take all the weight"
    return None


def pin_large_scores_finite(impl, dtype):
    """Scores of order 1e4 must not overflow (max subtraction) and O = V[argmax]."""
    d = 4
    q = np.full((1, 1, 2, d), 64.0)
    k = np.zeros((1, 1, 3, d))
    k[0, 0, 0] = 64.0
    k[0, 0, 1] = -64.0
    k[0, 0, 2] = 32.0
    rng = np.random.default_rng(14)
    _, _, v = rand_inputs(rng, 1, 1, 1, 2, 3, d, dtype)
    o, lse = impl(q, k, v, False, 0.5, dtype)
    if not (np.all(np.isfinite(o)) and np.all(np.isfinite(lse))):
        return "large scores produce non-finite values"
    if not _close(o, np.broadcast_to(v[:, :, 0:1], o.shape), 1e-13):
        return "large scores: O != V[argmax]"
    if not _close(lse, np.full((1, 1, 2), 0.5 * 64 * 64 * d), 1e-9):
        return "large scores: LSE != max score"
    return None


def pin_permutation_invariance(impl, dtype):
    rng = np.random.default_rng(15)
    q, k, v = rand_inputs(rng, 1, 2, 2, 4, 7, 4, dtype)
    o, lse = impl(q, k, v, False, 0.5, dtype)
    perm = rng.permutation(7)
    o2, lse2 = impl(q, k[:, :, perm], v[:, :, perm], False, 0.5, dtype)
    if not _close(o, o2, 1e-13) or not _close(lse, lse2, 1e-13):
        return "not invariant under a joint permutation of K and V rows"
    return None


def pin_key_shift(impl, dtype):
    """k_j -> k_j + c for all j leaves O unchanged and adds scale*q.c to the LSE."""
    rng = np.random.default_rng(16)
    B, H, Sq, Sk, d = 1, 2, 4, 5, 4
    q = rng.integers(-3, 4, size=(B, H, Sq, d)).astype(np.float64)
    k = rng.integers(-3, 4, size=(B, H, Sk, d)).astype(np.float64) * 0.5
    _, _, v = rand_inputs(rng, B, H, H, Sq, Sk, d, dtype)
    c = np.array([0.5, -1.0, 1.5, 0.0])
    scale = 0.25
    for causal in (False, True):
        o, lse = impl(q, k, v, causal, scale, dtype)
        o2, lse2 = impl(q, k + c, v, causal, scale, dtype)
        if not _close(o, o2, 1e-12):
            return "O changes under a common key shift (causal=%s)" % causal
        if not _close(lse2 - lse, scale * np.einsum("bhic,c->bhi", q, c), 1e-12):
            return "LSE shift != scale q.c (causal=%s)" % causal
    return None


def pin_gqa_repeat(impl, dtype):
    """Grouped query heads equal plain multi-head attention with each K/V head
    repeated for its group of consecutive query heads."""
    rng = np.random.default_rng(17)
    for causal in (False, True):
        q, k, v = rand_inputs(rng, 2, 6, 2, 4, 5, 4, dtype)
        o, lse = impl(q, k, v, causal, 0.5, dtype)
        o2, lse2 = impl(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), causal, 0.5, dtype)
        if not _close(o, o2, 0.0) or not _close(lse, lse2, 0.0):
            return "GQA != MHA with repeated K/V heads (causal=%s)" % causal
    return None


def pin_scale_zero(impl, dtype):
    rng = np.random.default_rng(18)
    q, k, v = rand_inputs(rng, 1, 2, 2, 3, 4, 4, dtype)
    o, lse = impl(q, k, v, False, 0.0, dtype)
    o2, lse2 = impl(np.zeros_like(q), k, v, False, 0.7, dtype)
    if not _close(o, o2, 1e-15) or not _close(lse, lse2, 1e-15):
        return "scale = 0 differs from Q = 0"
    return None


def pin_fully_masked_rows(impl, dtype):
    """Causal with Sq > Sk: rows i < Sq - Sk see no key: O = 0, LSE = -inf; the
    next row sees exactly key 0."""
    rng = np.random.default_rng(19)
    q, k, v = rand_inputs(rng, 1, 2, 2, 6, 3, 4, dtype)
    o, lse = impl(q, k, v, True, 0.5, dtype)
    if not (np.all(o[:, :, :3] == 0) and np.all(np.isneginf(lse[:, :, :3]))):
        return "fully masked rows are not O = 0, LSE = -inf"
    if not np.array_equal(o[:, :, 3], v[:, :, 0]):
        return "first visible row != V[0]"
    return None


ALL_PINS = [
    pin_brute_force, pin_zero_query, pin_constant_v, pin_causal_row0, pin_single_key,
    pin_two_keys, pin_identity_v_is_softmax, pin_dominant_key, pin_large_scores_finite,
    pin_permutation_invariance, pin_key_shift, pin_gqa_repeat, pin_scale_zero,
    pin_fully_masked_rows,
]
