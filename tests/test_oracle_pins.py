"""The oracle checked against facts that do not come from the oracle (CPU only).

* every pin in ``pins.py`` holds for the oracle, in both dtypes;
* each plausible mistake, planted in a numpy copy of the definition, fails at
  least one pin (so the pins are strong enough to catch it);
* the dtype conversions agree with numpy's and torch's round-to-nearest-even;
* the same-dtype reference rounds exactly the library softmax probabilities;
* the split-KV partials merged by ``combine`` give the unsplit result.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests import pins

F16, BF16 = 0, 1


def _to_bits(x, dtype):
    x = np.ascontiguousarray(x, dtype=np.float64)
    if dtype == F16:
        b = x.astype(np.float16).view(np.uint16)
        assert np.array_equal(b.view(np.float16).astype(np.float64), x), "not representable"
        return b
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(t.to(torch.float64), torch.from_numpy(x)), "not representable"
    return t.view(torch.int16).numpy().view(np.uint16)


def oracle_impl(qf, kf, vf, causal, scale, dtype):
    o, lse, _ = oracle.attention(_to_bits(qf, dtype), _to_bits(kf, dtype), _to_bits(vf, dtype),
                                 dtype, causal, float(np.float32(scale)), want_ref=False)
    return o, lse


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_satisfies_pin(pin, dtype):
    msg = pin(oracle_impl, dtype)
    assert msg is None, msg


# ------------------------------------------------------------ planted mistakes

def _numpy_attention(qf, kf, vf, causal, scale, mutation=None):
    """A numpy copy of the definition, with one planted mistake when `mutation` is set."""
    B, Hq, Sq, d = qf.shape
    _, Hkv, Sk, _ = kf.shape
    G = Hq // Hkv
    sc = float(np.float32(scale))
    if mutation == "no_scale":
        sc = 1.0
    if mutation == "gqa_modulo":
        heads = [h % Hkv for h in range(Hq)]
    else:
        heads = [h // G for h in range(Hq)]
    k = kf[:, heads]
    v = vf[:, heads]
    if mutation == "v_shifted":
        v = np.roll(v, 1, axis=2)
    if mutation == "q_for_k":
        s = sc * np.matmul(qf, np.swapaxes(qf[:, :, :Sk] if Sk <= Sq else k, -1, -2))
    else:
        s = sc * np.matmul(qf, np.swapaxes(k, -1, -2))
    if mutation == "neg_sign":
        s = -s
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    off = Sk - Sq
    if mutation == "causal_off_by_one":
        off += 1
    if mutation == "causal_strict":
        off -= 1
    if mutation == "causal_top_left":
        off = 0
    vis = (j <= i + off) if causal else np.ones((Sq, Sk), bool)
    if mutation == "drop_last_key":
        vis = vis & (j < Sk - 1) if Sk > 1 else vis
    s = np.where(vis, s, -np.inf)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        m = s.max(axis=-1, keepdims=True)
        m_eff = np.where(np.isneginf(m), 0.0, m)
        if mutation == "no_max_subtraction":
            m_eff = np.zeros_like(m_eff)
        p = np.exp(s - m_eff)
        if mutation == "mean_weights":
            p = np.where(vis, 1.0, 0.0) * np.ones_like(p)
        l = p.sum(axis=-1, keepdims=True)
        if mutation == "softmax_over_queries":
            p = np.exp(s - np.where(np.isneginf(s.max(axis=-2, keepdims=True)), 0,
                                    s.max(axis=-2, keepdims=True)))
            l = p.sum(axis=-2, keepdims=True)
        P = p / np.where(l == 0, 1.0, l)
        if mutation == "no_normalisation":
            P = p
        o = np.matmul(P, v)
        lse = (m_eff + np.log(l))[..., 0]
        if mutation == "lse_log2":
            lse = (m_eff / math.log(2) + np.log2(l))[..., 0]
        if mutation == "lse_no_max":
            lse = np.log(l)[..., 0]
    return o, lse


MUTATIONS = ["no_scale", "gqa_modulo", "v_shifted", "q_for_k", "neg_sign", "causal_off_by_one",
             "causal_strict", "causal_top_left", "drop_last_key", "no_max_subtraction",
             "mean_weights", "softmax_over_queries", "no_normalisation", "lse_log2",
             "lse_no_max"]


def test_numpy_copy_without_mutation_passes_pins():
    impl = lambda q, k, v, c, s, dt: _numpy_attention(q, k, v, c, s)
    for pin in pins.ALL_PINS:
        assert pin(impl, F16) is None, pin.__name__


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_planted_mistake_fails_a_pin(mutation):
    impl = lambda q, k, v, c, s, dt: _numpy_attention(q, k, v, c, s, mutation)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            msg = pin(impl, F16)
        except Exception as e:  # a crash also counts as a failed pin
            msg = repr(e)
        if msg is not None:
            failed.append(pin.__name__)
    assert failed, "mutation %s passes every pin" % mutation


# ------------------------------------------------------------ dtype conversion

def _tricky_values(rng):
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24,
            2.0 ** -25, 1.5 * 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
            1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8,
            3.3895313892515355e38, 3.4e38, 2.0 ** -126, 2.0 ** -133, 2.0 ** -134,
            1.5 * 2.0 ** -134, math.inf, -math.inf]
    vals += list(rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000))
    # exact ties of both formats
    vals += list((rng.integers(1, 2 ** 12, 2000) * 2 + 1) * 2.0 ** -12)
    vals += list((rng.integers(1, 2 ** 9, 2000) * 2 + 1) * 2.0 ** -9)
    return np.array(vals, dtype=np.float64)


def test_round_f16_matches_numpy():
    x = _tricky_values(np.random.default_rng(0))
    with np.errstate(over="ignore"):
        expect = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.round_to(x, F16), expect)


def test_round_bf16_matches_torch():
    # torch rounds float64 -> bfloat16 through float32 (two roundings), so the
    # comparison uses float32-exact inputs, where its cast is a single RNE.
    x = _tricky_values(np.random.default_rng(1))
    with np.errstate(over="ignore"):
        x = x.astype(np.float32).astype(np.float64)
    expect = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to(x, BF16), expect)


def test_round_bf16_single_rounding_of_doubles():
    # bfloat16 near 1 has spacing 2^-7.  1 + 2^-8 is a tie -> even (1.0);
    # 1 + 2^-8 + 2^-40 is just above the tie -> 1 + 2^-7 (a float32 detour
    # would drop the 2^-40 and round to 1.0); 1 + 3*2^-8 is a tie -> 1 + 2^-6.
    x = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8,
                  -(1 + 2.0 ** -8 + 2.0 ** -40)])
    got = oracle.decode(oracle.round_to(x, BF16), BF16)
    assert list(got) == [1.0, 1 + 2.0 ** -7, 1 + 2.0 ** -6, -(1 + 2.0 ** -7)]


def test_decode_matches_libraries():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.decode(allbits, F16)
    g = allbits.view(np.float16).astype(np.float64)
    same = (f == g) | (np.isnan(f) & np.isnan(g))
    assert same.all()
    b = oracle.decode(allbits, BF16)
    t = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (b == t) | (np.isnan(b) & np.isnan(t))
    assert same.all()


def test_nan_rounds_to_nan():
    out = oracle.round_to(np.array([math.nan]), F16)
    assert np.isnan(out.view(np.float16)[0])


# ------------------------------------------------------------ same-dtype reference

@pytest.mark.parametrize("dtype", [F16, BF16])
def test_dtype_reference_rounds_the_library_softmax(dtype):
    """With V = I the same-dtype reference row is round(P) (then rounded again,
    which is exact), where P is scipy's softmax of the scores."""
    rng = np.random.default_rng(21)
    B, H, Sq, Sk, d = 1, 2, 4, 6, 8
    q = pins.representable(rng.standard_normal((B, H, Sq, d)) * 1.5, dtype)
    k = pins.representable(rng.standard_normal((B, H, Sk, d)) * 1.5, dtype)
    v = np.zeros((B, H, Sk, d))
    for j in range(Sk):
        v[:, :, j, j] = 1.0
    scale = 0.5
    _, _, o_ref = oracle.attention(_to_bits(q, dtype), _to_bits(k, dtype), _to_bits(v, dtype),
                                   dtype, False, scale)
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    p = scipy.special.softmax(s, axis=-1)
    assert np.array_equal(o_ref[..., :Sk], pins.representable(p, dtype))
    assert np.all(o_ref[..., Sk:] == 0)


def test_dtype_reference_differs_from_exact_by_dtype_rounding_only():
    rng = np.random.default_rng(22)
    q, k, v = pins.rand_inputs(rng, 1, 2, 2, 16, 32, 8, F16)
    o, _, o_ref = oracle.attention(_to_bits(q, F16), _to_bits(k, F16), _to_bits(v, F16), F16,
                                   True, 0.35)
    err = np.abs(o_ref - o).max()
    assert 0 < err < 2e-2
    # the reference is itself representable in fp16
    assert np.array_equal(pins.representable(o_ref, F16), o_ref)


# ------------------------------------------------------------ split-KV partials

@pytest.mark.parametrize("dtype", [F16, BF16])
def test_split_then_combine_equals_unsplit(dtype):
    rng = np.random.default_rng(23)
    B, Hq, Hkv, Sk, d = 2, 4, 2, 37, 8
    q, k, v = pins.rand_inputs(rng, B, Hq, Hkv, 1, Sk, d, dtype, spread=1.5)
    qb, kb, vb = _to_bits(q, dtype), _to_bits(k, dtype), _to_bits(v, dtype)
    o, lse, _ = oracle.attention(qb, kb, vb, dtype, False, 0.3, want_ref=False)
    for ns in list(range(1, 17)) + [36, 37]:
        o_part, lse_part = oracle.split_partials(qb, kb, vb, dtype, 0.3, ns)
        chunk = -(-Sk // ns)
        n_nonempty = -(-Sk // chunk)
        assert np.all(np.isneginf(lse_part[..., n_nonempty:]))
        assert np.all(o_part[..., n_nonempty:, :] == 0)
        oc, lsec = oracle.combine(o_part, lse_part)
        assert np.abs(oc - o[:, :, 0]).max() <= 1e-12, ns
        assert np.abs(lsec - lse[:, :, 0]).max() <= 1e-12, ns


def test_split_partial_is_attention_over_its_chunk():
    rng = np.random.default_rng(24)
    B, Hq, Hkv, Sk, d = 1, 2, 1, 20, 4
    q, k, v = pins.rand_inputs(rng, B, Hq, Hkv, 1, Sk, d, F16)
    o_part, lse_part = oracle.split_partials(_to_bits(q, F16), _to_bits(k, F16),
                                             _to_bits(v, F16), F16, 0.5, 3)
    chunk = 7
    for s in range(3):
        sl = slice(s * chunk, min(Sk, (s + 1) * chunk))
        ob, lseb = pins.brute_force(q, k[:, :, sl], v[:, :, sl], False, 0.5)
        assert np.abs(o_part[:, :, s] - ob[:, :, 0]).max() <= 1e-12
        assert np.abs(lse_part[:, :, s] - lseb[:, :, 0]).max() <= 1e-12


def test_combine_closed_forms():
    d = 3
    a = np.array([1.0, 2.0, 3.0])
    b = np.array([-1.0, 0.0, 5.0])
    # equal LSEs: plain average, LSE + ln 2
    o, lse = oracle.combine(np.stack([a, b])[None], np.array([[0.7, 0.7]]))
    assert np.allclose(o[0], (a + b) / 2, atol=1e-15, rtol=0)
    assert abs(lse[0] - (0.7 + math.log(2))) < 1e-15
    # a -inf partial carries no weight
    o, lse = oracle.combine(np.stack([a, b])[None], np.array([[-math.inf, 1.25]]))
    assert np.array_equal(o[0], b) and lse[0] == 1.25
    # all -inf: O = 0, LSE = -inf
    o, lse = oracle.combine(np.zeros((1, 2, d)), np.array([[-math.inf, -math.inf]]))
    assert np.all(o == 0) and np.isneginf(lse[0])
    # weights are softmax of the partial LSEs
    ls = np.array([0.1, -2.0, 3.5])
    parts = np.random.default_rng(3).standard_normal((3, d))
    o, lse = oracle.combine(parts[None], ls[None])
    w = scipy.special.softmax(ls)
    assert np.allclose(o[0], w @ parts, atol=1e-14, rtol=0)
    assert abs(lse[0] - scipy.special.logsumexp(ls)) < 1e-14


def test_rows_subset_matches_full():
    rng = np.random.default_rng(25)
    q, k, v = pins.rand_inputs(rng, 2, 4, 2, 9, 11, 8, BF16)
    qb, kb, vb = _to_bits(q, BF16), _to_bits(k, BF16), _to_bits(v, BF16)
    o, lse, o_ref = oracle.attention(qb, kb, vb, BF16, True, 0.4)
    rows = np.array([0, 5, 17, 40, 71], dtype=np.int64)
    o2, lse2, o_ref2 = oracle.attention_rows(qb, kb, vb, BF16, True, 0.4, rows)
    assert np.array_equal(o2, o.reshape(-1, 8)[rows])
    assert np.array_equal(lse2, lse.reshape(-1)[rows])
    assert np.array_equal(o_ref2, o_ref.reshape(-1, 8)[rows])


def test_bad_arguments_raise():
    z = np.zeros((1, 3, 2, 4), dtype=np.uint16)
    kz = np.zeros((1, 2, 2, 4), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.attention(z, kz, kz, F16, False, 1.0)  # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.attention_rows(z[:, :2], kz, kz, F16, False, 1.0, np.array([99]))
