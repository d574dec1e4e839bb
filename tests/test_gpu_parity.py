"""Parity of the HIP path (through the C ABI) with the FP64 oracle, on an MI355X.

The gate ("The FA5090 Optimization Journey", sec. 2.1, with the FP64 oracle and
the 1e-5 constant of this build): a result passes iff

    max_abs(gpu - oracle) <= 2 * max_abs(ref_dtype - oracle) + 1e-5

over the compared rows, where ref_dtype is the oracle with P rounded to the
input dtype before P.V and O rounded to the dtype.  The absolute cap
max_abs <= 4e-3 binds on the fp16 workloads and on decode; on the bf16 causal
workloads it binds on rows >= 128 only, because the first rows see a handful of
keys, |O| reaches ~3 and a correctly rounded bf16 output alone can be 7.8e-3
away from the exact value there (the same-dtype reference errs by ~1.2e-2).
LSE: |lse_gpu - lse| <= 1e-4 + 1e-6 |lse|.

Small shapes compare every row; the full-size workloads compare sampled rows
(first rows of heads, tile boundaries, last rows, uniform random rows).
Outputs are poisoned with NaN before each call to catch unwritten elements.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_forward_amd import attn_fwd, attn_fwd_decode, attn_splitkv_combine
from attention_forward_amd.synthetic import (ALL_WORKLOADS, BF16, F16, TORCH_DTYPE, bits,
                                             make_qkv)

pytestmark = pytest.mark.gpu

CAP = 4e-3


def say(*a):
    print(*a, flush=True)


def gate(o_gpu, o, o_ref, cap_rows=None, name=""):
    """o_gpu, o, o_ref: [n, d] float64.  cap_rows: boolean mask of rows the cap binds on."""
    assert np.isfinite(o_gpu).all(), "%s: non-finite output" % name
    err = np.abs(o_gpu - o).max(axis=1)
    floor = np.abs(o_ref - o).max()
    bound = 2.0 * floor + 1e-5
    say("%s: max_abs %.3e  bound %.3e  (ref_dtype %.3e)  ratio %.3f"
        % (name, err.max(), bound, floor, err.max() / bound))
    assert err.max() <= bound, "%s: gate A fails: %.3e > %.3e" % (name, err.max(), bound)
    if cap_rows is not None and cap_rows.any():
        capped = err[cap_rows].max()
        say("%s: max_abs over capped rows %.3e (cap %.1e)" % (name, capped, CAP))
        assert capped <= CAP, "%s: cap fails %.3e" % (name, capped)
    return err.max(), bound


def check_lse(lse_gpu, lse, name=""):
    fin = np.isfinite(lse)
    assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(lse)), "%s: -inf LSE rows differ" % name
    d = np.abs(lse_gpu[fin] - lse[fin])
    tol = 1e-4 + 1e-6 * np.abs(lse[fin])
    say("%s: lse max diff %.3e" % (name, d.max() if d.size else 0.0))
    assert (d <= tol).all(), "%s: LSE off by %.3e" % (name, d.max())


def gpu_fwd(q, k, v, causal, scale, dtype):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    attn_fwd(qd, kd, vd, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def rows_of(t, rows):
    d = t.shape[-1]
    return t.reshape(-1, d)[torch.from_numpy(rows)].to(torch.float64).numpy()


SMALL = [
    # B, Hq, Hkv, Sq, Sk, dtype, causal
    (1, 1, 1, 1, 1, F16, False),
    (1, 2, 2, 64, 64, F16, False),
    (1, 2, 2, 200, 200, F16, False),
    (1, 2, 2, 333, 333, BF16, True),
    (2, 8, 2, 130, 257, BF16, False),
    (1, 4, 1, 100, 300, F16, True),
    (1, 2, 2, 300, 100, BF16, True),
    (1, 2, 2, 257, 1, F16, False),
    (1, 2, 2, 1, 700, BF16, False),
    (1, 3, 3, 129, 63, F16, True),
    (1, 32, 8, 40, 90, BF16, False),
    (2, 4, 4, 640, 640, F16, True),
    (1, 2, 1, 513, 1000, BF16, False),
]


SMALL_D64 = [
    # B, Hq, Hkv, Sq, Sk, dtype, causal -- head dimension 64
    (1, 1, 1, 1, 1, F16, False),
    (1, 2, 2, 64, 64, BF16, False),
    (1, 2, 2, 333, 333, BF16, True),
    (2, 8, 2, 130, 257, F16, False),
    (1, 4, 1, 100, 300, BF16, True),
    (1, 2, 2, 300, 100, F16, True),
    (1, 2, 2, 1, 700, BF16, False),
    (2, 4, 4, 640, 640, BF16, True),
]


# More work items (kv heads x query tiles) than a 256-CU persistent grid, so
# each workgroup takes several: grouped-query shapes whose kv heads divide
# into the 8 XCDs (the XCD-grouped item order, with several kv heads per XCD
# and batches > 1) and one whose kv heads do not (the global order).
MANY_ITEMS = [
    # B, Hq, Hkv, Sq, Sk, dtype, causal, d
    (1, 16, 8, 2200, 2200, BF16, True, 128),
    (2, 32, 8, 700, 700, F16, False, 128),
    (1, 16, 8, 2200, 2200, F16, True, 64),
    (1, 12, 4, 3000, 3000, BF16, True, 128),
]


@pytest.mark.parametrize("shape", [s + (128,) for s in SMALL] + [s + (64,) for s in SMALL_D64] +
                         MANY_ITEMS,
                         ids=lambda s: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s_d%d" % (
    s[0], s[1], s[2], s[3], s[4], "bf16" if s[5] else "f16", "causal" if s[6] else "full", s[7]))
def test_small_shapes_all_rows(shape):
    B, Hq, Hkv, Sq, Sk, dtype, causal, d = shape
    name = "small %s" % (shape,)
    say("case", name)
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype, seed=100 + Sq + Sk + d)
    scale = 1.0 / math.sqrt(d)
    o_gpu, lse_gpu = gpu_fwd(q, k, v, causal, scale, dtype)
    o, lse, o_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, causal, scale)
    n = B * Hq * Sq
    gate(o_gpu.to(torch.float64).numpy().reshape(n, d), o.reshape(n, d), o_ref.reshape(n, d),
         name=name)
    check_lse(lse_gpu.to(torch.float64).numpy().reshape(-1), lse.reshape(-1), name)
    if causal and Sq > Sk:
        hidden = o_gpu[:, :, : Sq - Sk]
        assert torch.all(hidden == 0), "fully masked rows must be exactly zero"


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_growing_scores_move_the_reference_max(dtype, causal, d):
    """Key norms grow sixfold along the sequence, so later tiles' scores pass
    the first tile's maximum by far more than the rescale threshold: the
    reference max moves mid-loop and O must be rescaled from then on."""
    B, H, S = 1, 2, 1000
    name = "growing scores %s %s d%d" % ("bf16" if dtype else "f16",
                                         "causal" if causal else "full", d)
    say("case", name)
    q, k, v = make_qkv(B, H, H, S, S, d, dtype, seed=77)
    ramp = torch.linspace(1.0, 6.0, S).view(1, 1, S, 1)  # q.k / sqrt(d) has unit variance
    k = (k.float() * ramp).to(TORCH_DTYPE[dtype])
    scale = 1.0 / math.sqrt(d)
    o_gpu, lse_gpu = gpu_fwd(q, k, v, causal, scale, dtype)
    o, lse, o_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, causal, scale)
    n = B * H * S
    gate(o_gpu.to(torch.float64).numpy().reshape(n, d), o.reshape(n, d), o_ref.reshape(n, d),
         name=name)
    check_lse(lse_gpu.to(torch.float64).numpy().reshape(-1), lse.reshape(-1), name)


def sample_rows(B, H, S, rng, n_random):
    heads = [0, B * H - 1, int(rng.integers(0, B * H))]
    rows = []
    for h in heads:
        base = h * S
        rows += [base + i for i in range(min(S, 160))]
        for edge in range(128, S, 1024):
            rows += [base + i for i in (edge - 1, edge, edge + 1) if i < S]
        rows += [base + S - 1 - i for i in range(min(S, 8))]
    rows += list(rng.integers(0, B * H * S, n_random))
    return np.unique(np.array(rows, dtype=np.int64))


@pytest.mark.parametrize("wname", [w for w in ALL_WORKLOADS if not ALL_WORKLOADS[w].decode])
def test_workload_fwd(wname):
    w = ALL_WORKLOADS[wname]
    say("case workload", wname)
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.dtype, w.seed)
    o_gpu, lse_gpu = gpu_fwd(q, k, v, w.causal, w.scale, w.dtype)
    assert not torch.isnan(o_gpu).any(), "unwritten output elements"
    assert not torch.isnan(lse_gpu).any(), "unwritten LSE elements"
    rng = np.random.default_rng(w.seed)
    if w.B * w.Hq * w.Sq <= 4096:
        rows = np.arange(w.B * w.Hq * w.Sq, dtype=np.int64)
    else:
        rows = sample_rows(w.B, w.Hq, w.Sq, rng, 1024 if w.Sq < 16384 else 512)
    o, lse, o_ref = oracle.attention_rows(bits(q), bits(k), bits(v), w.dtype, w.causal, w.scale,
                                          rows)
    cap_rows = None
    if w.dtype == F16 and not w.causal:
        cap_rows = np.ones(rows.size, bool)
    elif w.causal:
        cap_rows = (rows % w.Sq) >= 128
    gate(rows_of(o_gpu, rows), o, o_ref, cap_rows, name=wname)
    check_lse(lse_gpu.reshape(-1)[torch.from_numpy(rows)].double().numpy(), lse, wname)


@pytest.mark.parametrize("wname", [w for w in ALL_WORKLOADS if ALL_WORKLOADS[w].decode])
def test_workload_decode(wname):
    w = ALL_WORKLOADS[wname]
    say("case workload", w.name)
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, 1, w.Sk, w.d, w.dtype, w.seed)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.Hq), float("nan"), device="cuda")
    attn_fwd_decode(qd, kd, vd, w.num_splits, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_gpu, lse_gpu = o.cpu(), lse.cpu()
    del qd, kd, vd
    rows = np.arange(w.B * w.Hq, dtype=np.int64)
    o_, lse_, o_ref = oracle.attention_rows(bits(q), bits(k), bits(v), w.dtype, False, w.scale, rows)
    gate(rows_of(o_gpu, rows), o_, o_ref, np.ones(rows.size, bool), name=w.name)
    check_lse(lse_gpu.reshape(-1).double().numpy(), lse_, w.name)


DECODE_SMALL = [
    # B, Hq, Hkv, Sk, num_splits, dtype
    (1, 1, 1, 1, 1, BF16),
    (2, 4, 4, 100, 3, F16),
    (2, 8, 2, 1000, 16, BF16),
    (1, 32, 1, 513, 7, F16),
    (3, 16, 2, 64, 64, BF16),
    (1, 4, 2, 10, 8, F16),
    (2, 12, 4, 777, 5, BF16),
    (2, 8, 8, 40, 32, F16),  # splits 20..31 hold no keys
]
DECODE_SMALL_D64 = [
    (1, 1, 1, 1, 1, F16),
    (2, 8, 2, 1000, 16, BF16),
    (1, 32, 1, 513, 7, BF16),
    (3, 16, 2, 64, 64, F16),
    (2, 8, 8, 40, 32, BF16),
]


@pytest.mark.parametrize("shape", [s + (128,) for s in DECODE_SMALL] +
                         [s + (64,) for s in DECODE_SMALL_D64],
                         ids=lambda s: "B%d_Hq%d_Hkv%d_Sk%d_ns%d_d%d" % (s[:5] + s[6:]))
def test_decode_small(shape):
    B, Hq, Hkv, Sk, ns, dtype, d = shape
    say("case decode", shape)
    q, k, v = make_qkv(B, Hq, Hkv, 1, Sk, d, dtype, seed=200 + Sk + d)
    scale = 1.0 / math.sqrt(d)
    o = torch.full((B, Hq, 1, d), float("nan"), device="cuda", dtype=TORCH_DTYPE[dtype])
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    attn_fwd_decode(q.cuda(), k.cuda(), v.cuda(), ns, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_, lse_, o_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, False, scale)
    n = B * Hq
    gate(o.cpu().double().numpy().reshape(n, d), o_.reshape(n, d), o_ref.reshape(n, d),
         np.ones(n, bool), name="decode %s" % (shape,))
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), "decode")


# Larger decode shapes: 16 splits of 128 keys with a ragged last tile, and 128
# splits of 64 keys where the last holding keys has a partial tile and the one
# after it is empty.
DECODE_LARGER = [
    # B, Hq, Hkv, Sk, num_splits, dtype, d
    (32, 32, 8, 2038, 16, BF16, 128),
    (4, 32, 8, 8100, 128, F16, 128),
    (32, 32, 8, 2038, 16, F16, 64),
]


@pytest.mark.parametrize("shape", DECODE_LARGER,
                         ids=lambda s: "B%d_Hq%d_Hkv%d_Sk%d_ns%d_d%d" % (s[:5] + s[6:]))
def test_decode_many_items(shape):
    B, Hq, Hkv, Sk, ns, dtype, d = shape
    say("case decode many items", shape)
    q, k, v = make_qkv(B, Hq, Hkv, 1, Sk, d, dtype, seed=250 + ns + d)
    scale = 1.0 / math.sqrt(d)
    o = torch.full((B, Hq, 1, d), float("nan"), device="cuda", dtype=TORCH_DTYPE[dtype])
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    attn_fwd_decode(q.cuda(), k.cuda(), v.cuda(), ns, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_, lse_, o_ref = oracle.attention(bits(q), bits(k), bits(v), dtype, False, scale)
    n = B * Hq
    gate(o.cpu().double().numpy().reshape(n, d), o_.reshape(n, d), o_ref.reshape(n, d),
         np.ones(n, bool), name="decode many items %s" % (shape,))
    check_lse(lse.cpu().double().numpy().reshape(-1), lse_.reshape(-1), "decode many items")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("S", [11, 16, 37, 70])
def test_combine_matches_oracle(dtype, S, d):
    """Split counts below, at and past whole blocks of merged splits, and past 64."""
    say("case combine", dtype, S, d)
    rng = np.random.default_rng(5 + S + d)
    B, Hq = 3, 5
    o_part = rng.standard_normal((B, Hq, S, d))
    lse_part = rng.standard_normal((B, Hq, S)) * 3
    lse_part[0, 0, 3:] = -np.inf          # some empty splits
    lse_part[1, 2, :] = -np.inf           # a row with no keys at all
    lse_part[2, 1, :min(S - 1, 20)] = -np.inf  # leading empty splits, then keys
    lse_part[2, 3, -1] = 40.0             # one split dominates the rest
    o_part[lse_part == -np.inf] = 0.0
    o_part = o_part.astype(np.float32).astype(np.float64)
    lse_part = lse_part.astype(np.float32).astype(np.float64)
    o, lse = oracle.combine(o_part, lse_part)
    og, lg = attn_splitkv_combine(torch.from_numpy(o_part).float().cuda(),
                                  torch.from_numpy(lse_part).float().cuda(), TORCH_DTYPE[dtype])
    torch.cuda.synchronize()
    og = og.cpu().double().numpy()
    lg = lg.cpu().double().numpy()
    # the GPU result is o rounded to the dtype (+ fp32 arithmetic)
    half_ulp = np.abs(o) * (2.0 ** -11 if dtype == F16 else 2.0 ** -8)
    assert (np.abs(og - o) <= half_ulp + 1e-5).all()
    assert np.array_equal(np.isneginf(lg), np.isneginf(lse))
    fin = np.isfinite(lse)
    assert np.abs(lg[fin] - lse[fin]).max() <= 1e-5
    assert np.all(og[1, 2] == 0)


def test_repeat_runs_are_bitwise_identical():
    say("case determinism")
    q, k, v = make_qkv(2, 8, 8, 1024, 1024, 128, BF16, seed=7)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref, ref_lse = attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    big = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    for i in range(3):
        if i == 2:  # memory traffic on another stream while the kernel runs
            with torch.cuda.stream(side):
                for _ in range(4):
                    big.copy_(big.flip(0))
        o, lse = attn_fwd(qd, kd, vd, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(lse, ref_lse)


def test_side_stream_and_no_lse():
    say("case side stream")
    q, k, v = make_qkv(1, 4, 2, 300, 500, 128, F16, seed=8)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref, _ = attn_fwd(qd, kd, vd)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = attn_fwd(qd, kd, vd, want_lse=False)
    s.synchronize()
    torch.cuda.synchronize()
    assert lse is None
    assert torch.equal(o, ref)
