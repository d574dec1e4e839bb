"""The longest heads the library accepts (2^24 - 1 keys, 2^32 - 256 bytes of
K per head at d = 128), checked against closed forms.

At this length the byte offsets of a head's last tiles come within a tile of
2^32, so these tests pin the load addressing at its limit.  The inputs make
the exact result a closed form (no oracle run over 16.7 million keys):
- Q rows are (16, 0, ..., 0).  K is zero except at a few probe keys, around
  the 2^31-byte point and in the last tiles, whose rows are (32, 0, ..., 0):
  a probe's score is S = 512 * scale (about 45), every other key's 0.  So the
  probes carry all but about 1e-13 of each row's softmax mass, equally:
  O = the mean of the visible probes' V rows, LSE = S + ln(visible probes).
- V is zero except at the probes, whose rows hold (k mod 256) / 256,
  (floor(k / 256) mod 256) / 256 and floor(k / 65536) / 256 in columns 0-2
  (exact in bf16).  A probe tile read from the wrong place loses its weight,
  which moves O by a large fraction of a column's value.
- Causal rows see different probe counts (the last probes sit on the
  diagonal of the last rows).
Prefill (plain, causal, split-KV) and the split-KV decode.  Gate:
|O - exact| <= 4e-3 (the parity tests' cap) and the parity tests' LSE bound.
"""
import math

import numpy as np
import pytest
import torch

from attention_forward_amd import attn_fwd, attn_fwd_decode, attn_fwd_split
from attention_forward_amd.synthetic import BF16, TORCH_DTYPE
from tests.test_gpu_parity import CAP, check_lse, say

pytestmark = pytest.mark.gpu

SK = (1 << 24) - 1  # the library's limit
D = 128
SCALE = 1.0 / math.sqrt(D)
PROBES = [(1 << 23) - 3, (1 << 23) + 1, (1 << 23) + 71, SK - 300, SK - 70, SK - 5, SK - 1]


def digits(k):
    return np.array([k & 255, (k >> 8) & 255, k >> 16], dtype=np.float64) / 256.0


@pytest.fixture(scope="module")
def kv():
    """K and V of the probe construction on the device (8 GiB), built once and
    released after this file's tests."""
    bf = TORCH_DTYPE[BF16]
    k = torch.zeros((1, 1, SK, D), dtype=bf, device="cuda")
    v = torch.zeros((1, 1, SK, D), dtype=bf, device="cuda")
    for p in PROBES:
        k[0, 0, p, 0] = 32.0
        v[0, 0, p, :3] = torch.tensor(digits(p), dtype=torch.float32).to(bf)
    torch.cuda.synchronize()
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def q_device(h, s):
    q = torch.zeros((1, h, s, D), dtype=TORCH_DTYPE[BF16], device="cuda")
    q[..., 0] = 16.0
    return q


def check(o_gpu, lse_gpu, last_key, name):
    """Rows r seeing keys 0 .. last_key[r]."""
    n = len(last_key)
    o = np.zeros((n, D))
    lse = np.zeros(n)
    for r, last in enumerate(last_key):
        seen = [p for p in PROBES if p <= last]
        o[r, :3] = np.mean([digits(p) for p in seen], axis=0)
        lse[r] = 512.0 * SCALE + math.log(len(seen))
    og = o_gpu.reshape(n, D).double().cpu().numpy()
    assert np.isfinite(og).all(), "%s: non-finite output" % name
    err = np.abs(og - o).max()
    say("%s: max_abs %.3e (cap %.1e)" % (name, err, CAP))
    assert err <= CAP, "%s: %.3e" % (name, err)
    check_lse(lse_gpu.reshape(-1).double().cpu().numpy(), lse, name)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_prefill_longest_head(kv, causal):
    Sq = 64
    say("case prefill Sk=%d causal=%s" % (SK, causal))
    k, v = kv
    q = q_device(1, Sq)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, Sq), float("nan"), device="cuda")
    attn_fwd(q, k, v, causal=causal, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    # causal rows are aligned bottom-right: row r sees keys 0 .. r + Sk - Sq
    check(o, lse, [r + SK - Sq if causal else SK - 1 for r in range(Sq)],
          "prefill %s" % ("causal" if causal else "full"))


def test_split_prefill_longest_head(kv):
    Sq, splits = 64, 64
    say("case split prefill Sk=%d splits=%d" % (SK, splits))
    k, v = kv
    q = q_device(1, Sq)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, Sq), float("nan"), device="cuda")
    attn_fwd_split(q, k, v, num_splits=splits, causal=True, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    check(o, lse, [r + SK - Sq for r in range(Sq)], "split prefill causal")


def test_decode_longest_head(kv):
    Hq, splits = 4, 64
    say("case decode Sk=%d Hq=%d splits=%d" % (SK, Hq, splits))
    k, v = kv
    q = q_device(Hq, 1)
    o = torch.full((1, Hq, 1, D), float("nan"), device="cuda", dtype=TORCH_DTYPE[BF16])
    lse = torch.full((1, Hq), float("nan"), device="cuda")
    attn_fwd_decode(q, k, v, splits, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    check(o, lse, [SK - 1] * Hq, "decode")
