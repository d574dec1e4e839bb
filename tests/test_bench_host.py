"""Host-side logic of bench.py: byte and FLOP conventions, the counter-summary
lookup, the spread statistics, the read-stream probe's argument checks and the
one-GPU guard.  No GPU is used."""
import ctypes
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attention_forward_amd.profsum import kernel_sources_hash  # noqa: E402
from attention_forward_amd.synthetic import WORKLOADS  # noqa: E402


def test_algorithmic_bytes_and_flops():
    # Q, K, V read once and O, LSE written once: 4 * 67,108,864 + 1,048,576
    assert bench.prefill_algorithmic_bytes(bench.PREFILL) == 269_484_032
    # K and V once per kv head, plus Q, O and LSE
    assert bench.decode_algorithmic_bytes(bench.DECODE) == 2_148_540_416
    assert bench.PREFILL.flops == 549_755_813_888  # 4*B*H*S*S*d / 2 (causal)
    assert WORKLOADS["fwd_f16_b4_h16_s2048"].flops == 137_438_953_472


def _traffic_file(tmp_path, sha):
    t = {"kernel_sources_sha256": sha, "copy_mib": 1024, "fetch_scale": 2.0, "write_scale": 1.0,
         "kernels": {
             "attn::fa_fwd_kernel<attn::In16<1, 128>, false>": {
                 "read_bytes": 4.0e8, "write_bytes": 6.0e7, "dispatches": 3},
             "attn::fa_fwd_kernel<attn::In16<0, 128>, false>": {
                 "read_bytes": 1.0, "write_bytes": 1.0, "dispatches": 1},
             "attn::fa_fwd_kernel<attn::In16<1, 128>, true>": {
                 "read_bytes": 2.0, "write_bytes": 2.0, "dispatches": 1},
             "attn::fa_fwd_kernel<attn::In8<1>, false>": {
                 "read_bytes": 3.0, "write_bytes": 3.0, "dispatches": 1},
             "attn::fa_decode_split_kernel<1>": {"read_bytes": 2.0e9, "write_bytes": 1.0e7,
                                                 "dispatches": 3},
             "attn::fa_combine_kernel<1>": {"read_bytes": 1.0e7, "write_bytes": 5.0e5,
                                            "dispatches": 3}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(t))
    return str(p)


def test_traffic_lookup_takes_the_bf16_kernels(tmp_path):
    pre, dec = bench.measured_traffic(_traffic_file(tmp_path, kernel_sources_hash()))
    assert pre == {"bytes": 460_000_000, "read": 400_000_000, "write": 60_000_000}
    assert dec == {"bytes": 2_020_500_000, "read": 2_010_000_000, "write": 10_500_000}


def test_traffic_is_dropped_when_the_kernels_changed(tmp_path):
    assert bench.measured_traffic(_traffic_file(tmp_path, "0" * 64)) == (None, None)
    assert bench.measured_traffic(str(tmp_path / "missing.json")) == (None, None)


def test_spread_and_ratio():
    assert bench.spread([5, 1, 2, 3, 4, 6, 7, 8, 9, 10]) == {"median": 5, "p10": 2, "p90": 9}
    assert bench.spread([3.0]) == {"median": 3.0, "p10": 3.0, "p90": 3.0}
    assert bench.ratio(3.0, 4.0) == 0.75
    assert bench.ratio(3.0, float("nan")) is None


def test_stream_probe_rejects_bad_arguments_before_any_hip_call():
    path = os.path.join(ROOT, "attention_forward_amd", "libattn_bench.so")
    if not os.path.exists(path):
        pytest.skip("libattn_bench.so not built")
    lib = ctypes.CDLL(path)
    f = lib.stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its checks
    assert f(None, 1024, fake, 1, 64, None) == 1
    assert f(fake, 1024, None, 1, 64, None) == 1
    assert f(fake, 1000, fake, 1, 64, None) == 1          # not a multiple of 16
    assert f(ctypes.c_void_p((1 << 20) + 8), 1024, fake, 1, 64, None) == 1  # misaligned
    assert f(fake, 1024, fake, 0, 64, None) == 1
    assert f(fake, 1024, fake, 1, 96, None) == 1          # not whole waves
    assert f(fake, 1024, fake, 1, 2048, None) == 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profsum_counters_means_clock_and_mfma_busy(tmp_path):
    """The counter summary averages each counter over a kernel's dispatches and
    derives the clock (GRBM cycles per XCD over the duration) and MFMA busy."""
    from attention_forward_amd.profsum import counters

    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    rows = []
    for d, (grbm, busy) in enumerate([(8.0e6, 5.12e8), (8.8e6, 5.632e8)]):
        # 500 us at 2.0 / 2.2 GHz on 8 XCDs; busy = half of 1024 SIMDs x cycles
        for c, v in (("GRBM_GUI_ACTIVE", grbm), ("SQ_VALU_MFMA_BUSY_CYCLES", busy)):
            rows.append([d, "void attn::k<1>(int)", c, v, 1000, 501000])
            rows.append([d, "Cijk_gemm", c, 1.0, 0, 1000])
    with open(tmp_path / "p_counter_collection.csv", "w") as fh:
        fh.write(",".join(cols) + "\n")
        for r in rows:
            fh.write(",".join(str(x) for x in r) + "\n")
    text = counters(str(tmp_path), ["p"], ["<cmd>"])
    line = [x for x in text.splitlines() if "attn::k<1>" in x]
    assert len(line) == 1 and "Cijk" not in text.split("Pass")[1]
    cells = [c.strip() for c in line[0].strip("|").split("|")]
    assert cells[1] == "2" and cells[2] == "500.0"  # dispatches, mean µs
    assert cells[-2] == "2.10" and cells[-1] == "50.0%"
    # NAME@SUBSTR selects other kernels for one pass
    assert "Cijk_gemm" in counters(str(tmp_path), ["p@Cijk"], ["<cmd>"])
