"""Benchmark of the gfx950 attention forward path on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:

  * prefill forward, bf16, causal, B=2, H=16, S=8192, d=128 (the headline
    workload; FLOPs counted as 4*B*H*Sq*Sk*d, halved for causal), and
  * split-KV decode, bf16, B=64, Hq=32, Hkv=8, Sk=8192, 16 splits, plus its
    LSE combine (reported in HBM GB/s of algorithmic bytes).

Inputs are seeded N(0,1) values already resident in HBM when the timed region
starts.  Kernel durations come from HIP events recorded on the stream the
library launches on (torch's current stream).  `value` is the prefill
throughput in TFLOP/s; the decode rate, GEMM ceilings (square and
attention-shaped batched) and an HBM read-stream ceiling measured on the same
GPU, the other prefill workloads, the roofline of the dominant kernel and the
FP64 CPU oracle timed on a bounded sample of the prefill workload are reported
beside it.  The oracle's
sample also checks the GPU output on those rows; a failing check prints no
throughput.

    python bench.py [--gpus 1] [--steps 100] [--warmup 30] [--warmup-seconds 2]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

import attention_forward_amd as A
from attention_forward_amd.synthetic import (ALL_WORKLOADS, BF16, FP8_WORKLOADS, TORCH_DTYPE,
                                             WORKLOADS, bits, make_qkv_fp8, make_workload_inputs)

PREFILL = WORKLOADS["fwd_bf16_causal_b2_h16_s8192"]
DECODE = WORKLOADS["decode_bf16_b64_hq32_hkv8_sk8192_split16"]
METRIC = "attention fwd TFLOP/s and % of MFMA ceiling (S=8k d=128); decode HBM GB/s"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published


def prefill_algorithmic_bytes(w) -> int:
    """Q, K, V read once, O and LSE written once."""
    e = 2
    return (w.B * w.Hq * w.Sq * w.d * e + 2 * w.B * w.Hkv * w.Sk * w.d * e +
            w.B * w.Hq * w.Sq * w.d * e + w.B * w.Hq * w.Sq * 4)


def decode_algorithmic_bytes(w) -> int:
    """K and V read once per kv head, Q read, O (dtype) and LSE (fp32) written."""
    e = 2
    kv = 2 * w.B * w.Hkv * w.Sk * w.d * e
    q = w.B * w.Hq * w.d * e
    o = w.B * w.Hq * w.d * e
    lse = w.B * w.Hq * 4
    return kv + q + o + lse


def measured_traffic(path=None):
    """HBM bytes per launch of the prefill and decode kernels from the committed
    rocprofv3 counter summary (profiles/traffic.json), or None for a kernel
    whose sources changed since the counters were taken."""
    from attention_forward_amd.profsum import kernel_sources_hash

    if path is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "traffic.json")
    if not os.path.exists(path):
        return None, None
    t = json.load(open(path))
    if t.get("kernel_sources_sha256") != kernel_sources_hash():
        return None, None
    k = t["kernels"]

    def find(prefix):  # the bf16 instantiation of a kernel template
        hits = [v for name, v in k.items() if name.startswith(prefix)]
        return hits[0] if len(hits) == 1 else None

    fwd = find("attn::fa_fwd_kernel<attn::In16<1, 128>, false>")
    split = find("attn::fa_decode_split_kernel<1")
    comb = find("attn::fa_combine_kernel<1")
    pre = None if fwd is None else {"bytes": round(fwd["read_bytes"] + fwd["write_bytes"]),
                                    "read": round(fwd["read_bytes"]),
                                    "write": round(fwd["write_bytes"])}
    dec = None
    if split is not None and comb is not None:
        rd = split["read_bytes"] + comb["read_bytes"]
        wr = split["write_bytes"] + comb["write_bytes"]
        dec = {"bytes": round(rd + wr), "read": round(rd), "write": round(wr)}
    return pre, dec


def _time_ms(fn, iters, warmup=3):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def _time_ms_median(fn, iters, warm_s=0.75, rounds=5):
    """Median over `rounds` of _time_ms, after at least warm_s seconds of the same
    launches: the engine clock rises under sustained load and settles within
    about a second, so each figure is taken in the loaded state, as the
    headline steps are."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    ts = sorted(_time_ms(fn, iters, 1) for r in range(rounds))
    return ts[len(ts) // 2]


def bmm_ceiling(dtype=torch.bfloat16, bh=32, n=8192, d=128, iters=10):
    """The attention-shaped product S = Q K^T of the headline workload as one
    batched GEMM ([32, 8192, 128] x [32, 128, 8192], both operands contiguous)."""
    a = torch.randn(bh, n, d, device="cuda", dtype=dtype)
    b = torch.randn(bh, d, n, device="cuda", dtype=dtype)
    c = torch.empty(bh, n, n, device="cuda", dtype=dtype)
    ms = _time_ms(lambda: torch.bmm(a, b, out=c), iters)
    del a, b, c
    return 2.0 * bh * n * n * d / (ms * 1e-3) / 1e12


def hbm_read_ceiling(gib=4, iters=10):
    """Best read rate of a plain streaming kernel (libattn_bench.so) over a few
    launch shapes; returns (GB/s, shape)."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(os.path.dirname(A.__file__), "libattn_bench.so"))
    lib.stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p]
    lib.stream_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = (0.0, None)
    for threads, blocks in ((512, 8192), (512, 16384), (512, 32768), (256, 16384)):
        def run():
            if lib.stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                               ctypes.c_void_p(sink.data_ptr()), blocks, threads, stream) != 0:
                raise RuntimeError("stream_read launch failed")
        gbs = nbytes / (_time_ms(run, iters) * 1e-3) / 1e9
        if gbs > best[0]:
            best = (gbs, "%d x %d threads" % (blocks, threads))
    del buf, sink
    return best


def decode_read_ceiling(iters=10):
    """Read rate of the decode's memory side without its math
    (csrc_bench/decode_read.hip) at the decode workload's geometry: one
    single-wave workgroup per (batch, kv head, split), its K and V tiles through
    direct-to-LDS loads one tile ahead.  Returns GB/s of K and V bytes with the
    two arrays the decode reads, and with one contiguous array."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(os.path.dirname(A.__file__), "libattn_bench.so"))
    lib.decode_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.decode_read.restype = ctypes.c_int
    wgs = DECODE.B * DECODE.Hkv * DECODE.num_splits
    tiles = DECODE.Sk // DECODE.num_splits // 64
    tile_bytes = 64 * DECODE.d * 2
    assert DECODE.d == 128 and tiles * DECODE.num_splits * 64 == DECODE.Sk
    half = wgs * tiles * tile_bytes
    buf = torch.zeros(2 * half, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for one, name in ((0, "two_arrays"), (1, "one_array")):
        def run():
            if lib.decode_read(ctypes.c_void_p(buf.data_ptr()),
                               ctypes.c_void_p(buf.data_ptr() + half), wgs, tiles, one,
                               ctypes.c_void_p(sink.data_ptr()), stream) != 0:
                raise RuntimeError("decode_read launch failed")
        out[name] = round(2 * half / (_time_ms(run, iters) * 1e-3) / 1e9, 1)
    del buf, sink
    return out


def other_workloads(iters=20):
    """Throughput of the other workloads (context; their parity is checked by the
    GPU tests): the other prefill shapes in TFLOP/s, and the headline prefill
    and decode shapes at head dimension 64 (TFLOP/s, GB/s)."""
    out = {}
    for name, w in ALL_WORKLOADS.items():
        if w is PREFILL or w is DECODE:
            continue
        q, k, v = [t.cuda() for t in make_workload_inputs(w)]
        o = torch.empty_like(q)
        if w.decode:
            lse = torch.empty((w.B, w.Hq), device="cuda", dtype=torch.float32)
            ws = torch.empty(A.attn_decode_workspace_bytes(w.B, w.Hq, w.d, w.num_splits),
                             device="cuda", dtype=torch.uint8)
            ms = _time_ms_median(lambda: A.attn_fwd_decode(q, k, v, w.num_splits, scale=w.scale, out=o,
                                                    lse=lse, workspace=ws), iters)
            out[name] = {"ms": round(ms, 4),
                         "gbs": round(decode_algorithmic_bytes(w) / (ms * 1e-3) / 1e9, 1)}
            del ws
        else:
            lse = torch.empty(q.shape[:3], device="cuda", dtype=torch.float32)
            ms = _time_ms_median(lambda: A.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o,
                                             lse=lse), iters)
            out[name] = {"ms": round(ms, 4), "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2)}
            # under-filled grids: the split-KV form with the recommended split count
            ns = A.attn_fwd_num_splits(w.B, w.Hq, w.Sq, w.Sk, w.d)
            if ns > 1:
                ws = torch.empty(A.attn_fwd_split_workspace_bytes(w.B, w.Hq, w.Sq, w.d, ns),
                                 device="cuda", dtype=torch.uint8)
                ms = _time_ms_median(lambda: A.attn_fwd_split(q, k, v, ns, causal=w.causal,
                                                       scale=w.scale, out=o, lse=lse,
                                                       workspace=ws), iters)
                out[name]["split"] = {"num_splits": ns, "ms": round(ms, 4),
                                      "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2)}
                del ws
        del q, k, v, o, lse
    for name, w in FP8_WORKLOADS.items():
        (q, k, v), ds = make_qkv_fp8(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.seed)
        q, k, v = q.cuda(), k.cuda(), v.cuda()
        o = torch.empty((w.B, w.Hq, w.Sq, w.d), device="cuda", dtype=TORCH_DTYPE[w.dtype])
        lse = torch.empty((w.B, w.Hq, w.Sq), device="cuda", dtype=torch.float32)
        ms = _time_ms_median(lambda: A.attn_fwd_fp8(q, k, v, causal=w.causal, scale=w.scale,
                                             q_descale=ds[0], k_descale=ds[1], v_descale=ds[2],
                                             out=o, lse=lse), iters)
        tf = w.flops / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                     "frac_fp8_mfma_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
        del q, k, v, o, lse
    return out


def ratio(a, b):
    """a / b rounded, or None when the ceiling b was not measured."""
    return None if b is None or not math.isfinite(b) else round(a / b, 4)


def gpu_state():
    """Clocks, power and temperature of GPU 0 as rocm-smi reports them (None
    where the tool is missing or fails); taken before and after the timed steps."""
    import shutil
    import subprocess

    # rocm-smi is a Python script behind an env shebang; starting it with this
    # interpreter avoids the env process, which would replace itself by exec
    # after a preloaded profiler library had already opened the GPU in it.
    tool = shutil.which("rocm-smi")
    if tool is None:
        return None
    try:
        r = subprocess.run([sys.executable, os.path.realpath(tool), "--showclocks",
                            "--showpower", "--showtemp", "--json"],
                           capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
    except Exception:  # no tool, no permission, or not JSON: report nothing
        return None
    card = data.get("card0") if isinstance(data, dict) else None
    if not isinstance(card, dict):
        return None
    keep = ("sclk", "mclk", "fclk", "socclk", "power", "temperature", "junction", "edge",
            "memory")
    return {k: v for k, v in card.items() if any(w in k.lower() for w in keep)}


def spread(xs):
    """median, p10 and p90 of a list of durations (ms)."""
    t = sorted(xs)

    def pct(p):
        return t[min(len(t) - 1, int(round(p * (len(t) - 1))))]

    return {"median": round(pct(0.5), 4), "p10": round(pct(0.1), 4), "p90": round(pct(0.9), 4)}


def warm_up(step, min_steps, min_seconds, settle=True, batch=20, tol=0.01, max_seconds=10.0):
    """Untimed steps: at least `min_steps` and `min_seconds` of wall time; then,
    with `settle`, batches of `batch` steps until two consecutive batches agree
    within `tol` (or `max_seconds` have passed).  Returns what was run."""
    t0 = time.perf_counter()
    n = 0
    while n < min_steps or time.perf_counter() - t0 < min_seconds:
        step()
        n += 1
        if n % batch == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    batches = []
    while settle and time.perf_counter() - t0 < max_seconds:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(batch):
            step()
        e.record()
        e.synchronize()
        n += batch
        batches.append(s.elapsed_time(e) / batch)
        if len(batches) >= 2 and abs(batches[-1] - batches[-2]) <= tol * batches[-2]:
            break
    return {"steps": n, "seconds": round(time.perf_counter() - t0, 2),
            "last_batches_ms": [round(x, 4) for x in batches[-2:]]}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gemm_ceiling(dtype, n=8192, iters=50, warm_s=0.5):
    """hipBLASLt (torch.matmul) on an n^3 product, timed after at least warm_s
    seconds of the same product so that the clock is in its loaded state, as it
    is for the attention steps."""
    a = torch.randn(n, n, device="cuda", dtype=dtype)
    b = torch.randn(n, n, device="cuda", dtype=dtype)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(5):
            torch.matmul(a, b)
        torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        torch.matmul(a, b)
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / iters
    del a, b
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def cpu_baseline(q, k, v, o_gpu, target_s: float):
    """The oracle as it stands, timed on the host cores over a uniform random
    sample of the prefill rows; also checks the GPU rows of that sample."""
    import oracle

    w = PREFILL
    nthreads = len(os.sched_getaffinity(0))
    qb, kb, vb = bits(q), bits(k), bits(v)
    n_rows = w.B * w.Hq * w.Sq
    flops_per_row = w.flops / n_rows  # the metric's counting convention, per row
    rng = np.random.default_rng(0)
    # grow the sample until one timed run takes at least half of target_s
    n = 2048
    while True:
        rows = np.sort(rng.choice(n_rows, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        o, lse, o_ref = oracle.attention_rows(qb, kb, vb, w.dtype, w.causal, w.scale, rows,
                                              want_ref=True, nthreads=nthreads)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= n_rows:
            break
        n = int(min(n_rows, n * min(8.0, max(1.5, target_s / max(dt, 1e-3)))))
    og = o_gpu.reshape(-1, w.d)[torch.from_numpy(rows)].double().numpy()
    err = float(np.abs(og - o).max())
    bound = float(2 * np.abs(o_ref - o).max() + 1e-5)
    base = {
        "value": round(flops_per_row * n / dt / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads,
        "cpu": cpu_model(), "kind": "oracle",
        "sample": "%d uniform random query rows of %s (FP64, %.1f s wall, %d threads)"
                  % (n, w.name, dt, nthreads),
    }
    parity = {"rows": n, "max_abs": err, "bound": bound, "pass": err <= bound}
    return base, parity


def decode_parity(q, k, v, o_gpu, n_rows=64):
    import oracle

    w = DECODE
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(w.B * w.Hq, n_rows, replace=False)).astype(np.int64)
    o, _, o_ref = oracle.attention_rows(bits(q), bits(k), bits(v), w.dtype, False, w.scale, rows)
    og = o_gpu.reshape(-1, w.d)[torch.from_numpy(rows)].double().numpy()
    err = float(np.abs(og - o).max())
    bound = float(2 * np.abs(o_ref - o).max() + 1e-5)
    return {"rows": n_rows, "max_abs": err, "bound": bound, "pass": err <= bound}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first (at least; see --warmup-seconds)")
    ap.add_argument("--warmup-seconds", type=float, default=2.0,
                    help="warm up for at least this long, and then until two consecutive "
                         "batches of steps agree: the clock under sustained matrix load "
                         "takes a second or more to settle, whatever the step count")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle's CPU-baseline sample")
    ap.add_argument("--skip-cpu-baseline", action="store_true",
                    help="for profiler runs: no oracle leg (and no parity rows)")
    ap.add_argument("--skip-context", "--skip-gemm", dest="skip_context", action="store_true",
                    help="for profiler runs: measure no ceilings (GEMM, batched GEMM, HBM read "
                         "stream) and no other workloads, so only the step's kernels run")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(a known-size kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    A.lib()  # fail loudly if libattn.so is not built
    dev = torch.device("cuda", 0)

    # inputs resident in HBM before the timed region
    q, k, v = make_workload_inputs(PREFILL)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], device=dev, dtype=torch.float32)
    dq, dk, dv = make_workload_inputs(DECODE)
    dqd, dkd, dvd = dq.to(dev), dk.to(dev), dv.to(dev)
    do = torch.empty_like(dqd)
    dlse = torch.empty((DECODE.B, DECODE.Hq), device=dev, dtype=torch.float32)
    ws = torch.empty(A.attn_decode_workspace_bytes(DECODE.B, DECODE.Hq, DECODE.d,
                                                   DECODE.num_splits), device=dev,
                     dtype=torch.uint8)

    def step(ev=None):
        if ev:
            ev[0].record()
        A.attn_fwd(qd, kd, vd, causal=True, scale=PREFILL.scale, out=o, lse=lse)
        if ev:
            ev[1].record()
        A.attn_fwd_decode(dqd, dkd, dvd, DECODE.num_splits, scale=DECODE.scale, out=do, lse=dlse,
                          workspace=ws)
        if ev:
            ev[2].record()

    warm = warm_up(step, args.warmup, args.warmup_seconds)
    state_before = None if args.skip_context else gpu_state()
    # the state query leaves the GPU idle for a moment: bring the clock back
    # under load before the timed steps
    warm_up(step, 0, 0.3, settle=False)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state_after = None if args.skip_context else gpu_state()
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    tflops = PREFILL.flops / (pre_avg * 1e-3) / 1e12
    dec_bytes = decode_algorithmic_bytes(DECODE)
    dec_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9

    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.skip_context:
        gemm = {}
        gemm_best = float("nan")
        stream_gbs, stream_shape = float("nan"), None
        dec_read = {}
        others = {}
    else:
        gemm = {"bf16_8192^3": round(gemm_ceiling(torch.bfloat16), 1),
                "fp16_8192^3": round(gemm_ceiling(torch.float16), 1),
                "bf16_bmm_32x8192x8192x128": round(bmm_ceiling(), 1)}
        gemm_best = max(gemm.values())
        stream_gbs, stream_shape = hbm_read_ceiling()
        dec_read = decode_read_ceiling()
        others = other_workloads()

    traffic_pre, traffic_dec = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "attention fwd bf16 causal B=2 H=16 Sq=Sk=8192 d=128 + split-KV decode "
                        "bf16 B=64 Hq=32 Hkv=8 Sk=8192 16 splits",
            "prefill": {"B": PREFILL.B, "Hq": PREFILL.Hq, "Hkv": PREFILL.Hkv, "Sq": PREFILL.Sq,
                        "Sk": PREFILL.Sk, "d": PREFILL.d, "causal": True},
            "decode": {"B": DECODE.B, "Hq": DECODE.Hq, "Hkv": DECODE.Hkv, "Sk": DECODE.Sk,
                       "d": DECODE.d, "num_splits": DECODE.num_splits},
            "parallelism": "none (1 GPU)",
        },
        "prefill": {"ms": round(pre_avg, 4), "ms_spread": spread(pre_ms),
                    "tflops": round(tflops, 2),
                    "frac_mfma_peak": round(tflops / PEAK_MFMA_TFLOPS, 4),
                    "frac_gemm_ceiling": ratio(tflops, gemm_best),
                    "flops": PREFILL.flops, "exp2_per_launch": PREFILL.flops // (4 * PREFILL.d)},
        "decode": {"ms": round(dec_avg, 4), "ms_spread": spread(dec_ms),
                   "value": round(dec_gbs, 1), "unit": "GB/s",
                   "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "frac_read_stream_ceiling": ratio(dec_gbs, stream_gbs),
                   "frac_decode_read_ceiling": ratio(dec_gbs, dec_read.get("two_arrays",
                                                                           float("nan"))),
                   "algorithmic_bytes": dec_bytes},
        "gemm_ceiling_tflops": gemm,
        "hbm_read_stream_ceiling": {"value": None if stream_shape is None else round(stream_gbs, 1),
                                    "unit": "GB/s",
                                    "shape": stream_shape, "bytes": 4 << 30},
        "decode_read_ceiling": {"unit": "GB/s", **dec_read},
        "other_workloads": others,
        "warmup_run": warm,
        "gpu_state": {"before": state_before, "after": state_after},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
                     "traffic": None if traffic_pre is None else traffic_pre["bytes"],
                     "traffic_detail": traffic_pre,
                     "algorithmic_bytes": prefill_algorithmic_bytes(PREFILL),
                     "kernel": "fa_fwd_kernel (bf16)"},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                            "traffic": None if traffic_dec is None else traffic_dec["bytes"],
                            "traffic_detail": traffic_dec,
                            "kernel": "fa_decode_split_kernel + fa_combine_kernel (bf16)"},
        "cpu_baseline": None,
    }
    ok = True
    if not args.skip_cpu_baseline:
        o_host = o.cpu()
        base, parity = cpu_baseline(q, k, v, o_host, args.cpu_seconds)
        result["cpu_baseline"] = base
        result["parity"] = {"prefill": parity, "decode": decode_parity(dq, dk, dv, do.cpu())}
        ok = parity["pass"] and result["parity"]["decode"]["pass"]
    if not ok:
        result["value"] = None
        print(json.dumps(result))
        sys.exit(1)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
