"""Run one workload's launches alone, for a profiler to record.

    python attention_forward_amd/profile_run.py WORKLOAD [--launches N] [--warmup-seconds S]
        [--split] [--copy-mib M]

WORKLOAD is a name from synthetic.ALL_WORKLOADS or synthetic.FP8_WORKLOADS.
The process generates that workload's seeded inputs, moves them to the GPU,
warms the kernels up for S seconds (the clock under sustained load settles
within about a second), then issues N more launches and prints their mean
duration from HIP events.  Under `rocprofv3 --kernel-trace`, the last N
dispatches of each kernel are the measured ones (`profsum stats --last N`);
one process per workload keeps shapes from mixing in a kernel's statistics.
Prefill workloads whose grid leaves compute units idle also run the split-KV
form with the recommended split count when `--split` is given.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    import torch

    import attention_forward_amd as A
    from attention_forward_amd.synthetic import (ALL_WORKLOADS, FP8_WORKLOADS, TORCH_DTYPE,
                                                 make_qkv_fp8, make_workload_inputs)

    ap = argparse.ArgumentParser()
    ap.add_argument("workload", choices=sorted(ALL_WORKLOADS) + sorted(FP8_WORKLOADS))
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--warmup-seconds", type=float, default=1.5)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="afterwards, one plain device copy of this many MiB (a known-size "
                         "kernel for scaling HBM byte counters)")
    ap.add_argument("--split", action="store_true",
                    help="run attn_fwd_split with the recommended split count instead")
    a = ap.parse_args()
    A.lib()
    dev = torch.device("cuda", 0)
    fp8 = a.workload in FP8_WORKLOADS
    w = FP8_WORKLOADS[a.workload] if fp8 else ALL_WORKLOADS[a.workload]
    if fp8:
        (q, k, v), ds = make_qkv_fp8(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.seed)
        o = torch.empty((w.B, w.Hq, w.Sq, w.d), device=dev, dtype=TORCH_DTYPE[w.dtype])
    else:
        q, k, v = make_workload_inputs(w)
        o = torch.empty(q.shape, device=dev, dtype=q.dtype)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    if w.decode:
        lse = torch.empty((w.B, w.Hq), device=dev, dtype=torch.float32)
        ws = torch.empty(A.attn_decode_workspace_bytes(w.B, w.Hq, w.d, w.num_splits),
                         device=dev, dtype=torch.uint8)

        def run():
            A.attn_fwd_decode(q, k, v, w.num_splits, scale=w.scale, out=o, lse=lse, workspace=ws)
    else:
        lse = torch.empty((w.B, w.Hq, w.Sq), device=dev, dtype=torch.float32)
        if fp8:
            def run():
                A.attn_fwd_fp8(q, k, v, causal=w.causal, scale=w.scale, q_descale=ds[0],
                               k_descale=ds[1], v_descale=ds[2], out=o, lse=lse)
        elif a.split:
            ns = A.attn_fwd_num_splits(w.B, w.Hq, w.Sq, w.Sk, w.d)
            ws = torch.empty(A.attn_fwd_split_workspace_bytes(w.B, w.Hq, w.Sq, w.d, ns),
                             device=dev, dtype=torch.uint8)

            def run():
                A.attn_fwd_split(q, k, v, ns, causal=w.causal, scale=w.scale, out=o, lse=lse,
                                 workspace=ws)
        else:
            def run():
                A.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    t0 = time.perf_counter()
    n_warm = 0
    while time.perf_counter() - t0 < a.warmup_seconds:
        for _ in range(5):
            run()
        n_warm += 5
        torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(a.launches):
        run()
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / a.launches
    rate = ("%.1f GB/s (K/V bytes)" % (2 * w.B * w.Hkv * w.Sk * w.d * 2 / (ms * 1e-3) / 1e9)
            if w.decode else "%.1f TFLOP/s" % (w.flops / (ms * 1e-3) / 1e12))
    if a.copy_mib > 0:
        src = torch.ones(a.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    print("%s%s: %d warmup launches, then %d launches at %.4f ms each (%s)"
          % (w.name, " split" if a.split else "", n_warm, a.launches, ms, rate), flush=True)


if __name__ == "__main__":
    main()
