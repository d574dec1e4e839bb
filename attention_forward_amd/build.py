"""Build libattn.so (the gfx950 kernels and their C ABI) in-tree with hipcc, and
libattn_bench.so (the benchmark's HBM read-stream probe, csrc_bench/).

    python -m attention_forward_amd.build            # build
    python -m attention_forward_amd.build --asm DIR  # also keep the gfx950 assembly
"""
from __future__ import annotations

import argparse
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
CSRC_BENCH = os.path.join(HERE, "csrc_bench")
LIB_BENCH = os.path.join(HERE, "libattn_bench.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libattn.so)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
        # keep packed-fp32 instructions out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


def _link(cc, srcs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc] + flags() + ["-shared", "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in res.stderr.splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err)
    os.replace(tmp, out)


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    _link(cc, sources(), LIB, verbose)
    _link(cc, sorted(glob.glob(os.path.join(CSRC_BENCH, "*.hip"))), LIB_BENCH, verbose)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for src in sources():
            out = os.path.join(asm_dir, os.path.basename(src) + ".s")
            subprocess.run([cc] + flags() + ["--cuda-device-only", "-S", "-o", out, src],
                           check=True, capture_output=True)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for gfx950 assembly listings")
    args = ap.parse_args()
    print(build(args.asm, verbose=True))
