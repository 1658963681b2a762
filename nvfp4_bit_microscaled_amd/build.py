"""Build the gfx950 HIP library libnvfp4_amd.so in-tree with hipcc.

Flags: -ffp-contract=off keeps every binary32 step of the quantizer a single
IEEE operation (the codes must match the oracle bit for bit); packed-FP32 ops
are disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4_amd.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "ns.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 4) -> str:
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs)
            procs = []
    _wait(procs)
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(procs):
    bad = [p.args for p in procs if p.wait() != 0]
    if bad:
        raise RuntimeError(f"hipcc failed: {bad[0]}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
