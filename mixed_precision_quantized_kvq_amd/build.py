"""Build libkvq.so (HIP for gfx950 + host C++) in-tree with hipcc.

Usage: python -m mixed_precision_quantized_kvq_amd.build  (or build() from Python).
Every source is compiled each time this runs; objects go to _build/ next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkvq.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++20", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-I", CSRC, "-Wall", "-Wno-unused-function",
          # packed-FP32 instructions are kept out of every kernel
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# exact-rounding sources: no fused multiply-add anywhere (quantizer, SSE, fit, allocator)
EXACT = ["-ffp-contract=off"]

SOURCES = {
    "kvq_host.cpp": EXACT,
    "kvq_abi.cpp": EXACT,
    "append.hip": EXACT,
    "calib.hip": EXACT,
    # MFMA accumulators in ordinary VGPRs: no accumulator-register copies in the decode loop.
    # The iterative ILP scheduler: 2-3 % faster split-K decode on the 32k- and 128k-token
    # workloads than the default schedule (same instructions, no spills); it made the append
    # flush slower and does not compile the 16-row tile, so those keep the default
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "decode_dense.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(name, extra):
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, name + ".o")
    # every source, the host-only .cpp files included, is compiled as HIP: those call the HIP
    # runtime and launch through the .hip files' launchers, and one language keeps the
    # runtime headers' configuration identical across objects
    cmd = [HIPCC] + COMMON + extra + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile {name} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    objs = [o for o, _ in results]
    for (name, _), (_, warn) in zip(SOURCES.items(), results):
        if warn and verbose:
            print(f"[{name}]\n{warn}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
