"""Compile libmla_absorb.so (HIP kernels + C ABI) and the measurement probes
libmla_probe.so for gfx950, in-tree."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_absorb.so")
PROBE_LIB = os.path.join(HERE, "libmla_probe.so")
SOURCES = ["append.hip", "gemm.hip", "linear.hip", "attn.hip", "expand.hip", "plan.cpp", "capi.cpp"]
# the expanded-form prefill's two expansion GEMMs are plain matrix products (hipBLASLt)
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops stay off: the compiler would otherwise form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    # the attention kernel includes instruction sequences written by a generator
    sys.path.insert(0, CSRC)
    try:
        import gen_own_asm
    finally:
        sys.path.pop(0)
    gen_own_asm.main()
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES] + LIBS
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmla_absorb.so")
    os.replace(tmp, LIB)
    # the measurement probes bench.py reports next to the datasheet peaks
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc, *HIPCC_FLAGS, "-o", tmp, os.path.join(CSRC, "probe.hip")], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmla_probe.so")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
