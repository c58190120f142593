"""Build libfa2.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m exact_attention_63_amd.build [--verbose]

The library is compiled every time this runs.  Compiler resource-usage
remarks (VGPRs, AGPRs, spills, LDS, occupancy per kernel) are written next to
the library as ``libfa2.resource-usage.txt``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfa2.so")
SOURCES = [os.path.join(PKG, "csrc", "fa2_api.hip")]
HEADERS = [os.path.join(PKG, "csrc", "fa2_fwd_kernel.hpp"), os.path.join(PKG, "csrc", "fa2_fwd_sched.hpp"),
           os.path.join(PKG, "csrc", "fa2_fwd_sched.inc"), os.path.join(PKG, "csrc", "fa2_fwd_fp8.hpp"),
           os.path.join(PKG, "csrc", "fa2_fwd_fp8_sched.hpp"), os.path.join(PKG, "csrc", "fa2_fwd_fp8_sched.inc"),
           os.path.join(ROOT, "include", "fa2.h")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # no packed fp32 arithmetic (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code only: no NaN-quieting canonicalisation around max/min, so a
    # 3-input max is one v_max3_f32 (infinities, used for masking, are kept)
    "-Xarch_device", "-fno-honor-nans",
    "-Rpass-analysis=kernel-resource-usage",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(ROOT, "bench_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile bench.py's measurement probe (bench_probe.hip -> bench_probe.so,
    beside bench.py); it is not part of the library."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode} on {PROBE_SRC}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    remarks = [ln for ln in res.stderr.splitlines() if "remark" in ln or "Function Name" in ln
               or ln.strip().startswith(("VGPRs", "AGPRs", "SGPRs", "ScratchSize", "Occupancy", "LDS"))]
    with open(os.path.join(PKG, "libfa2.resource-usage.txt"), "w") as f:
        f.write("\n".join(remarks) + "\n")
    errors = [ln for ln in res.stderr.splitlines()
              if "remark" not in ln and "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        sys.stderr.write("\n".join(errors) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and errors:
        sys.stderr.write("\n".join(errors) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
    print(build_probe(verbose="--verbose" in sys.argv))
