"""Every kernel a default configuration launches is free of register spills
and private (scratch) memory, by the compiler's resource-usage remarks that
the build writes next to the library (libfa2.resource-usage.txt)."""

import os
import re
import shutil
import subprocess

import pytest

import exact_attention_63_amd as fa2
from exact_attention_63_amd import build as fa2_build

REPORT = os.path.join(os.path.dirname(fa2_build.LIB), "libfa2.resource-usage.txt")

# The kernels behind variant 0 of the forward and backward calls, for both
# dtypes and causal flags, and the FP8 forward kernels (demangled names).
B = ("false", "true")
DEFAULT_KERNELS = (
    [f"void fa2::fa2_fwd_sched_kernel<{b}, {c}>(fa2::Args)" for b in B for c in B]
    + [f"void fa2::fa2_fwd_sched_persist_kernel<{b}>(fa2::Args)" for b in B]
    + [f"void fa2::fa2_fwd_kernel<{b}, 64, {c}, fa2::Tile<8, 1, 4, 2, 2, 4, 0> >(fa2::Args)" for b in B for c in B]
    + [f"void fa2::fa2_bwd_delta_kernel<{b}, {d}>(fa2::BwdArgs, long long)" for b in B for d in (64, 128)]
    + [f"void fa2::fa2_bwd_dkdv_pipe_kernel<{b}, {d}, {c}, 2>(fa2::BwdArgs)" for b in B for d in (64, 128) for c in B]
    + [f"void fa2::fa2_bwd_dq_kernel<{b}, {d}, {c}, fa2::BwdTile<8, 2>, 4>(fa2::BwdArgs)"
       for b in B for d in (64, 128) for c in B]
    + [f"void fa2::fa2_fwd_fp8_kernel<{d}, false, 4, 3>(fa2::Fp8Args)" for d in (64, 128)]
    + ["void fa2::fa2_fwd_fp8_kernel<64, true, 8, 2>(fa2::Fp8Args)"]
    + ["void fa2::fa2_fwd_fp8_sched_kernel<true>(fa2::Fp8Args)"]
)

# variant 0 resolves to these tile variants (the list above follows them)
DEFAULT_FWD = {(128, 0): "w8_q32_k64_sched_persist", (128, 1): "w8_q32_k64_sched_persist",
               (64, 0): "w8_q32_k128_dma2_look4", (64, 1): "w8_q32_k128_dma2_look4"}


def _sources():
    csrc = os.path.join(os.path.dirname(fa2_build.LIB), "csrc")
    return [os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".inc"))]


@pytest.fixture(scope="module")
def usage():
    stale = not os.path.exists(REPORT) or not os.path.exists(fa2_build.LIB) or \
        os.path.getmtime(REPORT) < max(os.path.getmtime(p) for p in _sources())
    if stale:
        fa2_build.build()
    filt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    if filt is None:
        pytest.skip("no c++filt to demangle kernel names")
    entries = {}
    name = None
    with open(REPORT) as f:
        for line in f:
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                entries[name] = {}
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
            if m and name:
                entries[name][m.group(1).strip()] = int(m.group(2))
    mangled = list(entries)
    out = subprocess.run([filt], input="\n".join(mangled), capture_output=True, text=True, check=True).stdout
    return {dem: entries[m] for m, dem in zip(mangled, out.splitlines())}


# FP8: variant 0 resolves to these (the list above follows them)
DEFAULT_FP8 = {(128, 0): "tile_by_tile", (128, 1): "sched_ring4", (64, 0): "tile_by_tile", (64, 1): "tile_by_tile"}


def test_defaults_are_the_listed_variants():
    for (d, causal), name in DEFAULT_FWD.items():
        for dt in (fa2.FA2_DTYPE_FP16, fa2.FA2_DTYPE_BF16):
            assert fa2.variant_name(fa2.default_variant(dt, d, causal)) == name
    for (d, causal), name in DEFAULT_FP8.items():
        assert fa2.fp8_variant_name(fa2.lib().fa2_fp8_default_variant(d, causal)) == name


def test_default_kernels_do_not_spill(usage):
    bad = []
    for k in DEFAULT_KERNELS:
        assert k in usage, f"{k} not in the resource report"
        u = usage[k]
        for key in ("ScratchSize", "VGPRs Spill", "SGPRs Spill"):
            assert key in u, (k, key)
            if u[key] != 0:
                bad.append(f"{k}: {key} {u[key]}")
    assert not bad, "\n".join(bad)
