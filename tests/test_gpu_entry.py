"""GPU: the C-ABI forward entry points called directly, the persistent form
of the d = 128 kernel, and the throughput workload compared in full.

Tolerances as in test_gpu_parity: O within 2e-3 (fp16) / 1e-2 (bf16), LSE
within 1e-3, max-abs against the fp64 oracle on the same rounded inputs.
"""

import math

import numpy as np
import pytest
import torch

import exact_attention_63_amd as fa2
import oracle
from workloads import WORKLOADS, make_inputs, to_f64, workload_inputs

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3
CODE = {"fp16": fa2.FA2_DTYPE_FP16, "bf16": fa2.FA2_DTYPE_BF16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    fa2.lib()


def max_err(o, lse, o_ref, l_ref):
    og = o if isinstance(o, np.ndarray) else to_f64(o)
    lg = lse if isinstance(lse, np.ndarray) else to_f64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    return np.abs(og - o_ref).max(), np.abs(lg - l_ref).max()


def assert_close(o, lse, o_ref, l_ref, dtype, what):
    eo, el = max_err(o, lse, o_ref, l_ref)
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype], what
    assert el <= TOL_LSE, what


# ------------------------------------------------------------ fa2_fwd and the typed entry points

@pytest.mark.parametrize("B,H,N,d,dtype,causal", [
    (1, 1, 128, 64, "fp16", False),      # the small workload
    (2, 3, 1000, 128, "bf16", True),     # ragged, causal (diagonal and tail tiles)
    (2, 3, 1000, 128, "fp16", True),
    (1, 2, 333, 64, "bf16", True),
])
def test_entry_points_match_binding(B, H, N, d, dtype, causal):
    """fa2_fwd (with its dtype argument) and fa2_fwd_fp16 / fa2_fwd_bf16 give
    the bits of the binding's call, and those match the oracle."""
    q, k, v = (x.cuda() for x in make_inputs(B, H, N, d, dtype, seed=91 + N))
    scale = 1.0 / math.sqrt(d)
    ref_o, ref_l = fa2.forward(q, k, v, causal=causal, scale=scale)
    lib = fa2.lib()
    typed = lib.fa2_fwd_fp16 if dtype == "fp16" else lib.fa2_fwd_bf16
    stream = torch.cuda.current_stream().cuda_stream
    for call in ("fa2_fwd", "typed"):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
        args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                int(causal), scale, stream]
        rc = lib.fa2_fwd(*args, CODE[dtype]) if call == "fa2_fwd" else typed(*args)
        assert rc == fa2.FA2_OK, call
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), call
    o_ref, l_ref = oracle.attention_3pass(to_f64(q), to_f64(k), to_f64(v), causal, scale)
    assert_close(ref_o, ref_l, o_ref, l_ref, dtype, f"B={B} H={H} N={N} d={d} {dtype} causal={causal}")


def test_entry_point_rejects_empty_problem():
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16, device="cuda")
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device="cuda")
    lib = fa2.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for B, H, N in ((0, 1, 64), (1, 0, 64), (1, 1, 0)):
        rc = lib.fa2_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr() + 8192, lse.data_ptr(),
                         B, H, N, 64, 0, 0.125, stream, fa2.FA2_DTYPE_FP16)
        assert rc == fa2.FA2_ERR_SHAPE


def test_binding_empty_problems():
    """The binding returns empty outputs for B, H or N == 0 without a library
    call, and still rejects what no size makes valid."""
    for shape in ((0, 2, 64, 64), (2, 0, 64, 128), (2, 3, 0, 64)):
        z = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        o, lse = fa2.forward(z, z, z)
        assert o.shape == shape and lse.shape == shape[:3]
    z = torch.empty((0, 2, 64, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa2.Fa2Error) as ei:
        fa2.forward(z, z, z)
    assert ei.value.status == fa2.FA2_ERR_UNSUPPORTED


# ------------------------------------------------------------ the throughput workload in full

def test_headline_workload_every_row():
    """B=8, H=32, N=2048, d=128 bf16, non-causal: every row of every head
    against the oracle, in the launch the benchmark times."""
    w = WORKLOADS["b8h32n2048d128_bf16"]
    q, k, v = workload_inputs(w)
    o, lse = fa2.forward(q.cuda(), k.cuda(), v.cuda(), causal=False, scale=w.scale)
    torch.cuda.synchronize()
    o64, l64 = to_f64(o), to_f64(lse)
    worst_o = worst_l = 0.0
    for b in range(w.B):
        o_ref, l_ref = oracle.attention_3pass(to_f64(q[b]), to_f64(k[b]), to_f64(v[b]), False, w.scale)
        assert np.all(np.isfinite(o64[b])) and np.all(np.isfinite(l64[b]))
        worst_o = max(worst_o, np.abs(o64[b] - o_ref).max())
        worst_l = max(worst_l, np.abs(l64[b] - l_ref).max())
        print(f"batch {b}: max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}", flush=True)
        assert worst_o <= TOL_O["bf16"] and worst_l <= TOL_LSE


# ------------------------------------------------------------ persistent workgroups

def persistent_variant():
    for vi in range(fa2.num_variants()):
        if fa2.variant_name(vi) == "w8_q32_k64_sched_persist":
            return vi
    pytest.fail("no persistent variant in the library")


def sched_variant():
    for vi in range(fa2.num_variants()):
        if fa2.variant_name(vi) == "w8_q32_k64_sched_ring4":
            return vi
    pytest.fail("no scheduled variant in the library")


@pytest.mark.parametrize("B,H,N,dtype,scale", [
    (1, 1, 256, "bf16", None),     # one item, four tiles
    (4, 40, 512, "bf16", None),    # 320 items: some workgroups run two
    (3, 31, 1024, "fp16", None),   # 372 items (not a multiple of 8)
    (4, 40, 512, "bf16", -0.3),    # negative scale: the next item's Q is sign-folded too
    (2, 64, 1280, "fp16", 0.05),   # 5 items per head, 640 items
])
def test_persistent_matches_oracle(B, H, N, dtype, scale):
    """The persistent kernel (one workgroup per CU, each loop prefetching the
    next item) gives the bits of the one-workgroup-per-item kernel, whose
    arithmetic it shares, and matches the oracle."""
    d = 128
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v = (x.cuda() for x in make_inputs(B, H, N, d, dtype, seed=7 + N + H))
    o_p, l_p = fa2.forward(q, k, v, causal=False, scale=scale, variant=persistent_variant())
    o_s, l_s = fa2.forward(q, k, v, causal=False, scale=scale, variant=sched_variant())
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_s) and torch.equal(l_p, l_s)
    heads = sorted({0, B * H // 2, B * H - 1})
    qf, kf, vf = (to_f64(x).reshape(B * H, N, d) for x in (q, k, v))
    o_ref, l_ref = oracle.attention_3pass(qf[heads], kf[heads], vf[heads], False, scale)
    o64 = to_f64(o_p).reshape(B * H, N, d)[heads]
    l64 = to_f64(l_p).reshape(B * H, N)[heads]
    eo, el = np.abs(o64 - o_ref).max(), np.abs(l64 - l_ref).max()
    print(f"persistent B={B} H={H} N={N}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype] + (2.0 ** -6 if scale < 0 else 0) and el <= TOL_LSE


def test_persistent_falls_back_off_shape():
    """Shapes the persistent form does not take (causal, N % 256 != 0, d = 64)
    run the variant's ordinary kernels."""
    vi = persistent_variant()
    for B, H, N, d, causal in ((1, 3, 1000, 128, False), (1, 3, 512, 128, True), (1, 3, 512, 64, False)):
        q, k, v = (x.cuda() for x in make_inputs(B, H, N, d, "bf16", seed=3 + N))
        o, lse = fa2.forward(q, k, v, causal=causal, variant=vi)
        o_ref, l_ref = oracle.attention_3pass(to_f64(q), to_f64(k), to_f64(v), causal, 1 / math.sqrt(d))
        assert_close(o, lse, o_ref, l_ref, "bf16", f"N={N} d={d} causal={causal}")


# ------------------------------------------------------------ causal grid order

@pytest.mark.parametrize("B,H,N,d,dtype", [
    (1, 8, 8192, 64, "fp16"),     # 64 query blocks of 128 rows per head: heads one after the other per XCD
    (1, 16, 16384, 128, "bf16"),  # 64 blocks of 256 rows
    (1, 3, 8192, 64, "bf16"),     # B*H not a multiple of 8: level by level
])
def test_causal_long_sequence_grid(B, H, N, d, dtype):
    """Causal launches whose grid takes each XCD's heads one after the other
    (or level by level): every row of one head, strided rows of all heads."""
    q, k, v = make_inputs(B, H, N, d, dtype, seed=5 + H)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa2.forward(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    o64, l64 = to_f64(o), to_f64(lse)
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    o_ref, l_ref = oracle.attention_3pass(q64[0, H - 1], k64[0, H - 1], v64[0, H - 1], True, scale)
    assert_close(o64[0, H - 1], l64[0, H - 1], o_ref, l_ref, dtype, f"head {H - 1} all rows")
    rows = np.unique(np.concatenate([np.arange(0, N, 97), np.arange(N - 40, N)]))
    o_ref, l_ref = oracle.attention_3pass(q64, k64, v64, True, scale, rows=rows)
    assert_close(o64[:, :, rows], l64[:, :, rows], o_ref, l_ref, dtype, f"{rows.size} rows x all heads")
