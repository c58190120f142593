"""The generated main loop of the scheduled FP8 forward kernel, executed on the
CPU by the instruction-level emulator (tests/gfx950_emu.py) for whole
workgroups, against the FP8 oracle's tiled model (no GPU needed).

Besides the values, the emulator checks load waits, hazard wait states (20
after an FP8 MFMA), barrier matching and LDS copy/read races of the schedule.
"""

import importlib.util
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle.fp8 import attention_fp8, attention_online_fp8, dequantise
from tests.gfx950_emu import Emulator

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_63_amd", "csrc")
D = 128
BC = 64
LN2 = math.log(2.0)


def _gen():
    spec = importlib.util.spec_from_file_location("gen_fwd_fp8_sched", os.path.join(CSRC, "gen_fwd_fp8_sched.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GEN = _gen()


def test_committed_file_matches_generator():
    with open(GEN.OUTPUT) as f:
        assert f.read() == GEN.generate()


def swz(row):
    """XOR pattern of the 16-byte chunks of a 128-byte LDS row: bits 1, 3, 2
    of the row give bits 1, 2, 0."""
    row = np.asarray(row)
    return (row & 2) | ((row >> 1) & 4) | ((row >> 2) & 1)


def init_wave(w, wave, q8, qblk, T, c, ntv):
    """Register state the C++ side establishes before the loop (LDS at 0)."""
    N = q8.shape[0]
    lanes = np.arange(64)
    lr, lh = lanes % 32, lanes // 32
    rows = qblk * 256 + 32 * w + lr
    for s in range(2):
        for i in range(8):
            word = np.zeros(64, dtype=np.uint32)
            for b in range(4):
                col = 64 * s + 32 * lh + 4 * i + b
                byte = np.where(rows < N, q8[np.minimum(rows, N - 1), col], 0).astype(np.uint32)
                word |= byte << (8 * b)
            wave.v[GEN.R_Q + 8 * s + i] = word
    for s in range(2):
        for e in range(2):
            ka = lr * D + 16 * ((2 * lh + e) ^ swz(lr))
            wave.v[GEN.R_KA + 2 * s + e] = ka ^ (64 * s)
    g, j = lanes // 16, lanes % 16
    r = j // 2
    vrow = 8 * (r // 4) + 4 * (g // 2) + r % 4
    vb = vrow * D + 16 * ((g & 1) ^ swz(vrow)) + 8 * (j & 1)
    for db in range(4):
        wave.v[GEN.R_VA + db] = vb ^ (32 * db)
    b = w * 1024 + 16 * lanes
    row, phys = b // D, (b % D) // 16
    wave.v[GEN.R_DSRC] = row * D + 16 * (phys ^ swz(row))
    wave.s[GEN.S_KDESC] = 1
    wave.s[GEN.S_VDESC] = 2
    wave.s[GEN.S_C] = int(np.float32(c).view(np.uint32))
    wave.s[GEN.S_T] = T
    wave.s[GEN.S_M0B] = 1024 * w
    wave.s[GEN.S_NTV] = ntv


def run_workgroup(q8, k8, v8, desc, scale, qblk, text=None, hits=None, T=None, lds_out=None):
    """One workgroup (query block qblk of 256 rows) over the first T full
    tiles of keys (all N = 64 T keys by default; N / 64 whole tiles bound the
    copies); returns the workgroup's O and LSE as the C++ epilogue forms
    them, over those T tiles."""
    N = q8.shape[0]
    ntv = N // BC
    T = ntv if T is None else T
    c = abs(scale * desc[0] * desc[1]) * math.log2(math.e)
    assert scale * desc[0] * desc[1] >= 0
    if text is None:
        text = "\n".join(GEN.block())
    emu = Emulator([text] * 8, 64 * 1024, {1: k8.tobytes(), 2: v8.tobytes()})
    for w, wave in enumerate(emu.waves):
        init_wave(w, wave, q8, qblk, T, c, ntv)
    # the C++ side copies K of tiles 0-2 and V of tiles 0-1 before the loop
    for tile in range(min(T, 3)):
        halves = [(k8, tile * GEN.TSZ)] + ([(v8, GEN.VOFF + tile * GEN.TSZ)] if tile < 2 else [])
        for src, base in halves:
            for rr in range(BC):
                for p in range(8):
                    ch = p ^ int(swz(rr))
                    dst = base + rr * D + 16 * p
                    emu.lds[dst:dst + 16] = src[tile * BC + rr, 16 * ch:16 * ch + 16]
    emu.run()
    if hits is not None:
        hits.update(emu.label_hits)
    if lds_out is not None:
        lds_out.append(emu.lds.copy())
    o = np.zeros((256, D))
    lse = np.zeros(256)
    for w, wave in enumerate(emu.waves):
        accf = wave.v[GEN.R_ACC:GEN.R_ACC + 64].view(np.float32).astype(np.float64)
        m = wave.v[GEN.R_M].view(np.float32).astype(np.float64)
        l = wave.v[GEN.R_L].view(np.float32).astype(np.float64)
        ltot = l[:32] + l[32:]
        assert np.array_equal(m[:32], m[32:]), "row reference differs between lane halves"
        for db in range(4):
            for r in range(16):
                for lh in range(2):
                    d = 32 * db + 8 * (r // 4) + 4 * lh + r % 4
                    o[32 * w:32 * w + 32, d] = accf[16 * db + r, 32 * lh:32 * lh + 32] * desc[2] / ltot
        lse[32 * w:32 * w + 32] = (m[:32] + np.log2(ltot) - 6) * LN2
    n = min(N, (qblk + 1) * 256) - qblk * 256
    return o[:n], lse[:n]


def model(q8, k8, v8, desc, scale, qblk):
    """The oracle's tiled model for the workgroup's rows, and the weight
    sum_j P~_j |v_j| / l of the accumulation bound."""
    tiles = []
    o, lse = attention_online_fp8(q8, k8, v8, *desc, False, scale, BC,
                                  trace=lambda j0, m, ps, pr: tiles.append((j0, m, ps, pr)))
    av = np.abs(dequantise(v8, desc[2]))
    m_f = tiles[-1][1]
    l = np.zeros(q8.shape[0])
    wr = np.zeros(q8.shape)
    for j0, m, ps, pr in tiles:
        f = np.exp(m - m_f)[:, None]
        l += (ps * f).sum(axis=1)
        wr += (pr * f) @ av[j0:j0 + ps.shape[1]]
    rows = slice(qblk * 256, min(q8.shape[0], (qblk + 1) * 256))
    return o[rows], lse[rows], (wr / l[:, None])[rows]


def head(x):
    return x[0, 0].numpy()


@pytest.mark.parametrize("N,qblk", [(256, 0), (64, 0), (128, 0), (192, 0), (320, 1), (512, 1)])
def test_loop_exact_inputs(N, qblk):
    """Integer base-2 scores: every 2^6 P is on the E4M3 grid, so the loop
    must agree with the model up to fp32 accumulation (no output cast here)."""
    (q8, k8, v8), desc, scale = W.make_exact_fp8(1, 1, N, D, seed=N + 7)
    q8, k8, v8 = head(q8), head(k8), head(v8)
    hits = {}
    o, lse, = run_workgroup(q8, k8, v8, desc, scale, qblk, hits=hits)
    om, lm, wr = model(q8, k8, v8, desc, scale, qblk)
    err = np.abs(o - om)
    assert (err <= 2.0 ** -11 * wr + 1e-12).all(), err.max()
    assert np.abs(lse - lm).max() <= 1e-5 + 2.0 ** -20 * np.abs(lm).max()


@pytest.mark.parametrize("N,qblk,seed", [(256, 0, 1), (448, 1, 2), (640, 2, 3)])
def test_loop_realistic_inputs(N, qblk, seed):
    """N(0, 1) inputs in E4M3: against exact attention within the LSE bar,
    and much closer to the model than the model is to exact attention."""
    (q8, k8, v8), desc = W.make_inputs_fp8(1, 1, N, D, seed=seed)
    q8, k8, v8 = head(q8), head(k8), head(v8)
    scale = 1 / math.sqrt(D)
    o, lse = run_workgroup(q8, k8, v8, desc, scale, qblk)
    om, lm, _ = model(q8, k8, v8, desc, scale, qblk)
    rows = np.arange(qblk * 256, min(N, (qblk + 1) * 256))
    ox, lx = attention_fp8(q8, k8, v8, *desc, False, scale, rows=rows)
    assert np.abs(lse - lx).max() <= 1e-3
    rms = lambda x: np.sqrt(np.mean(x ** 2))
    assert rms(o - om) <= 0.25 * rms(om - ox) + 2.0 ** -12 * rms(om)


def test_reference_moves():
    """Larger scores move the reference in several intervals: the
    out-of-line update and the end-of-interval rescale run, and the result
    still follows the model."""
    N = 448
    (q8, k8, v8), desc = W.make_inputs_fp8(1, 1, N, D, seed=9)
    q8, k8, v8 = head(q8), head(k8), head(v8)
    scale = 1.0 / math.sqrt(D) * 4.0
    hits = {}
    o, lse = run_workgroup(q8, k8, v8, desc, scale, 0, hits=hits)
    om, lm, _ = model(q8, k8, v8, desc, scale, 0)
    ox, lx = attention_fp8(q8, k8, v8, *desc, False, scale, rows=np.arange(256))
    assert np.abs(lse - lx).max() <= 1e-3
    rms = lambda x: np.sqrt(np.mean(x ** 2))
    assert rms(o - om) <= 0.25 * rms(om - ox) + 2.0 ** -12 * rms(om)
    assert hits.get(".Lfa2f8_move_0", 0) >= 3, hits


# ---- the emulator's own checks catch planted schedule mistakes --------------

def _planted(mutate):
    (q8, k8, v8), desc = W.make_inputs_fp8(1, 1, 512, D, seed=5)
    lines = mutate(list(GEN.block()))
    with pytest.raises(AssertionError) as ei:
        run_workgroup(head(q8), head(k8), head(v8), desc, 1 / math.sqrt(D), 0, text="\n".join(lines))
    return str(ei.value)


def test_emulator_catches_a_short_lds_wait():
    def mutate(lines):
        i = next(i for i, l in enumerate(lines) if l.startswith("s_waitcnt lgkmcnt(") and "(0)" not in l
                 and i > 200)
        n = int(lines[i][len("s_waitcnt lgkmcnt("):-1])
        lines[i] = f"s_waitcnt lgkmcnt({n + 2})"
        return lines
    assert "pending" in _planted(mutate)


def test_emulator_catches_a_missing_hazard_nop():
    def mutate(lines):
        i = next(i for i, l in enumerate(lines) if l == "s_nop 2")   # after the prologue's score MFMAs
        del lines[i]
        return lines
    assert "20 wait states" in _planted(mutate)


def test_emulator_catches_a_copy_race():
    def mutate(lines):
        return [l.replace("s_waitcnt vmcnt(2)", "s_waitcnt vmcnt(4)") for l in lines]
    assert "copy" in _planted(mutate)


def test_emulator_catches_a_missing_barrier():
    def mutate(lines):
        start = lines.index(".Lfa2f8_body1_%=:")
        i = next(i for i in range(start, len(lines)) if lines[i] == "s_barrier")
        del lines[i]
        return lines
    assert "copy" in _planted(mutate)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_tiles_after_the_loop(T):
    """With whole tiles after the loop's T (a causal workgroup's diagonal
    tiles), the loop's last copies leave K of tiles T..T+2 and V of tiles
    T..T+1 (those of them from tile 3 and 2 on, below N / 64) in their ring
    stages, and its result covers the first T tiles only."""
    N = 64 * (T + 4)
    (q8, k8, v8), desc = W.make_inputs_fp8(1, 1, N, D, seed=T)
    q8, k8, v8 = head(q8), head(k8), head(v8)
    scale = 1 / math.sqrt(D)
    lds = []
    o, lse = run_workgroup(q8, k8, v8, desc, scale, 0, T=T, lds_out=lds)
    # the first 64 T keys; rows below min(256, 64 T) as a 64 T-row problem
    n = min(256, 64 * T)
    ox, lx = attention_fp8(q8[:64 * T], k8[:64 * T], v8[:64 * T], *desc, False, scale, rows=np.arange(n))
    assert np.abs(lse[:n] - lx).max() <= 1e-3
    for kind, src, first, last, base in (("K", k8, 3, T + 2, 0), ("V", v8, 2, T + 1, GEN.VOFF)):
        for t in range(max(T, first), last + 1):
            st = base + (t % 4) * GEN.TSZ
            for rr in range(BC):
                for p in range(8):
                    ch = p ^ int(swz(rr))
                    got = lds[0][st + rr * D + 16 * p:st + rr * D + 16 * p + 16]
                    assert np.array_equal(got, src[t * BC + rr, 16 * ch:16 * ch + 16]), (kind, t, rr, p)
