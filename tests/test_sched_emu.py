"""The generated main loop of the scheduled forward kernel, executed on the
CPU by an instruction-level emulator (tests/gfx950_emu.py) for whole
workgroups, against the fp64 oracle (no GPU needed).

Besides the values, the emulator checks load waits, hazard wait states,
barrier matching and LDS copy/read races of the schedule.
"""

import importlib.util
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gfx950_emu import Emulator

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_63_amd", "csrc")
D = 128


def _gen():
    spec = importlib.util.spec_from_file_location("gen_fwd_sched", os.path.join(CSRC, "gen_fwd_sched.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GEN = _gen()


def test_committed_file_matches_generator():
    with open(GEN.OUTPUT) as f:
        assert f.read() == GEN.generate()


def swz(row):
    """XOR pattern of the 16-byte chunks of LDS row `row` (d = 128)."""
    return ((row & 3) << 2) | ((row >> 2) & 3)


def bits16(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16), t.to(torch.float64).numpy()


def init_wave(w, wave, qbits, N, qblk, T, c, ntv=None):
    """Register state the C++ side establishes before the loop."""
    lanes = np.arange(64)
    lr, lh = lanes % 32, lanes // 32
    q_w = qblk * 256 + 32 * w
    rows = q_w + lr
    for dk in range(8):
        for i in range(4):
            d0 = 16 * dk + 8 * lh + 2 * i
            lo = np.where(rows < N, qbits[np.minimum(rows, N - 1), d0], 0).astype(np.uint32)
            hi = np.where(rows < N, qbits[np.minimum(rows, N - 1), d0 + 1], 0).astype(np.uint32)
            wave.v[4 * dk + i] = lo | (hi << 16)
    for dk in range(8):
        wave.v[GEN.R_KA + dk] = lr * 256 + 16 * ((2 * dk + lh) ^ np.vectorize(swz)(lr))
    g, e, cc = lanes // 16, (lanes % 16) // 4, lanes % 4
    for db in range(4):
        for h in range(2):
            rr = 4 * (g // 2) + e + 8 * h
            chunk = 4 * db + 2 * (g % 2) + cc // 2
            wave.v[GEN.R_VA + 2 * db + h] = GEN.VOFF + rr * 256 + 16 * (chunk ^ np.vectorize(swz)(rr)) + 8 * (cc % 2)
    for k in range(2):
        r = (2 * w + k) * 4 + lanes // 16
        wave.v[GEN.R_DSRC + k] = r * 256 + 16 * ((lanes % 16) ^ np.vectorize(swz)(r))
    wave.s[GEN.S_KDESC] = 1
    wave.s[GEN.S_VDESC] = 2
    wave.s[GEN.S_C] = int(np.float32(c).view(np.uint32))
    wave.s[GEN.S_T] = T
    wave.s[GEN.S_M0B] = 2048 * w
    # no next item: its descriptors are the current ones; past tile T-1 the
    # copies fetch this head's whole tiles
    wave.s[GEN.S_NKD] = 1
    wave.s[GEN.S_NVD] = 2
    wave.s[GEN.S_HASN] = 0
    wave.s[GEN.S_NSUB] = 0
    wave.s[GEN.S_NTV] = ntv if ntv is not None else T


def run_workgroup(dtype, q, k, v, qblk, T, scale, text=None, hits=None):
    N = q.shape[0]
    qb, q64 = bits16(q, dtype)
    kb, k64 = bits16(k, dtype)
    vb, v64 = bits16(v, dtype)
    c = abs(scale) * math.log2(math.e)
    assert scale >= 0
    dt = "bf16" if dtype == "bf16" else "f16"
    if text is None:
        text = "\n".join(GEN.block(dt))
    emu = Emulator([text] * 8, 128 * 1024, {1: kb.tobytes(), 2: vb.tobytes()})
    for w, wave in enumerate(emu.waves):
        init_wave(w, wave, qb, N, qblk, T, c)
    # the C++ side copies K of tiles 0-2 and V of tiles 0-1 before the loop
    for tile in range(min(T, 3)):
        halves = [(kb, tile * GEN.TSZ)] + ([(vb, GEN.VOFF + tile * GEN.TSZ)] if tile < 2 else [])
        for src, base in halves:
            for r in range(64):
                for p in range(16):
                    row, ch = tile * 64 + r, p ^ swz(r)
                    dst = base + r * 256 + 16 * p
                    emu.lds[dst:dst + 16] = np.frombuffer(src[row, 8 * ch:8 * ch + 8].tobytes(), dtype=np.uint8)
    emu.run()
    if hits is not None:
        hits.update(emu.label_hits)
    # epilogue: O = acc / l, LSE = (m + log2 l) ln 2
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
                    o[32 * w:32 * w + 32, d] = accf[16 * db + r, 32 * lh:32 * lh + 32] / ltot
        lse[32 * w:32 * w + 32] = (m[:32] + np.log2(ltot)) * math.log(2)
    assert N == 64 * T, "the loop covers every key: N = 64 T"
    rows = np.arange(qblk * 256, min(N, qblk * 256 + 256))
    o_ref, l_ref = oracle.attention_3pass(q64, k64, v64, False, scale, rows=rows)
    return o[:rows.size], lse[:rows.size], o_ref, l_ref


TOL_O = {"bf16": 1e-2, "fp16": 2e-3}


@pytest.mark.parametrize("dtype,N,qblk,T,seed", [
    ("bf16", 256, 0, 4, 1),
    ("bf16", 64, 0, 1, 2),
    ("bf16", 128, 0, 2, 3),
    ("bf16", 320, 1, 5, 4),
    ("fp16", 192, 0, 3, 5),
    ("bf16", 512, 1, 8, 6),
    ("fp16", 640, 2, 10, 7),
])
def test_loop_matches_oracle(dtype, N, qblk, T, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((N, D), dtype=np.float32) for _ in range(3))
    hits = {}
    o, lse, o_ref, l_ref = run_workgroup(dtype, q, k, v, qblk, T, 1 / math.sqrt(D), hits=hits)
    assert np.abs(o - o_ref).max() <= TOL_O[dtype]
    assert np.abs(lse - l_ref).max() <= 1e-3
    # N(0, 1) inputs at scale 1/sqrt(d) never need the exact update
    assert not any("_exact" in name for name in hits)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_exact_update_path(dtype):
    """Later tiles with much larger scores force the out-of-line exact update
    (the lane row sums exceed the bound) in several intervals."""
    rng = np.random.default_rng(11)
    N, T = 320, 5
    q = rng.standard_normal((N, D), dtype=np.float32)
    k = rng.standard_normal((N, D), dtype=np.float32)
    k *= (0.05 + 0.5 * (np.arange(N) // 64))[:, None].astype(np.float32)
    v = rng.standard_normal((N, D), dtype=np.float32)
    hits = {}
    o, lse, o_ref, l_ref = run_workgroup(dtype, q, k, v, 0, T, 0.4, hits=hits)
    assert np.abs(o - o_ref).max() <= TOL_O[dtype]
    assert np.abs(lse - l_ref).max() <= 1e-3
    taken = {name for name in hits if "_exact" in name}
    assert len(taken) >= 3, taken        # several ring stages went through it


# ---- the emulator's own checks catch planted schedule mistakes --------------

def _planted(mutate):
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((512, D), dtype=np.float32) for _ in range(3))
    lines = GEN.block("bf16")
    lines = mutate(list(lines))
    with pytest.raises(AssertionError) as ei:
        run_workgroup("bf16", q, k, v, 0, 8, 1 / math.sqrt(D), text="\n".join(lines))
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
        i = next(i for i, l in enumerate(lines) if l == "s_nop 3")   # after the prologue's score MFMAs
        del lines[i]
        del lines[i - 1]
        return lines
    assert "12 wait states" in _planted(mutate)


def test_emulator_catches_a_copy_race():
    def mutate(lines):
        # let the copies of the interval stay in flight across the barrier
        return [l.replace("s_waitcnt vmcnt(4)", "s_waitcnt vmcnt(8)") for l in lines]
    assert "copy" in _planted(mutate)


def test_emulator_catches_a_missing_barrier():
    def mutate(lines):
        start = lines.index(".Lfa2s_body1_%=:")
        i = next(i for i in range(start, len(lines)) if lines[i] == "s_barrier")
        del lines[i]
        return lines
    assert "copy" in _planted(mutate)


# ---- persistent workgroups: one workgroup runs several items in a row ------

def _desc(s, base, buf_id, nbytes):
    s[base], s[base + 1], s[base + 2], s[base + 3] = buf_id, 0, nbytes, 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_consecutive_items(dtype):
    """Three items (head, query block) of different heads through one
    workgroup: each loop copies the next item's first K/V tiles and loads its
    Q in its last intervals, the next loop starts from them."""
    rng = np.random.default_rng(21)
    N, T = 512, 8
    heads = [tuple(rng.standard_normal((N, D), dtype=np.float32) for _ in range(3)) for _ in range(2)]
    items = [(0, 1), (1, 0), (1, 1)]          # (head, query block)
    scale = 1 / math.sqrt(D)
    c = scale * math.log2(math.e)
    bits = [tuple(bits16(x, dtype)[0] for x in h) for h in heads]
    f64 = [tuple(bits16(x, dtype)[1] for x in h) for h in heads]
    buffers = {}
    for h, (qb_, kb_, vb_) in enumerate(bits):
        buffers[10 + 3 * h], buffers[11 + 3 * h], buffers[12 + 3 * h] = qb_.tobytes(), kb_.tobytes(), vb_.tobytes()
    dt = "bf16" if dtype == "bf16" else "f16"
    text = "\n".join(GEN.block(dt))
    state = None
    for i, (h, qblk) in enumerate(items):
        emu = Emulator([text] * 8, 128 * 1024, buffers, copies_may_continue=i + 1 < len(items))
        for w, wave in enumerate(emu.waves):
            init_wave(w, wave, bits[h][0], N, qblk, T, c)
            if state is not None:                 # the previous block's registers and LDS
                wave.v[:GEN.R_Q + 32] = state[0][w][:GEN.R_Q + 32]
            lanes = np.arange(64)
            wave.v[GEN.R_QOFF] = (lanes % 32) * 256 + 16 * (lanes // 32)
            _desc(wave.s, GEN.S_KDESC, 11 + 3 * h, N * 256)
            _desc(wave.s, GEN.S_VDESC, 12 + 3 * h, N * 256)
            wave.s[GEN.S_NSUB] = T          # persistent: past tile T-1, the next item's tiles
            wave.s[GEN.S_NTV] = T
            if i + 1 == len(items):
                _desc(wave.s, GEN.S_NKD, 11 + 3 * h, N * 256)
                _desc(wave.s, GEN.S_NVD, 12 + 3 * h, N * 256)
            else:
                hn, qn = items[i + 1]
                _desc(wave.s, GEN.S_NKD, 11 + 3 * hn, N * 256)
                _desc(wave.s, GEN.S_NVD, 12 + 3 * hn, N * 256)
                _desc(wave.s, GEN.S_NQD, 10 + 3 * hn, N * 256)
                wave.s[GEN.S_NQOFF] = (qn * 256 + 32 * w) * 256
                wave.s[GEN.S_HASN] = 1
        if state is None:
            for tile in range(3):
                halves = [(bits[h][1], tile * GEN.TSZ)] + ([(bits[h][2], GEN.VOFF + tile * GEN.TSZ)] if tile < 2 else [])
                for src, base in halves:
                    for r in range(64):
                        for p in range(16):
                            row, ch = tile * 64 + r, p ^ swz(r)
                            dst = base + r * 256 + 16 * p
                            emu.lds[dst:dst + 16] = np.frombuffer(src[row, 8 * ch:8 * ch + 8].tobytes(), dtype=np.uint8)
        else:
            emu.lds[:] = state[1]
        emu.run()
        state = ([wave.v.copy() for wave in emu.waves], emu.lds.copy())
        # this item's output
        o = np.zeros((256, D))
        lse = np.zeros(256)
        for w, wave in enumerate(emu.waves):
            accf = wave.v[GEN.R_ACC:GEN.R_ACC + 64].view(np.float32).astype(np.float64)
            m = wave.v[GEN.R_M].view(np.float32).astype(np.float64)
            l = wave.v[GEN.R_L].view(np.float32).astype(np.float64)
            ltot = l[:32] + l[32:]
            for db in range(4):
                for r in range(16):
                    for lh in range(2):
                        d = 32 * db + 8 * (r // 4) + 4 * lh + r % 4
                        o[32 * w:32 * w + 32, d] = accf[16 * db + r, 32 * lh:32 * lh + 32] / ltot
            lse[32 * w:32 * w + 32] = (m[:32] + np.log2(ltot)) * math.log(2)
        rows = np.arange(qblk * 256, qblk * 256 + 256)
        o_ref, l_ref = oracle.attention_3pass(*f64[h], False, scale, rows=rows)
        assert np.abs(o - o_ref).max() <= TOL_O[dtype], (i, np.abs(o - o_ref).max())
        assert np.abs(lse - l_ref).max() <= 1e-3, i


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_tiles_after_the_loop(T):
    """One item whose head has 4 whole tiles after the loop's T (a causal
    workgroup's diagonal tiles): the loop's last copies leave K of tiles
    T..T+2 and V of tiles T..T+1 (those of them from tile 3 and 2 on) in
    their ring stages, and its result covers the first T tiles."""
    rng = np.random.default_rng(30 + T)
    N = 64 * (T + 4)
    q, k, v = (rng.standard_normal((N, D), dtype=np.float32) for _ in range(3))
    qb, q64 = bits16(q, "bf16")
    kb, k64 = bits16(k, "bf16")
    vb, v64 = bits16(v, "bf16")
    scale = 1 / math.sqrt(D)
    text = "\n".join(GEN.block("bf16"))
    emu = Emulator([text] * 8, 128 * 1024, {1: kb.tobytes(), 2: vb.tobytes()})
    for w, wave in enumerate(emu.waves):
        init_wave(w, wave, qb, N, 0, T, scale * math.log2(math.e), ntv=N // 64)
    for tile in range(min(T, 3)):
        halves = [(kb, tile * GEN.TSZ)] + ([(vb, GEN.VOFF + tile * GEN.TSZ)] if tile < 2 else [])
        for src, base in halves:
            for r in range(64):
                for p in range(16):
                    row, ch = tile * 64 + r, p ^ swz(r)
                    dst = base + r * 256 + 16 * p
                    emu.lds[dst:dst + 16] = np.frombuffer(src[row, 8 * ch:8 * ch + 8].tobytes(), dtype=np.uint8)
    emu.run()
    for src, first, last, base in ((kb, 3, T + 2, 0), (vb, 2, T + 1, GEN.VOFF)):
        for t in range(max(T, first), last + 1):
            st = base + (t % 4) * GEN.TSZ
            for r in range(64):
                for p in range(16):
                    ch = p ^ swz(r)
                    want = np.frombuffer(src[t * 64 + r, 8 * ch:8 * ch + 8].tobytes(), dtype=np.uint8)
                    assert np.array_equal(emu.lds[st + r * 256 + 16 * p:st + r * 256 + 16 * p + 16], want), (t, r, p)
    # the loop's own result: the first T tiles of keys
    lse = np.zeros(256)
    for w, wave in enumerate(emu.waves):
        m = wave.v[GEN.R_M].view(np.float32).astype(np.float64)
        l = wave.v[GEN.R_L].view(np.float32).astype(np.float64)
        lse[32 * w:32 * w + 32] = (m[:32] + np.log2(l[:32] + l[32:])) * math.log(2)
    n = min(256, 64 * T)
    _, l_ref = oracle.attention_3pass(q64[:64 * T], k64[:64 * T], v64[:64 * T], False, scale, rows=np.arange(n))
    assert np.abs(lse[:n] - l_ref).max() <= 1e-3
