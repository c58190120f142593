#!/usr/bin/env python3
"""Generate fa2_fwd_fp8_sched.inc: the main loop of the scheduled FP8 (E4M3)
forward kernel (fa2_fwd_fp8_sched.hpp) as gfx950 assembly.

    python exact_attention_63_amd/csrc/gen_fwd_fp8_sched.py

What the loop computes (one workgroup of 8 waves x 32 query rows, d = 128,
64-key tiles of 8 KiB; "FlashAttention v2 better parallelism + work
partitioning" diagram, concept pseudo-code panel; the FP8 scheme of
fa2_fwd_fp8.hpp): for every full key tile j, S(j)^T = K(j) Q^T on the FP8
matrix cores, the lazy reference rule (the row's reference m moves to the
tile max only when that exceeds m by more than 2.75, base 2), P(j) =
2^(S(j) c - m + 6) added to l in fp32 and rounded to E4M3, then
acc += V(j)^T P(j)^T on the FP8 matrix cores.

Schedule (as in gen_fwd_sched.py, with FP8 operands).  Tile j lives in ring
stage j % 4 (K and V, 8 KiB each), copied with buffer_load ... lds: K(j+3)
and V(j+2) in interval j, one 1 KiB instruction per wave and tensor.  The
copies of the last intervals fetch the tiles after the last full one when
they are whole tiles of the head (the diagonal tiles of a causal workgroup,
which the C++ code after the loop then finds in their ring stages), else
tile 0 again into a stage no wave reads.  Every wave
runs the same program; in interval j it issues the 4 P.V MFMAs of tile j-1,
then the 4 score MFMAs of tile j+1, and between those 8 MFMAs the softmax of
tile j: first the lane max of the raw scores (two v_max3 chains) and the
check of the reference rule, then staggered rounds (x = s c - ref of four
values, 2^x of the four before, row sums and E4M3 packing of the four before
those), so that no VALU result is used by the next instruction.  A wave in
which some row moves its reference branches to a short out-of-line path (row
max, new m, alpha = 2^(m_old - m_new)) before any 2^x; acc is multiplied by
alpha at the end of the interval, after the P.V MFMAs of tile j-1 and before
those of tile j.  That is the conditional rescale of the "FlashAttention v4
Blackwell pipeline co-design" diagram with the threshold of the FP8 scheme,
and the overlap its pseudo-code panel asks for (softmax of one tile while
the matrix cores work on the neighbouring ones), by software pipelining
inside each wave.

P(j) is packed into the first 8 registers of its own score buffer (the
packing of group g, registers 4g..4g+3, goes to register g, which is free
once groups 0 and 1 are packed); the P.V MFMAs of tile j read it in interval
j+1 before the score MFMAs of tile j+2 overwrite that buffer.

Registers are fixed (the C++ side binds its values to them, see
fa2_fwd_fp8_sched.hpp), so the output is plain assembly with no operand
references; labels carry %= so that every instance is unique.
"""

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUTPUT = os.path.join(HERE, "fa2_fwd_fp8_sched.inc")

# ---- problem geometry ------------------------------------------------------
D = 128                 # head dimension (bytes per K / V row)
BC = 64                 # keys per tile
TSZ = BC * D            # bytes of one K (or V) tile: 8 KiB
NS = 4                  # ring stages
VOFF = NS * TSZ         # V stages follow the K stages (in the read offsets)
KS = D // 64            # 64-wide d steps of the score product (2)
DB = D // 32            # 32-row blocks of O^T (4)
LAZY = 0x40300000       # 2.75f: the reference moves past m + 2.75 (base 2)
MSHIFT = 0xC0C00000     # -6.0f: ref = m - 6, so P = 2^(s c - m + 6)
LK = 2                  # K operands read ahead of the score MFMAs
LV = 2                  # V^T operands read ahead of the P.V MFMAs
NKB = LK + 2            # K operand buffers (refilled two MFMAs after their use)
NVB = LV + 2            # V^T operand buffers
MFMA_WAIT = 20          # wait states from an FP8 MFMA to a VALU read of its result

# ---- register map (VGPRs) ---------------------------------------------------
R_Q = 0                 # v[0:15]    Q fragments, B operand of S^T = K Q^T (2 x 8)
R_ACC = 16              # v[16:79]   O^T accumulators (4 x 16)
R_S = 80                # v[80:143]  two score buffers (2 x 2 x 16); P packed into the first 8
R_KA = 144              # v[144:147] K fragment LDS addresses (d step s, half e: 2 s + e)
R_VA = 148              # v[148:151] V^T fragment LDS addresses (d block)
R_DSRC = 152            # this lane's copy source offset inside a tile (its 1 KiB block)
R_M = 153               # reference max m (base 2)
R_L = R_M + 1           # row sum (P scaled by 2^6)
R_ALPHA = R_M + 2       # 2^(m_old - m_new) of the current tile (1 when no row moved)
R_MT = R_M + 3          # m + 2.75
R_REF = R_M + 4         # m - 6
R_RS0, R_RS1, R_T0, R_T1 = R_M + 5, R_M + 6, R_M + 7, R_M + 8
R_KBUF = R_M + 11       # K operand buffers (8 registers each)
R_VBUF = R_KBUF + 8 * NKB
R_END = R_VBUF + 8 * NVB   # first VGPR the loop does not touch
# register tuples must start at an even register
assert all(r % 2 == 0 for r in (R_Q, R_ACC, R_S, R_KA, R_VA, R_KBUF, R_VBUF))

# ---- register map (SGPRs) ---------------------------------------------------
S_KDESC, S_VDESC = 40, 44   # buffer descriptors of this head's K and V
S_C = 48                # c = |scale * dq * dk| * log2(e)
S_T = 49                # number of full tiles T >= 1
S_J = 50                # interval counter j
S_SOFF = 51             # byte offset of the K tile this interval copies
S_M0B = 52              # LDS address of this wave's share of a tile
S_TM1 = 53              # T - 1
S_J2 = 54               # j + 2, j + 3
S_J3 = 55
S_VSOFF = 56            # byte offset of the V tile this interval copies
S_TMP = 57
S_RET = 58              # s[58:59]: return address of the reference-move path
S_NTV = 60              # whole tiles of the head (N / 64): the copies may fetch tiles below it
SGPR_CLOBBER = [S_J, S_SOFF, S_TM1, S_J2, S_J3, S_VSOFF, S_TMP, S_RET, S_RET + 1]

MFMA = "v_mfma_f32_32x32x64_f8f6f4"


def vr(lo, n=1):
    return f"v{lo}" if n == 1 else f"v[{lo}:{lo + n - 1}]"


def q_frag(s):
    return vr(R_Q + 8 * s, 8)


def acc(db):
    return vr(R_ACC + 16 * db, 16)


def s_blk(buf, kb):
    return vr(R_S + 32 * buf + 16 * kb, 16)


def s_reg(buf, i):
    """Register i (0..31) of score buffer buf: key block i // 16, accumulator
    register i % 16."""
    return R_S + 32 * buf + i


def p_frag(buf):
    return vr(R_S + 32 * buf, 8)


class Asm:
    def __init__(self, tag):
        self.tag = tag
        self.lines = []

    def __call__(self, s):
        self.lines.append(s)

    def lbl(self, name):
        return f".L{self.tag}_{name}_%="

    def label(self, name):
        self.lines.append(self.lbl(name) + ":")


class Reads:
    """LDS operand reads of one MFMA stream, in issue order, with exact
    lgkmcnt waits (LDS reads complete in order; at most 15 may be counted)."""

    def __init__(self, a, kstart=0, vstart=0):
        self.a = a
        self.ops = []        # one entry per ds_read, the key of the operand it fills
        self.kbuf = kstart   # next K / V buffer in the rings
        self.vbuf = vstart
        self.where = {}      # operand key -> first buffer register

    def k(self, key, s, kb, stage):
        b = R_KBUF + 8 * (self.kbuf % NKB)
        self.kbuf += 1
        off = stage * TSZ + kb * 32 * D
        for e in range(2):
            self.a(f"ds_read_b128 {vr(b + 4 * e, 4)}, {vr(R_KA + 2 * s + e)} offset:{off}")
        self.ops += [key, key]
        self.where[key] = b

    def v(self, key, db, stage):
        b = R_VBUF + 8 * (self.vbuf % NVB)
        self.vbuf += 1
        for x in range(4):
            off = VOFF + stage * TSZ + 16 * x * D
            self.a(f"ds_read_b64_tr_b8 {vr(b + 2 * x, 2)}, {vr(R_VA + db)} offset:{off}")
        self.ops += [key] * 4
        self.where[key] = b

    def wait(self, key):
        last = max(i for i, k in enumerate(self.ops) if k == key)
        self.a(f"s_waitcnt lgkmcnt({min(len(self.ops) - 1 - last, 15)})")
        return vr(self.where[key], 8)


def score_order():
    """Score MFMA i: d step i // 2, 32-key block i % 2 (two accumulation chains)."""
    return [(i // 2, i % 2) for i in range(2 * KS)]


def score_phase(a, rd, stage, nbuf, first_keys_issued, after=None):
    """The 4 score MFMAs of the tile in `stage` into buffer nbuf, K operands
    LK ahead; after(i) runs after MFMA i."""
    order = score_order()
    if not first_keys_issued:
        for i in range(LK):
            s, kb = order[i]
            rd.k(("K", i), s, kb, stage)
    for i, (s, kb) in enumerate(order):
        opnd = rd.wait(("K", i))
        src_c = "0" if s == 0 else s_blk(nbuf, kb)
        a(f"{MFMA} {s_blk(nbuf, kb)}, {opnd}, {q_frag(s)}, {src_c}")
        if i + LK < len(order):
            s2, kb2 = order[i + LK]
            rd.k(("K", i + LK), s2, kb2, stage)
        if after is not None:
            after(i)


def pv_phase(a, rd, vstage, pbuf, first_issued, tail_reads=None, after=None):
    """The 4 P.V MFMAs (d blocks 0-3) with V^T of `vstage` and P of buffer
    pbuf; the first `first_issued` operands were read earlier; tail_reads(m)
    issues the m-th read of the next phase once the V reads are done."""
    for i in range(first_issued, LV):
        rd.v(("V", i), i, vstage)
    for db in range(DB):
        opnd = rd.wait(("V", db))
        a(f"{MFMA} {acc(db)}, {opnd}, {p_frag(pbuf)}, {acc(db)}")
        if db + LV < DB:
            rd.v(("V", db + LV), db + LV, vstage)
        elif tail_reads is not None:
            tail_reads(db + LV - DB)
        if after is not None:
            after(db)


def v_prefetch(rd, vstage):
    """The first LV V^T operands of a P.V phase."""
    for i in range(LV):
        rd.v(("V", i), i, vstage)


def seeded_reads(a):
    """Reads state at the start of an interval: the first LV V^T operands of
    its P.V phase were read before the barrier (v_prefetch from buffer 0)."""
    rd = Reads(a)
    for i in range(LV):
        rd.ops += [("V", i)] * 4
        rd.where[("V", i)] = R_VBUF + 8 * (i % NVB)
    rd.vbuf = LV
    return rd


# ---- softmax of one tile ----------------------------------------------------
def lane_max(buf):
    """v{R_T0} = c * (max of the lane's 32 raw scores of buffer buf), as two
    v_max3 chains (one per key block) issued alternately."""
    ins = []
    chains = []
    for kb, dst in ((0, R_T0), (1, R_T1)):
        r = [s_reg(buf, 16 * kb + i) for i in range(16)]
        c = [f"v_max3_f32 v{dst}, v{r[0]}, v{r[1]}, v{r[2]}"]
        for i in range(3, 15, 2):
            c.append(f"v_max3_f32 v{dst}, v{dst}, v{r[i]}, v{r[i + 1]}")
        c.append(f"v_max_f32 v{dst}, v{dst}, v{r[15]}")
        chains.append(c)
    for x, y in zip(*chains):
        ins += [x, y]
    ins.append(f"v_max_f32 v{R_T0}, v{R_T0}, v{R_T1}")
    ins.append(f"v_mul_f32 v{R_T0}, s{S_C}, v{R_T0}")
    return ins


def check(a):
    """Some lane's max beyond m + 2.75: the out-of-line reference update,
    which returns to the instruction after the branch."""
    return [f"v_cmp_lt_f32 vcc, v{R_MT}, v{R_T0}",
            f"s_getpc_b64 s[{S_RET}:{S_RET + 1}]",
            f"s_cbranch_vccnz {a.lbl('move')}"]


def group_regs(buf, g):
    return [s_reg(buf, 4 * g + t) for t in range(4)]


def grp_fma(buf, g):
    return [f"v_fma_f32 v{e}, v{e}, s{S_C}, -v{R_REF}" for e in group_regs(buf, g)]


def grp_exp(buf, g):
    return [f"v_exp_f32 v{e}, v{e}" for e in group_regs(buf, g)]


def grp_sum_pack(buf, g):
    """Row sums in the order t = 0..3 alternating between the two partial
    sums, then the four values as E4M3 bytes (round to nearest even) into
    register g of the buffer: byte t of P register g is register 4g + t."""
    e = group_regs(buf, g)
    dst = s_reg(buf, g)
    return [f"v_add_f32 v{R_RS0}, v{R_RS0}, v{e[0]}", f"v_add_f32 v{R_RS1}, v{R_RS1}, v{e[1]}",
            f"v_add_f32 v{R_RS0}, v{R_RS0}, v{e[2]}", f"v_add_f32 v{R_RS1}, v{R_RS1}, v{e[3]}",
            f"v_cvt_pk_fp8_f32 v{dst}, v{e[0]}, v{e[1]}",
            f"v_cvt_pk_fp8_f32 v{dst}, v{e[2]}, v{e[3]} op_sel:[0,0,1]"]


class Softmax:
    """The softmax of the tile in score buffer buf as chunks of a few
    instructions, spread evenly over the MFMA slots of an interval: the lane
    max and the reference check, then rounds r = 0..9 of [sum and pack of
    group r-2] and [2^x of group r-1, x = s c - ref of group r]."""

    def __init__(self, a, buf):
        self.a = a
        chunks = [[f"v_mov_b32 v{R_RS0}, 0", f"v_mov_b32 v{R_RS1}, 0"]]
        mx = lane_max(buf)
        chunks += [mx[i:i + 4] for i in range(0, len(mx), 4)]
        chunks.append(check(a))
        for r in range(8 + 2):
            if 0 <= r - 2 < 8:
                chunks.append(grp_sum_pack(buf, r - 2))
            ins = []
            if 0 <= r - 1 < 8:
                ins += grp_exp(buf, r - 1)
            if r < 8:
                ins += grp_fma(buf, r)
            chunks.append(ins)
        self.chunks = chunks
        self.done = 0

    def emit_upto(self, num, den):
        want = (len(self.chunks) * num) // den
        while self.done < want:
            for ins in self.chunks[self.done]:
                self.a(ins)
            self.done += 1

    def finish(self):
        self.emit_upto(1, 1)


def end_softmax(a, k):
    """l = alpha l + row sum; acc *= alpha when some row of the wave moved
    (the P.V MFMAs of the previous tile are issued by now, those of this tile
    come next)."""
    a(f"v_add_f32 v{R_T0}, v{R_RS0}, v{R_RS1}")
    a(f"v_fma_f32 v{R_L}, v{R_L}, v{R_ALPHA}, v{R_T0}")
    a(f"v_cmp_neq_f32 vcc, 1.0, v{R_ALPHA}")
    a(f"s_cbranch_vccz {a.lbl(f'nors{k}')}")
    for r in range(R_ACC, R_ACC + 16 * DB):
        a(f"v_mul_f32 v{r}, v{r}, v{R_ALPHA}")
    a(f"v_mov_b32 v{R_ALPHA}, 1.0")
    a.label(f"nors{k}")


def move_path(a):
    """Out of line: some row's tile max exceeds its reference by more than
    2.75.  Row max (the two lane halves hold a row's keys), m_new = the row
    max where it exceeds m + 2.75, else m; alpha = 2^(m - m_new) (exactly 1
    where m stays); m + 2.75 and m - 6 follow."""
    a.label("move")
    a(f"v_mov_b32 v{R_T1}, v{R_T0}")
    a("s_nop 1")
    a(f"v_permlane32_swap_b32 v{R_T0}, v{R_T1}")
    a(f"v_max_f32 v{R_T0}, v{R_T0}, v{R_T1}")
    a(f"v_cmp_lt_f32 vcc, v{R_MT}, v{R_T0}")
    a(f"v_cndmask_b32 v{R_T1}, v{R_M}, v{R_T0}, vcc")
    a(f"v_sub_f32 v{R_T0}, v{R_M}, v{R_T1}")
    a(f"v_exp_f32 v{R_ALPHA}, v{R_T0}")
    a(f"v_mov_b32 v{R_M}, v{R_T1}")
    a(f"v_add_f32 v{R_MT}, 0x{LAZY:08x}, v{R_T1}")
    a(f"v_add_f32 v{R_REF}, 0x{MSHIFT:08x}, v{R_T1}")
    a(f"s_add_u32 s{S_RET}, s{S_RET}, 4")       # past the s_cbranch_vccnz (4 bytes)
    a(f"s_addc_u32 s{S_RET + 1}, s{S_RET + 1}, 0")
    a(f"s_setpc_b64 s[{S_RET}:{S_RET + 1}]")


# ---- copies and loop control --------------------------------------------------
def copy_setup(a):
    """Tile offsets of this interval's copies: K of tile j+3, V of tile j+2.
    A tile t that is not a whole tile of the head (t >= N / 64) is replaced
    by tile 0: the tile offset goes in soffset, which the buffer's range
    check does not cover, so every copy stays inside the head.  Tiles past
    the item's last full one land in stages no wave of the loop reads: the
    code after the loop uses them (diagonal tiles) or ignores them."""
    a(f"s_add_u32 s{S_J3}, s{S_J}, 3")
    a(f"s_add_u32 s{S_J2}, s{S_J}, 2")
    for jr, off in ((S_J3, S_SOFF), (S_J2, S_VSOFF)):
        a(f"s_cmp_lt_u32 s{jr}, s{S_NTV}")
        a(f"s_cselect_b32 s{S_TMP}, s{jr}, 0")
        a(f"s_lshl_b32 s{off}, s{S_TMP}, 13")


def dma_parts(k):
    """The copies of interval j (j % 4 == k): K of tile j+3 into K stage
    (k+3) % 4 (last read by the scores of tile j-1, in interval j-2) and V
    of tile j+2 into V stage (k+2) % 4 (last read by P.V(j-2), in interval
    j-1), one instruction each (the wave's 1 KiB block)."""
    parts = []
    for desc, off, base in ((S_KDESC, S_SOFF, ((k + 3) % 4) * TSZ), (S_VDESC, S_VSOFF, VOFF + ((k + 2) % 4) * TSZ)):
        parts.append([f"s_add_u32 m0, s{S_M0B}, {base}", "s_nop 0",
                      f"buffer_load_dwordx4 v{R_DSRC}, s[{desc}:{desc + 3}], s{off} offen lds"])
    return parts


def end_interval(a):
    """Interval j+1 reads K(j+2) and V(j+1) (its last instructions prefetch
    V^T operands of P.V(j+1)), both copied in interval j-1: wait for this
    wave's copies issued before interval j (every interval issues two), then
    the barrier publishes every wave's."""
    a("s_waitcnt vmcnt(2)")
    a("s_barrier")


def loop_control(a, k, fall_through):
    a(f"s_add_u32 s{S_J}, s{S_J}, 1")
    a(f"s_cmp_eq_u32 s{S_J}, s{S_TM1}")
    a(f"s_cbranch_scc1 {a.lbl(f'last{(k + 1) % 4}')}")
    if not fall_through:
        a(f"s_branch {a.lbl(f'body{(k + 1) % 4}')}")


def body(a, k, last, first):
    """Interval j (j % 4 == k): P.V of tile j-1 (unless first), the scores of
    tile j+1 (unless last), and between those 8 MFMAs the softmax of tile j,
    then the first V^T operands of P.V(j)."""
    name = f"{'first' if first else ''}{'last' if last else 'body'}{k}"
    a.label(name)
    cur, nxt = k % 2, (k + 1) % 2
    rd = Reads(a) if first else seeded_reads(a)
    copy_setup(a)
    parts = dma_parts(k)
    sm = Softmax(a, cur)
    nslots = (0 if first else DB) + (0 if last else 2 * KS)
    slot = [0]
    copy_at = {}
    for n in range(len(parts)):
        copy_at.setdefault(min(nslots - 1, (nslots * n) // len(parts) + 1), []).append(n)

    def after_mfma(_i):
        for n in copy_at.get(slot[0], []):
            for ins in parts[n]:
                a(ins)
        slot[0] += 1
        sm.emit_upto(slot[0], nslots)

    if not first:
        tail = None
        if not last:
            def tail(m):
                if m < LK:
                    s, kb = score_order()[m]
                    rd.k(("K", m), s, kb, (k + 1) % 4)
        pv_phase(a, rd, (k + 3) % 4, nxt, LV, tail, after_mfma)
    if not last:
        score_phase(a, rd, (k + 1) % 4, nxt, not first, after_mfma)
    if nslots == 0:
        for part in parts:
            for ins in part:
                a(ins)
    sm.finish()
    end_softmax(a, name)
    # P.V(j) opens the next interval (or follows the last one)
    v_prefetch(Reads(a), k)
    end_interval(a)
    if last:
        a(f"s_branch {a.lbl(f'exit{k}')}")
    else:
        loop_control(a, k, fall_through=not first and k < 3)


def exit_pv(a, k):
    """After the last interval: P.V of the last tile (its first V^T operands
    were read before the last barrier)."""
    a.label(f"exit{k}")
    pv_phase(a, seeded_reads(a), k, k % 2, LV)
    a(f"s_branch {a.lbl('done')}")


def prologue(a):
    """K of tiles 0-2 and V of tiles 0-1 are in stages 0-2 (copied, waited
    for and published by the C++ side).  S(0) into buffer 0; tile 0 always
    moves the reference (m starts at -inf): m = the row max of tile 0 times
    c; l = 0, alpha = 1."""
    a(f"s_mov_b32 s{S_J}, 0")
    a(f"s_add_u32 s{S_TM1}, s{S_T}, -1")
    score_phase(a, Reads(a), 0, 0, False)
    a(f"v_mov_b32 v{R_L}, 0")
    a(f"v_mov_b32 v{R_ALPHA}, 1.0")
    a("s_nop 7")
    a("s_nop 7")
    a("s_nop 2")     # MFMA result -> VALU read
    for ins in lane_max(0):
        a(ins)
    a(f"v_mov_b32 v{R_T1}, v{R_T0}")
    a("s_nop 1")
    a(f"v_permlane32_swap_b32 v{R_T0}, v{R_T1}")
    a(f"v_max_f32 v{R_M}, v{R_T0}, v{R_T1}")
    a(f"v_add_f32 v{R_MT}, 0x{LAZY:08x}, v{R_M}")
    a(f"v_add_f32 v{R_REF}, 0x{MSHIFT:08x}, v{R_M}")


def block():
    a = Asm("fa2f8")
    prologue(a)
    a(f"s_cmp_eq_u32 s{S_TM1}, 0")
    a(f"s_cbranch_scc1 {a.lbl('firstlast0')}")
    body(a, 0, False, True)
    for k in range(4):
        body(a, k, False, False)
    body(a, 0, True, True)
    for k in range(4):
        body(a, k, True, False)
    for k in range(4):
        exit_pv(a, k)
    move_path(a)
    a(f"{a.lbl('done')}:")
    # the copies of the last intervals land before the code after the block
    # reads or refills their stages; MFMA results -> the C++ code that reads acc
    a("s_waitcnt vmcnt(0) lgkmcnt(0)")
    a("s_nop 7")
    a("s_nop 7")
    a("s_nop 7")
    return a.lines


def clobbers():
    regs = [f'"v{r}"' for r in range(R_S, R_S + 64)]
    regs += [f'"v{r}"' for r in range(R_ALPHA, R_END)]
    regs += [f'"s{s}"' for s in SGPR_CLOBBER]
    return ", ".join(regs + ['"m0"', '"vcc"', '"scc"', '"memory"'])


def generate() -> str:
    out = ["// Generated by gen_fwd_fp8_sched.py; do not edit.", ""]
    text = "\\n\\t".join(block())
    out.append(f'#define FA2_FP8_SCHED "{text}"')
    out.append(f"#define FA2_FP8_SCHED_CLOBBERS {clobbers()}")
    out.append(f"#define FA2_FP8_SCHED_REG_END {R_END}")
    for name, val in (("R_Q", R_Q), ("R_ACC", R_ACC), ("R_KA", R_KA), ("R_VA", R_VA), ("R_DSRC", R_DSRC),
                      ("R_M", R_M), ("R_L", R_L), ("S_KDESC", S_KDESC), ("S_VDESC", S_VDESC), ("S_C", S_C),
                      ("S_T", S_T), ("S_M0B", S_M0B), ("S_NTV", S_NTV)):
        out.append(f"#define FA2_FP8_SCHED_{name} {val}")
    out.append("")
    return "\n".join(out)


def main():
    with open(OUTPUT, "w") as f:
        f.write(generate())


if __name__ == "__main__":
    main()
