#!/usr/bin/env python3
"""Generate fa2_fwd_sched.inc: the main loop of the scheduled forward kernel
(fa2_fwd_sched.hpp) as gfx950 assembly.

    python exact_attention_63_amd/csrc/gen_fwd_sched.py

What the loop computes (one workgroup, d = 128, 64-key tiles, 8 waves of 32
query rows; "FlashAttention v2 better parallelism + work partitioning"
diagram, concept pseudo-code panel): for every full key tile j, with the
scores S(j) = K(j) Q^T of the wave's 32 queries, the online softmax update
P(j) = 2^(S(j) c - m), l += rowsum(P(j)), then acc += V(j)^T P(j)^T.  The
1/l normalisation and the stores stay in the C++ epilogue.

Schedule.  Tile j lives in ring stage j % 4 (K and V, 16 KiB each, rows
XOR-swizzled), copied from HBM with buffer_load ... lds two intervals before
it is read (K of tiles 0-2 and V of tiles 0-1 by the C++ side, before the Q
loads).  One barrier per tile
("interval" j).  Every wave runs the same program; in interval j it issues the
16 P.V MFMAs of tile j-1 and the 16 score MFMAs of tile j+1, and between those
32 MFMAs the softmax of tile j, cut into staggered rounds (x = s c - m of one
pair, 2^x of the pair before, row sums and packing of the pair before that),
so that no VALU result is used before the next MFMA: the matrix pipe always
has MFMAs ready while the softmax runs, which is the overlap the
"FlashAttention v4 Blackwell pipeline co-design" diagram's pseudo-code panel
asks for ("while MMA runs: schedule softmax for previous S"), done here by
software pipelining inside each wave (and two waves per SIMD) instead of
asynchronous tensor-core instructions.  P of tile j waits one interval in the
registers of its scores; the scores of tile j+1 go to the other buffer.

Softmax without a per-tile max.  p = 2^(s c - m) uses the row's reference m
as it stands (m starts as the exact max of tile 0).  Each lane sums its 32 p
in fp32; if some lane's sum exceeds 2^13 (so some p may exceed 2^13 or be
inf), the wave takes a rare out-of-line path that recomputes S(j) from K(j),
still in LDS, and does the exact update with m_new = max(m, max S c) and the
rescale factor alpha = 2^(m - m_new).  Otherwise alpha = 1 and the result is
the same exact value (O = acc / l and LSE = m + log2 l share the reference):
the conditional rescale of the v4 diagram in an exact form.

Registers are fixed (the C++ side binds its values to them, see
fa2_fwd_sched.hpp), so the output is plain assembly with no operand
references; labels carry %= so that every instance is unique.
"""

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUTPUT = os.path.join(HERE, "fa2_fwd_sched.inc")

# ---- problem geometry ------------------------------------------------------
D = 128                 # head dimension
KROW = 2 * D            # bytes per K / V row
BC = 64                 # keys per tile
TSZ = BC * KROW         # bytes of one K (or V) tile: 16 KiB
NS = 4                  # ring stages
VOFF = NS * TSZ         # V stages follow the K stages; folded into the V base registers
DK = D // 16            # 16-wide d steps of the score product (8)
DB = D // 32            # 32-row blocks of O^T (4)
THRESH = 0x46000000     # 8192.0f: lane row-sum bound of the lazy reference
LK = 4                  # K fragment reads kept ahead of the score MFMAs
LV = 4                  # V^T fragments kept ahead of the P.V MFMAs (two reads each)
NKB = LK + 2            # K operand buffers (a buffer is refilled two MFMAs after its use)
NVB = LV + 2            # V^T operand buffers
# Where each operand stream starts its buffer ring.  A phase of 16 operands
# started at buffer b leaves its last two in buffers b + 2, b + 3 (mod 6); a
# stream that follows with no MFMA in between must not refill those first:
#   * K: score phases start at 0, the prologue's at 2 (so a score phase or the
#     exact update may follow it directly), the exact update's at 0 with two
#     reads ahead (it may follow a score phase started at 0 or 2);
#   * V: P.V phases start at 0, except the ones of the last interval, whose
#     operands are read right after the previous P.V phase: they start at 4.
K_START_PROLOGUE = 2
LK_EXACT = 2
V_START_LAST = 4

# ---- register map (VGPRs) ---------------------------------------------------
R_Q = 0                 # v[0:31]    Q fragments, B operand of S^T = K Q^T (8 x 4)
R_ACC = 32              # v[32:95]   O^T accumulators (4 x 16)
R_S = 96                # v[96:159]  two score buffers (2 x 2 x 16); P is packed in place
R_KA = 160              # v[160:167] K fragment LDS addresses, one per d step
R_VA = 168              # v[168:175] V^T fragment LDS addresses (d block, low/high 8 keys)
R_DSRC = 176            # v[176:177] global byte offsets of this lane's two copy chunks
R_M, R_L, R_ALPHA = 178, 179, 180
R_RS0, R_RS1, R_T0, R_T1 = 181, 182, 183, 184
R_QOFF = 185            # this lane's byte offset inside a Q block: (lane % 32) * 256 + 16 (lane / 32)
R_KBUF = 186            # K operand buffers
R_VBUF = R_KBUF + 4 * NKB
R_END = R_VBUF + 4 * NVB   # first VGPR the loop does not touch

# ---- register map (SGPRs) ---------------------------------------------------
S_KDESC, S_VDESC = 40, 44   # buffer descriptors of this head's K and V
S_C = 48                # c = |scale| * log2(e)
S_T = 49                # number of full tiles T >= 1
S_J = 50                # interval counter j
S_SOFF = 51             # byte offset (in its head) of the K tile this interval copies
S_M0B = 52              # LDS address of this wave's 2 KiB share of a tile
S_TM1 = 53              # T - 1
S_J2 = 54               # j + 2
S_J3 = 55               # j + 3
S_RET = 54              # s[54:55]: return address of the exact-update path (j + 2, j + 3
                        # are not needed after it: end_interval recomputes j + 3)
# The next work item of a persistent workgroup (when s{S_HASN} != 0): its K and
# V descriptors (they replace the current ones once the current item's copies
# are done), its Q descriptor and the byte offset of its query block.
S_NKD, S_NVD, S_NQD = 56, 60, 64
S_NQOFF = 68
S_HASN = 69
S_TMP = 70
S_VSOFF = 71            # byte offset of the V tile this interval copies
S_NSUB = 72             # past the last full tile T-1 a copy fetches tile t - s72 (T: the next item's, 0: this head's)
S_NTV = 73              # tiles below s73 may be fetched (whole tiles of the head the copies read)
SGPR_CLOBBER = [S_J, S_SOFF, S_TM1, S_J2, S_J3, S_TMP, S_VSOFF]


def vr(lo, n=1):
    return f"v{lo}" if n == 1 else f"v[{lo}:{lo + n - 1}]"


def q_frag(dk):
    return vr(R_Q + 4 * dk, 4)


def acc(db):
    return vr(R_ACC + 16 * db, 16)


def s_blk(buf, kb):
    return vr(R_S + 32 * buf + 16 * kb, 16)


def s_elem(buf, kb, r):
    return R_S + 32 * buf + 16 * kb + r


def p_frag(buf, kb, st):
    """Packed P of 16-key step st of 32-key block kb: the first four registers
    of the step's eight score registers."""
    return vr(R_S + 32 * buf + 16 * kb + 8 * st, 4)


class Asm:
    def __init__(self, dtype, tag):
        assert dtype in ("bf16", "f16")
        self.dt = dtype
        self.tag = tag
        self.lines = []

    def __call__(self, s):
        self.lines.append(s)

    def lbl(self, name):
        return f".L{self.tag}_{name}_%="

    def label(self, name):
        self.lines.append(self.lbl(name) + ":")

    @property
    def mfma(self):
        return "v_mfma_f32_32x32x16_" + self.dt

    @property
    def cvt(self):
        return "v_cvt_pk_bf16_f32" if self.dt == "bf16" else "v_cvt_pk_f16_f32"


class Reads:
    """LDS operand reads of one MFMA stream, in issue order, with exact
    lgkmcnt waits (LDS reads complete in order; at most 15 may be counted)."""

    def __init__(self, a, kstart=0, vstart=0):
        self.a = a
        self.ops = []        # one entry per ds_read, the key of the operand it fills
        self.kbuf = kstart   # next K / V buffer in the rings
        self.vbuf = vstart
        self.where = {}      # operand key -> buffer register

    def k(self, key, dk, kb, stage):
        b = R_KBUF + 4 * (self.kbuf % NKB)
        self.kbuf += 1
        self.a(f"ds_read_b128 {vr(b, 4)}, {vr(R_KA + dk)} offset:{stage * TSZ + kb * 32 * KROW}")
        self.ops.append(key)
        self.where[key] = b

    def v(self, key, db, kb, st, stage):
        b = R_VBUF + 4 * (self.vbuf % NVB)
        self.vbuf += 1
        off = stage * TSZ + (32 * kb + 16 * st) * KROW
        self.a(f"ds_read_b64_tr_b16 {vr(b, 2)}, {vr(R_VA + 2 * db)} offset:{off}")
        self.a(f"ds_read_b64_tr_b16 {vr(b + 2, 2)}, {vr(R_VA + 2 * db + 1)} offset:{off}")
        self.ops += [key, key]
        self.where[key] = b

    def wait(self, key):
        last = max(i for i, k in enumerate(self.ops) if k == key)
        self.a(f"s_waitcnt lgkmcnt({min(len(self.ops) - 1 - last, 15)})")
        return vr(self.where[key], 4)


def score_order():
    """Score MFMA i: d step i // 2, 32-key block i % 2 (two accumulation chains)."""
    return [(i // 2, i % 2) for i in range(2 * DK)]


def pv_order():
    """P.V MFMA i: 16-key step i // 4 (block, step), d block i % 4."""
    return [((i // 4) // 2, (i // 4) % 2, i % 4) for i in range(4 * DB)]


def softmax_pair(a, buf, q):
    """Elements 2t, 2t+1 of step st of block kb (q = 8 kb + 4 st + t): x = s c - m,
    p = 2^x in place, row sums, then the pair packed into register 8 st + t of
    the block (already consumed), which leaves P of each step in its first four
    registers."""
    for ins in pair_fma(buf, q) + pair_exp(buf, q) + pair_sum(a, buf, q):
        a(ins)


def softmax_start(a):
    a(f"v_mov_b32 v{R_RS0}, 0")
    a(f"v_mov_b32 v{R_RS1}, 0")


def softmax_check(a, k):
    """Lane row sum; the exact-update path when any lane's sum exceeds the
    bound (it rescales acc and l itself and returns to the instruction after
    the branch); then l += the row sum."""
    a(f"v_add_f32 v{R_T0}, v{R_RS0}, v{R_RS1}")
    a(f"v_cmp_lt_f32 vcc, 0x{THRESH:08x}, v{R_T0}")
    a(f"s_getpc_b64 s[{S_RET}:{S_RET + 1}]")
    a(f"s_cbranch_vccnz {a.lbl(f'exact{k}')}")
    a(f"v_add_f32 v{R_L}, v{R_L}, v{R_T0}")


def row_max(a, buf):
    """v{R_T0} = max over the row of the raw scores of buffer buf (both lane
    halves), two chains of v_max3."""
    for kb, dst in ((0, R_T0), (1, R_T1)):
        r = [s_elem(buf, kb, i) for i in range(16)]
        a(f"v_max3_f32 v{dst}, v{r[0]}, v{r[1]}, v{r[2]}")
        for i in range(3, 15, 2):
            a(f"v_max3_f32 v{dst}, v{dst}, v{r[i]}, v{r[i + 1]}")
        a(f"v_max_f32 v{dst}, v{dst}, v{r[15]}")
    a(f"v_max_f32 v{R_T0}, v{R_T0}, v{R_T1}")
    a(f"v_mov_b32 v{R_T1}, v{R_T0}")
    a("s_nop 1")
    # lanes 0-31 and 32-63 hold the two halves of a row's keys
    a(f"v_permlane32_swap_b32 v{R_T0}, v{R_T1}")
    a(f"v_max_f32 v{R_T0}, v{R_T0}, v{R_T1}")


def rescale(a, name):
    """acc *= alpha when some row of the wave moved its reference."""
    a(f"v_cmp_neq_f32 vcc, 1.0, v{R_ALPHA}")
    a(f"s_cbranch_vccz {a.lbl(name)}")
    for r in range(R_ACC, R_ACC + 16 * DB):
        a(f"v_mul_f32 v{r}, v{r}, v{R_ALPHA}")
    a(f"{a.lbl(name)}:")
    a("s_nop 1")     # VALU write -> MFMA source read


def copy_setup(a):
    """Descriptors and tile offsets of this interval's copies, without
    branches.  Interval j copies K of tile j+3 and V of tile j+2.  Past the
    item's last full tile T-1 the same slots copy either
      * the next item's tiles 0-2 (K) and 0-1 (V) (persistent workgroups,
        s{S_NSUB} = T): at j+3 == T (j+2 == T) the K (V) descriptor becomes
        the next item's, and tile t >= T is the next item's tile t - T
        (T % 4 == 0, so it lands in the ring stage of its index); or
      * tile t of the same head (one item per workgroup, s{S_NSUB} = 0, the
        next descriptors being the current ones): the masked tiles after the
        loop (a causal workgroup's diagonal) find K(T..T+2) and V(T..T+1) in
        their ring stages.
    A tile index not below s{S_NTV} (not a whole tile of the head) becomes
    tile 0, copied into a stage no wave reads: the tile offset goes in
    soffset, which the buffer's range check does not cover, so every copy
    stays inside the head.  Every interval issues four copies.
    s{S_J2} = j + 2, s{S_J3} = j + 3."""
    for jr, cur, nxt, off in ((S_J3, S_KDESC, S_NKD, S_SOFF), (S_J2, S_VDESC, S_NVD, S_VSOFF)):
        a(f"s_cmp_eq_u32 s{jr}, s{S_T}")
        a(f"s_cselect_b64 s[{cur}:{cur + 1}], s[{nxt}:{nxt + 1}], s[{cur}:{cur + 1}]")
        a(f"s_cselect_b64 s[{cur + 2}:{cur + 3}], s[{nxt + 2}:{nxt + 3}], s[{cur + 2}:{cur + 3}]")
        a(f"s_cmp_lt_u32 s{jr}, s{S_T}")
        a(f"s_cselect_b32 s{S_TMP}, 0, s{S_NSUB}")
        a(f"s_sub_u32 s{S_TMP}, s{jr}, s{S_TMP}")
        a(f"s_cmp_lt_u32 s{S_TMP}, s{S_NTV}")
        a(f"s_cselect_b32 s{S_TMP}, s{S_TMP}, 0")
        a(f"s_lshl_b32 s{off}, s{S_TMP}, 14")


def dma_parts(k):
    """The copies of interval j (j % 4 == k): K of tile j+3 into K stage
    (k+3) % 4 (last read by the scores of tile j-1 in interval j-2, or by
    the exact update of tile j-1 in interval j-1) and V of tile j+2 into V
    stage (k+2) % 4 (last read by P.V(j-2) in interval j-1), as four
    one-instruction pieces (this wave's two 1 KiB blocks of each).  K(j+3) is
    first read in interval j+2, V(j+2) at the end of interval j+2."""
    parts = []
    for desc, off, base in ((S_KDESC, S_SOFF, ((k + 3) % 4) * TSZ), (S_VDESC, S_VSOFF, VOFF + ((k + 2) % 4) * TSZ)):
        for kk in range(2):
            parts.append([f"s_add_u32 m0, s{S_M0B}, {base + 1024 * kk}", "s_nop 0",
                          f"buffer_load_dwordx4 {vr(R_DSRC + kk)}, s[{desc}:{desc + 3}], s{off} offen lds"])
    return parts


def load_next_q(a, name):
    """The next item's Q fragments into v[0:31] (free: the last interval has
    no score MFMA and no exact update)."""
    lbl = a.lbl(f"{name}nq")
    a(f"s_cmp_eq_u32 s{S_HASN}, 0")
    a(f"s_cbranch_scc1 {lbl}")
    for dk in range(DK):
        a(f"buffer_load_dwordx4 {q_frag(dk)}, v{R_QOFF}, s[{S_NQD}:{S_NQD + 3}], s{S_NQOFF} offen offset:{32 * dk}")
    a(f"{lbl}:")


def dma_half(a, desc, base):
    """This wave's two 1 KiB blocks of one K or V tile (tile offset in s{S_SOFF})."""
    for kk in range(2):
        a(f"s_add_u32 m0, s{S_M0B}, {base + 1024 * kk}")
        a("s_nop 0")
        a(f"buffer_load_dwordx4 {vr(R_DSRC + kk)}, s[{desc}:{desc + 3}], s{S_SOFF} offen lds")


def end_interval(a):
    """Interval j+1 reads K(j+2) and V(j+1) (its last instructions prefetch
    V^T operands of P.V(j+1)), both copied in interval j-1: wait for this
    wave's copies issued before interval j (every interval issues four), then
    the barrier publishes them."""
    a("s_waitcnt vmcnt(4)")
    a("s_barrier")


def loop_control(a, k, fall_through):
    """j += 1; the next interval is the last one or another full one (the
    next block in the layout when fall_through)."""
    a(f"s_add_u32 s{S_J}, s{S_J}, 1")
    a(f"s_cmp_eq_u32 s{S_J}, s{S_TM1}")
    a(f"s_cbranch_scc1 {a.lbl(f'last{(k + 1) % 4}')}")
    if not fall_through:
        a(f"s_branch {a.lbl(f'body{(k + 1) % 4}')}")


def score_phase(a, rd, stage, nbuf, first_keys_issued, after=None, look=LK):
    """The 16 score MFMAs of the tile in `stage` into buffer nbuf, K reads
    `look` ahead; after(i) runs after MFMA i."""
    order = score_order()
    if not first_keys_issued:
        for i in range(look):
            dk, kb = order[i]
            rd.k(("K", i), dk, kb, stage)
    for i, (dk, kb) in enumerate(order):
        opnd = rd.wait(("K", i))
        src_c = "0" if dk == 0 else s_blk(nbuf, kb)
        a(f"{a.mfma} {s_blk(nbuf, kb)}, {opnd}, {q_frag(dk)}, {src_c}")
        if i + look < len(order):
            dk2, kb2 = order[i + look]
            rd.k(("K", i + look), dk2, kb2, stage)
        if after is not None:
            after(i)


def pv_phase(a, rd, vstage, pbuf, first_issued, tail_reads=None, after=None):
    """The 16 P.V MFMAs with V^T of `vstage` and P of buffer pbuf; the first
    `first_issued` operands were read earlier; tail_reads(i) issues reads for
    the next phase once the V reads are done; after(i) runs after MFMA i."""
    order = pv_order()
    for i in range(first_issued, min(LV, len(order))):
        kb, st, db = order[i]
        rd.v(("V", i), db, kb, st, vstage)
    for i, (kb, st, db) in enumerate(order):
        opnd = rd.wait(("V", i))
        a(f"{a.mfma} {acc(db)}, {opnd}, {p_frag(pbuf, kb, st)}, {acc(db)}")
        if i + LV < len(order):
            kb2, st2, db2 = order[i + LV]
            rd.v(("V", i + LV), db2, kb2, st2, vstage)
        elif tail_reads is not None:
            tail_reads(i + LV - len(order))
        if after is not None:
            after(i)


def v_prefetch(rd, vstage):
    """The first LV V^T operands of a P.V phase."""
    order = pv_order()
    for i in range(LV):
        kb, st, db = order[i]
        rd.v(("V", i), db, kb, st, vstage)


class Rounds:
    """The softmax of one tile as staggered chunks: step r holds the row sums
    and packing of pair r-2 (one chunk), then the 2^x of pair r-1 with the
    x = s c - m of pair r (another), so that every result is used a chunk
    (at least one MFMA) after it is made.  The chunks (3 or 4 VALU
    instructions each) are spread evenly over the MFMA slots of an interval."""

    def __init__(self, a, buf, exact_max=False):
        self.a = a
        self.rounds = []
        if exact_max:
            # the last tile of an item: m_new = max(m, max S c), alpha, first
            self.rounds += exact_reference(a, buf)
        for r in range(16 + 2):
            if 0 <= r - 2 < 16:
                self.rounds.append(pair_sum(a, buf, r - 2))
            ins = []
            if 0 <= r - 1 < 16:
                ins += pair_exp(buf, r - 1)
            if r < 16:
                ins += pair_fma(buf, r)
            self.rounds.append(ins)
        self.done = 0

    def emit_upto(self, frac_num, frac_den):
        """Emit rounds until frac_num / frac_den of them are out."""
        want = (len(self.rounds) * frac_num) // frac_den
        while self.done < want:
            for ins in self.rounds[self.done]:
                self.a(ins)
            self.done += 1

    def finish(self):
        self.emit_upto(1, 1)


def exact_reference(a, buf):
    """Chunks that set the row's reference to max(m, max S c) of the scores in
    buffer buf and alpha = 2^(m_old - m_new)."""
    sub = Asm(a.dt, a.tag)
    row_max(sub, buf)
    sub(f"v_mul_f32 v{R_T0}, s{S_C}, v{R_T0}")
    sub(f"v_max_f32 v{R_T1}, v{R_M}, v{R_T0}")
    sub(f"v_sub_f32 v{R_T0}, v{R_M}, v{R_T1}")
    sub(f"v_mov_b32 v{R_M}, v{R_T1}")
    sub(f"v_exp_f32 v{R_ALPHA}, v{R_T0}")
    lines = sub.lines
    return [lines[i:i + 4] for i in range(0, len(lines), 4)]


def pair_regs(buf, q):
    kb, st, t = q // 8, (q % 8) // 4, q % 4
    e0 = s_elem(buf, kb, 8 * st + 2 * t)
    return e0, e0 + 1, s_elem(buf, kb, 8 * st + t)


def pair_fma(buf, q):
    e0, e1, _ = pair_regs(buf, q)
    return [f"v_fma_f32 v{e0}, v{e0}, s{S_C}, -v{R_M}", f"v_fma_f32 v{e1}, v{e1}, s{S_C}, -v{R_M}"]


def pair_exp(buf, q):
    e0, e1, _ = pair_regs(buf, q)
    return [f"v_exp_f32 v{e0}, v{e0}", f"v_exp_f32 v{e1}, v{e1}"]


def pair_sum(a, buf, q):
    e0, e1, dst = pair_regs(buf, q)
    return [f"v_add_f32 v{R_RS0}, v{R_RS0}, v{e0}", f"v_add_f32 v{R_RS1}, v{R_RS1}, v{e1}",
            f"{a.cvt} v{dst}, v{e0}, v{e1}"]


def seeded_reads(a, vstart=0):
    """Reads state at the start of an interval: the first LV V^T operands of
    its P.V were read before the barrier (v_prefetch of a ring started at
    vstart)."""
    rd = Reads(a, vstart=vstart)
    for i in range(LV):
        rd.ops += [("V", i), ("V", i)]
        rd.where[("V", i)] = R_VBUF + 4 * ((vstart + i) % NVB)
    rd.vbuf = vstart + LV
    return rd


def body(a, k, last, first):
    """Interval j (j % 4 == k): P.V of tile j-1 (unless first), the scores of
    tile j+1 (unless last), and between those 32 MFMAs the softmax of tile j,
    then the row-sum check and the first V^T operands of P.V(j)."""
    name = f"{'first' if first else ''}{'last' if last else 'body'}{k}"
    a.label(name)
    cur, nxt = k % 2, (k + 1) % 2
    rd = Reads(a) if first else seeded_reads(a)
    a(f"s_add_u32 s{S_J2}, s{S_J}, 2")
    a(f"s_add_u32 s{S_J3}, s{S_J}, 3")
    copy_setup(a)
    # the copies go out one at a time, after MFMAs 2, 6, 10 and 14 of the
    # interval (all at once when it has no MFMA): issued back to back right
    # after the barrier by every wave, they measured 1-2 % slower
    parts = dma_parts(k)
    softmax_start(a)
    rounds = Rounds(a, cur, exact_max=last)
    nslots = (0 if first else 16) + (0 if last else 16)
    slot = [0]

    copy_at = {}
    for n in range(4):
        copy_at.setdefault(min(nslots - 1, 4 * n + 2), []).append(n)

    def after_mfma(_i):
        for n in copy_at.get(slot[0], []):
            for ins in parts[n]:
                a(ins)
        if last and slot[0] == 1:
            # Q's last reader was the final score MFMA of the interval before
            load_next_q(a, name)
        slot[0] += 1
        rounds.emit_upto(slot[0], nslots)

    if not first:
        tail = None
        if not last:
            def tail(m):
                if m < LK:
                    dk, kb = score_order()[m]
                    rd.k(("K", m), dk, kb, (k + 1) % 4)
        pv_phase(a, rd, (k + 3) % 4, nxt, LV, tail, after_mfma)
    if not last:
        score_phase(a, rd, (k + 1) % 4, nxt, not first, after_mfma)
    if nslots == 0:
        if last:
            load_next_q(a, name)     # before the copies: the end waits for all but four
        for part in parts:
            for ins in part:
                a(ins)
    rounds.finish()
    if last:
        # reference from the exact row max: p <= 1, no check, no exact update
        a(f"v_add_f32 v{R_T0}, v{R_RS0}, v{R_RS1}")
        a(f"v_fma_f32 v{R_L}, v{R_L}, v{R_ALPHA}, v{R_T0}")
    else:
        softmax_check(a, k)
    # P.V(j) opens the next interval (or follows the last one)
    v_prefetch(Reads(a, vstart=V_START_LAST if last else 0), k)
    end_interval(a)
    if last:
        a(f"s_branch {a.lbl(f'exit{k}')}")
    else:
        # bodies 0-3 are laid out in order: 0-2 fall through to the next
        loop_control(a, k, fall_through=not first and k < 3)


def exit_pv(a, k):
    """After the last interval: P.V of the last tile (its V^T operands were
    read before the last barrier)."""
    a.label(f"exit{k}")
    rescale(a, f"exit{k}r")
    pv_phase(a, seeded_reads(a, V_START_LAST), k, k % 2, LV)
    a(f"s_branch {a.lbl('done')}")


def exact_update(a, k):
    """Out-of-line exact update for the tile in stage k (score buffer k % 2):
    recompute S from K (still in LDS), m_new = max(m, max S c),
    alpha = 2^(m - m_new), p = 2^(S c - m_new), acc and l times alpha;
    returns with the lane row sum in v{R_T0}."""
    a.label(f"exact{k}")
    buf = k % 2
    score_phase(a, Reads(a), k, buf, False, look=LK_EXACT)
    a("s_nop 7")
    a("s_nop 4")     # MFMA result -> VALU read
    for chunk in exact_reference(a, buf):
        for ins in chunk:
            a(ins)
    a(f"v_mov_b32 v{R_RS0}, 0")
    a(f"v_mov_b32 v{R_RS1}, 0")
    for q in range(16):
        softmax_pair(a, buf, q)
    a(f"v_add_f32 v{R_T0}, v{R_RS0}, v{R_RS1}")
    # acc and l to the new reference (this interval's P.V MFMAs, which write
    # acc, were issued 32 MFMAs ago)
    a(f"v_mul_f32 v{R_L}, v{R_L}, v{R_ALPHA}")
    for r in range(R_ACC, R_ACC + 16 * DB):
        a(f"v_mul_f32 v{r}, v{r}, v{R_ALPHA}")
    a(f"s_add_u32 s{S_RET}, s{S_RET}, 4")       # past the s_cbranch_vccnz (4 bytes)
    a(f"s_addc_u32 s{S_RET + 1}, s{S_RET + 1}, 0")
    a(f"s_setpc_b64 s[{S_RET}:{S_RET + 1}]")


def prologue(a):
    """K of tiles 0-2 and V of tiles 0-1 are in stages 0-2: copied by the C++
    side, which waited for them and synchronised the workgroup, or by the
    previous item's last three intervals, whose barriers published all but
    K of tile 2 and V of tile 1 (published by this item's first barrier,
    before their first reads).  S(0) into buffer 0, m = exact row max of
    tile 0."""
    a(f"s_mov_b32 s{S_J}, 0")
    a(f"s_add_u32 s{S_TM1}, s{S_T}, -1")
    score_phase(a, Reads(a, kstart=K_START_PROLOGUE), 0, 0, False)
    a(f"v_mov_b32 v{R_L}, 0")
    a("s_nop 7")
    a("s_nop 3")     # MFMA result -> VALU read
    row_max(a, 0)
    a(f"v_mul_f32 v{R_M}, s{S_C}, v{R_T0}")
    a(f"v_mov_b32 v{R_ALPHA}, 1.0")


def block(dtype):
    a = Asm(dtype, "fa2s")
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
    for k in range(4):
        exact_update(a, k)
    a(f"{a.lbl('done')}:")
    # The next item's Q landed before the last barrier (the last interval
    # waited for every load but its four copies, which the next item's first
    # interval waits for).  Without a next item, wait for those copies: the
    # code after the block may reuse their stages.
    a(f"s_cmp_eq_u32 s{S_HASN}, 0")
    a(f"s_cbranch_scc0 {a.lbl('dn')}")
    a("s_waitcnt vmcnt(0)")
    a(f"{a.lbl('dn')}:")
    a("s_waitcnt lgkmcnt(0)")
    a("s_nop 7")
    a("s_nop 7")     # MFMA results -> the C++ code that reads acc
    return a.lines


def clobbers():
    regs = [f'"v{r}"' for r in range(R_S, R_S + 64)]
    regs += [f'"v{r}"' for r in range(R_M + 2, R_END) if r != R_QOFF]
    regs += [f'"s{s}"' for s in SGPR_CLOBBER]
    return ", ".join(regs + ['"m0"', '"vcc"', '"scc"', '"memory"'])


def generate() -> str:
    out = ["// Generated by gen_fwd_sched.py; do not edit.", ""]
    for dt, name in (("bf16", "BF16"), ("f16", "F16")):
        text = "\\n\\t".join(block(dt))
        out.append(f'#define FA2_SCHED_{name} "{text}"')
    out.append(f"#define FA2_SCHED_CLOBBERS {clobbers()}")
    out.append(f"#define FA2_SCHED_REG_END {R_END}")
    out.append("")
    return "\n".join(out)


def main():
    with open(OUTPUT, "w") as f:
        f.write(generate())


if __name__ == "__main__":
    main()
