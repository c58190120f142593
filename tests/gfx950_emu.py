"""A small instruction-level emulator for the generated gfx950 main loops of the
scheduled forward kernels (exact_attention_63_amd/csrc/fa2_fwd_sched.inc and
fa2_fwd_fp8_sched.inc).

Test infrastructure only: it executes the assembly text of one workgroup (all
its waves, barrier by barrier) on the CPU and checks, besides the values:

  * every register read waits for the load that fills it (lgkmcnt / vmcnt);
  * the wait states the hardware does not enforce (MFMA result -> VALU: 12
    after a 32x32x16 bf16/f16 MFMA, 20 after a 32x32x64 FP8 one, the counts
    the compiler inserts;
    VALU -> MFMA source, transcendental result -> VALU, VALU -> permlane,
    M0 -> LDS copy), counted in issue slots (s_nop n = n + 1 slots);
  * an LDS operand buffer is refilled only after two further MFMAs;
  * every wave reaches the same barriers, and no wave ends while others wait;
  * no LDS byte is read while a copy into it may be in flight, and no copy
    starts into bytes another wave may still read in the same barrier phase;
  * every LDS access stays inside the allocation, every global copy inside
    its buffer.

Only the instructions the generator emits are implemented; anything else is
an error.  Semantics (documented ISA behaviour, measured where noted in the
kernel sources):
  * v_mfma_f32_32x32x16_{bf16,f16}: lane l holds A[l%32][8(l//32)+e] and
    B[8(l//32)+e][l%32] (e = 0..7, two 16-bit elements per register, low half
    first); D register r of lane l is D[8(r//4) + 4(l//32) + r%4][l%32].
  * ds_read_b64_tr_b16: in each 16-lane group, output lane i, element e is
    element i%4 of the 8 bytes addressed by lane 4e + i//4 of the group.
  * v_mfma_f32_32x32x64_f8f6f4 (E4M3 operands): lane l holds A[l%32][32(l//32)+b]
    and B[32(l//32)+b][l%32] in byte b = 0..31 of its eight registers (the
    pairing of A and B bytes is what matters: both take the same slot); D as
    above.
  * ds_read_b64_tr_b8: in each 16-lane group, output lane i, byte e is byte
    i%8 of the 8 bytes addressed by lane 2e + i//8 of the group.
  * v_cvt_pk_fp8_f32 d, a, b [op_sel:[0,0,1]]: a, b rounded to E4M3 (nearest
    even) into bytes 0, 1 (2, 3 with op_sel) of d, the other half of d kept;
    a magnitude above 448 is an error here (the kernel never produces one).
  * buffer_load_dwordx4 ... offen lds: lane l copies 16 bytes from
    soffset + voffset[l] of the buffer to LDS address M0 + 16 l; bytes past the
    buffer's size read as zero.
"""

from __future__ import annotations

import re

import numpy as np
import torch

LANES = 64


class EmuError(AssertionError):
    pass


def _f32(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def _u32(f):
    return np.asarray(f, dtype=np.float32).view(np.uint32)


def _bf16_rne(x):
    """float32 -> bf16 bit patterns (uint32), round to nearest even."""
    u = _u32(np.asarray(x, dtype=np.float32)).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    r = np.where(nan, 0x7FC0, r)
    return r.astype(np.uint32)


def _f16_rne(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)


def _unpack16(regs, bf16):
    """(n regs, 64) uint32 -> (64, 2n) float32 elements, low half first."""
    lo = regs & 0xFFFF
    hi = regs >> 16
    el = np.empty((regs.shape[0] * 2, LANES), dtype=np.uint32)
    el[0::2] = lo
    el[1::2] = hi
    if bf16:
        return (el << 16).view(np.float32).T.copy()
    return el.astype(np.uint16).view(np.float16).astype(np.float32).T.copy()


def _e4m3_values(regs):
    """(n regs, 64) uint32 -> (64, 4n) float64: the E4M3 values of the bytes,
    byte b of register r at index 4r + b."""
    by = np.ascontiguousarray(regs.T).view(np.uint8)               # (64, 4n), little endian
    t = torch.from_numpy(by.copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _e4m3_rne(x):
    """float32 values -> E4M3 codes (uint32), round to nearest even; the
    kernel never converts a magnitude above 448 (or a NaN)."""
    x = np.asarray(x, dtype=np.float32)
    if np.isnan(x).any() or (np.abs(x) > 448).any():
        raise EmuError("E4M3 conversion of a value outside [-448, 448]")
    t = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().astype(np.uint32)


VREG = re.compile(r"^v(\d+)$|^v\[(\d+):(\d+)\]$")
SREG = re.compile(r"^s(\d+)$|^s\[(\d+):(\d+)\]$")


def vrange(tok):
    m = VREG.match(tok)
    if not m:
        raise EmuError(f"not a VGPR operand: {tok}")
    if m.group(1) is not None:
        r = int(m.group(1))
        return r, r
    return int(m.group(2)), int(m.group(3))


def srange(tok):
    m = SREG.match(tok)
    if not m:
        raise EmuError(f"not an SGPR operand: {tok}")
    if m.group(1) is not None:
        r = int(m.group(1))
        return r, r
    return int(m.group(2)), int(m.group(3))


def parse(text):
    """Assembly text (lines separated by newlines or the inline-asm '\\n\\t')
    -> (instructions, labels, byte addresses)."""
    text = text.replace("%=", "0").replace("\\n\\t", "\n")
    ins, labels = [], {}
    for raw in text.split("\n"):
        line = raw.strip()
        if not line:
            continue
        if line.endswith(":"):
            labels[line[:-1]] = len(ins)
            continue
        op, _, rest = line.partition(" ")
        mods = re.findall(r"op_sel:\[[^\]]*\]", rest)       # modifiers whose lists hold commas
        rest = re.sub(r"\s*op_sel:\[[^\]]*\]", "", rest)
        args = ([a.strip() for a in rest.split(",")] if rest else []) + mods
        ins.append((op, args, line))
    addr, a = [], 0
    for op, args, line in ins:
        addr.append(a)
        a += _size(op, args)
    addr.append(a)
    return ins, labels, addr


def _size(op, args):
    lit = any(re.fullmatch(r"0x[0-9a-fA-F]+", x) for x in args)
    if op.startswith(("s_cbranch", "s_branch", "s_nop", "s_waitcnt", "s_barrier", "s_endpgm")):
        return 4
    if op.startswith(("s_",)):
        big = any(re.fullmatch(r"-?\d+", x) and not (-16 <= int(x) <= 64) for x in args)
        return 8 if (lit or big) else 4
    if op.startswith(("ds_", "buffer_", "v_mfma", "v_fma", "v_max3", "v_cvt_pk")):
        return 8
    if op.startswith("v_"):
        return 8 if lit else 4
    raise EmuError(f"unknown size of {op}")


class Program:
    def __init__(self, text):
        self.ins, self.labels, self.addr = parse(text)
        self.addr_to_index = {a: i for i, a in enumerate(self.addr[:-1])}


class Wave:
    def __init__(self, wid, emu, prog):
        self.wid = wid
        self.emu = emu
        self.prog = prog
        self.v = np.zeros((256, LANES), dtype=np.uint32)
        self.s = [0] * 108
        self.m0 = 0
        self.vcc = np.zeros(LANES, dtype=bool)
        self.scc = False
        self.pc = 0
        self.slot = 0                      # issue slots so far
        self.lds_q = []                    # pending LDS reads: (regs, data)
        self.vm_q = []                     # pending copies: dict
        self.pending = np.zeros(256, dtype=bool)
        self.valu_w = np.full(256, -10**9)  # slot of the last VALU write
        self.trans_w = np.full(256, -10**9)
        self.mfma_w = np.full(256, -10**9)
        self.mfma_need = np.zeros(256, dtype=np.int64)   # wait states after that MFMA
        self.mfma_dst = {}                 # reg -> dst range of the last MFMA that wrote it
        self.mfma_rd = np.full(256, -1)    # MFMA count at the last MFMA source read
        self.n_mfma = 0
        self.m0_w = -10**9
        self.done = False
        self.at_barrier = False
        self.executed = 0

    # ---- helpers -----------------------------------------------------------
    def err(self, msg):
        op, args, line = self.prog.ins[self.pc]
        raise EmuError(f"wave {self.wid}, instruction {self.pc} '{line}': {msg}")

    def rd_v(self, lo, hi, mfma=False, permlane=False, what="read"):
        rng = slice(lo, hi + 1)
        if self.pending[rng].any():
            self.err(f"v{lo}..v{hi} {what} while a load into it is pending")
        now = self.slot
        close = (now - self.mfma_w[rng] <= self.mfma_need[rng])
        if close.any() and not mfma:
            n = int(self.mfma_need[rng][close].max())
            self.err(f"MFMA result read by a non-MFMA instruction within {n} wait states")
        if (now - self.trans_w[rng] < 2).any():
            self.err("transcendental result read within 1 wait state")
        if mfma and (now - self.valu_w[rng] < 3).any():
            self.err("VALU result read by an MFMA within 2 wait states")
        if permlane and (now - self.valu_w[rng] < 3).any():
            self.err("VALU result read by v_permlane32_swap within 2 wait states")
        return self.v[rng]

    def wr_v(self, lo, hi, kind):
        rng = slice(lo, hi + 1)
        if self.pending[rng].any():
            self.err(f"v{lo}..v{hi} written while a load into it is pending")
        close = (self.slot - self.mfma_w[rng] <= self.mfma_need[rng])
        if kind != "mfma" and close.any():
            n = int(self.mfma_need[rng][close].max())
            self.err(f"register written within {n} wait states of an MFMA that wrote it")
        if kind in ("valu", "trans"):
            self.valu_w[rng] = self.slot
            if kind == "trans":
                self.trans_w[rng] = self.slot
        if kind == "load":
            used = self.mfma_rd[rng]
            if ((used >= 0) & (used >= self.n_mfma - 1)).any():
                self.err("operand buffer refilled less than two MFMAs after its use")

    def fsrc(self, tok):
        """VALU float source: VGPR, SGPR, literal, -VGPR."""
        neg = tok.startswith("-")
        t = tok[1:] if neg else tok
        if t.startswith("v"):
            lo, hi = vrange(t)
            x = _f32(self.rd_v(lo, hi)[0]).copy()
        elif t.startswith("s"):
            lo, hi = srange(t)
            x = np.full(LANES, _f32(np.uint32(self.s[lo])), dtype=np.float32)
        elif t.startswith("0x"):
            x = np.full(LANES, _f32(np.uint32(int(t, 16))), dtype=np.float32)
        else:
            x = np.full(LANES, np.float32(float(t)), dtype=np.float32)
        return -x if neg else x

    def ssrc(self, tok):
        if tok == "m0":
            return self.m0
        if tok.startswith("s"):
            return self.s[srange(tok)[0]]
        return int(tok, 0) & 0xFFFFFFFF

    # ---- memory ------------------------------------------------------------
    def complete_lds(self, keep):
        while len(self.lds_q) > keep:
            regs, data = self.lds_q.pop(0)
            lo, hi = regs
            self.v[lo:hi + 1] = data
            self.pending[lo:hi + 1] = False

    def complete_vm(self, keep):
        while len(self.vm_q) > keep:
            c = self.vm_q.pop(0)
            if "regs" in c:
                lo, hi = c["regs"]
                self.v[lo:hi + 1] = c["data"]
                self.pending[lo:hi + 1] = False
            else:
                self.emu.lds_write(c, self)

    # ---- execute one instruction ---------------------------------------------
    def step(self):
        emu = self.emu
        prog = self.prog
        op, args, line = prog.ins[self.pc]
        self.executed += 1
        if self.executed > emu.max_steps:
            self.err("too many instructions (no exit from the loop?)")
        nxt = self.pc + 1
        self.slot += 1
        if op == "s_nop":
            self.slot += int(args[0])
        elif op == "s_waitcnt":
            for f in line.split()[1:]:
                m = re.match(r"(vmcnt|lgkmcnt|expcnt)\((\d+)\)", f)
                if not m:
                    self.err("bad s_waitcnt")
                n = int(m.group(2))
                if m.group(1) == "lgkmcnt":
                    self.complete_lds(n)
                elif m.group(1) == "vmcnt":
                    self.complete_vm(n)
        elif op == "s_barrier":
            self.at_barrier = True
            self.pc = nxt
            return
        elif op == "s_mov_b32":
            self.sset(args[0], self.ssrc(args[1]))
        elif op == "s_mov_b64":
            dlo, _ = srange(args[0])
            slo, _ = srange(args[1])
            self.s[dlo], self.s[dlo + 1] = self.s[slo], self.s[slo + 1]
        elif op == "s_cselect_b32":
            self.sset(args[0], self.ssrc(args[1]) if self.scc else self.ssrc(args[2]))
        elif op == "s_cselect_b64":
            dlo, _ = srange(args[0])
            slo, _ = srange(args[1] if self.scc else args[2])
            self.s[dlo], self.s[dlo + 1] = self.s[slo], self.s[slo + 1]
        elif op == "s_sub_u32":
            r = self.ssrc(args[1]) - self.ssrc(args[2])
            self.scc = r < 0
            self.sset(args[0], r & 0xFFFFFFFF)
        elif op == "s_add_u32":
            r = self.ssrc(args[1]) + self.ssrc(args[2])
            self.scc = r > 0xFFFFFFFF
            self.sset(args[0], r & 0xFFFFFFFF)
        elif op == "s_addc_u32":
            r = self.ssrc(args[1]) + self.ssrc(args[2]) + int(self.scc)
            self.scc = r > 0xFFFFFFFF
            self.sset(args[0], r & 0xFFFFFFFF)
        elif op == "s_lshl_b32":
            r = (self.ssrc(args[1]) << self.ssrc(args[2])) & 0xFFFFFFFF
            self.scc = r != 0
            self.sset(args[0], r)
        elif op == "s_cmp_lt_u32":
            self.scc = self.ssrc(args[0]) < self.ssrc(args[1])
        elif op == "s_cmp_eq_u32":
            self.scc = self.ssrc(args[0]) == self.ssrc(args[1])
        elif op in ("s_branch", "s_cbranch_scc0", "s_cbranch_scc1", "s_cbranch_vccz", "s_cbranch_vccnz"):
            take = {"s_branch": True, "s_cbranch_scc0": not self.scc, "s_cbranch_scc1": self.scc,
                    "s_cbranch_vccz": not self.vcc.any(), "s_cbranch_vccnz": self.vcc.any()}[op]
            if take:
                if args[0] not in prog.labels:
                    self.err("unknown label")
                nxt = prog.labels[args[0]]
                emu.label_hits[args[0]] = emu.label_hits.get(args[0], 0) + 1
        elif op == "s_getpc_b64":
            lo, _ = srange(args[0])
            a = prog.addr[nxt]
            self.s[lo], self.s[lo + 1] = a & 0xFFFFFFFF, a >> 32
        elif op == "s_setpc_b64":
            lo, _ = srange(args[0])
            a = self.s[lo] | (self.s[lo + 1] << 32)
            if a not in prog.addr_to_index:
                self.err("s_setpc_b64 to an address that is not an instruction")
            nxt = prog.addr_to_index[a]
        elif op in ("ds_read_b128", "ds_read_b64_tr_b16", "ds_read_b64_tr_b8"):
            self.ds_read(op, args)
        elif op == "buffer_load_dwordx4" and "lds" in line:
            self.lds_copy(args, line)
        elif op == "buffer_load_dwordx4":
            self.vgpr_load(args, line)
        elif op.startswith("v_mfma_f32_32x32x16_") or op == "v_mfma_f32_32x32x64_f8f6f4":
            self.mfma(op, args)
        elif op.startswith("v_"):
            self.valu(op, args)
        else:
            self.err("unsupported instruction")
        self.pc = nxt

    def sset(self, tok, val):
        if tok == "m0":
            self.m0 = val
            self.m0_w = self.slot
        else:
            lo, _ = srange(tok)
            self.s[lo] = val

    def valu(self, op, args):
        if op == "v_mov_b32":
            x = self.fsrc(args[1])
            self.wr_v(*vrange(args[0]), "valu")
            self.v[vrange(args[0])[0]] = _u32(x)
        elif op in ("v_add_f32", "v_sub_f32", "v_mul_f32", "v_max_f32"):
            a, b = self.fsrc(args[1]), self.fsrc(args[2])
            r = {"v_add_f32": lambda: a + b, "v_sub_f32": lambda: a - b, "v_mul_f32": lambda: a * b,
                 "v_max_f32": lambda: np.fmax(a, b)}[op]()
            self.wr_v(*vrange(args[0]), "valu")
            self.v[vrange(args[0])[0]] = _u32(r.astype(np.float32))
        elif op == "v_fma_f32":
            a, b, c = (self.fsrc(t).astype(np.float64) for t in args[1:4])
            self.wr_v(*vrange(args[0]), "valu")
            self.v[vrange(args[0])[0]] = _u32((a * b + c).astype(np.float32))
        elif op == "v_max3_f32":
            a, b, c = (self.fsrc(t) for t in args[1:4])
            self.wr_v(*vrange(args[0]), "valu")
            self.v[vrange(args[0])[0]] = _u32(np.fmax(np.fmax(a, b), c))
        elif op == "v_exp_f32":
            a = self.fsrc(args[1])
            self.wr_v(*vrange(args[0]), "trans")
            with np.errstate(over="ignore"):
                self.v[vrange(args[0])[0]] = _u32(np.exp2(a.astype(np.float64)).astype(np.float32))
        elif op in ("v_cvt_pk_bf16_f32", "v_cvt_pk_f16_f32"):
            a, b = self.fsrc(args[1]), self.fsrc(args[2])
            f = _bf16_rne if op == "v_cvt_pk_bf16_f32" else _f16_rne
            self.wr_v(*vrange(args[0]), "valu")
            self.v[vrange(args[0])[0]] = f(a) | (f(b) << 16)
        elif op == "v_permlane32_swap_b32":
            (a, _), (b, _) = vrange(args[0]), vrange(args[1])
            xa = self.rd_v(a, a, permlane=True)[0].copy()
            xb = self.rd_v(b, b, permlane=True)[0].copy()
            self.wr_v(a, a, "valu")
            self.wr_v(b, b, "valu")
            na, nb = xa.copy(), xb.copy()
            na[32:] = xb[:32]
            nb[:32] = xa[32:]
            self.v[a], self.v[b] = na, nb
        elif op == "v_cvt_pk_fp8_f32":
            a, b = self.fsrc(args[1]), self.fsrc(args[2])
            hi = "op_sel:[0,0,1]" in args[3:]
            dlo, _ = vrange(args[0])
            old = self.rd_v(dlo, dlo)[0].copy()
            word = _e4m3_rne(a) | (_e4m3_rne(b) << 8)
            self.wr_v(dlo, dlo, "valu")
            self.v[dlo] = (old & 0x0000FFFF) | (word << 16) if hi else (old & 0xFFFF0000) | word
        elif op == "v_cndmask_b32":
            if args[3] != "vcc":
                self.err("v_cndmask_b32 must select on vcc")
            x0, x1 = _u32(self.fsrc(args[1])), _u32(self.fsrc(args[2]))
            self.wr_v(*vrange(args[0]), "valu")
            self.v[vrange(args[0])[0]] = np.where(self.vcc, x1, x0)
        elif op in ("v_cmp_lt_f32", "v_cmp_neq_f32"):
            if args[0] != "vcc":
                self.err("compare must write vcc")
            a, b = self.fsrc(args[1]), self.fsrc(args[2])
            with np.errstate(invalid="ignore"):
                self.vcc = (a < b) if op == "v_cmp_lt_f32" else ~(a == b)
        else:
            self.err("unsupported VALU instruction")

    def mfma(self, op, args):
        fp8 = op == "v_mfma_f32_32x32x64_f8f6f4"
        nreg = 8 if fp8 else 4            # A / B registers per lane
        kw = 32 if fp8 else 8             # k slots per lane half
        need = 20 if fp8 else 12          # wait states before a VALU may read the result
        dlo, dhi = vrange(args[0])
        alo, ahi = vrange(args[1])
        blo, bhi = vrange(args[2])
        if dhi - dlo != 15 or ahi - alo != nreg - 1 or bhi - blo != nreg - 1:
            self.err("operand sizes")
        if fp8:
            a = _e4m3_values(self.rd_v(alo, ahi, mfma=True))   # (64, 32)
            b = _e4m3_values(self.rd_v(blo, bhi, mfma=True))
        else:
            a = _unpack16(self.rd_v(alo, ahi, mfma=True), op.endswith("bf16"))   # (64, 8)
            b = _unpack16(self.rd_v(blo, bhi, mfma=True), op.endswith("bf16"))
        A = np.zeros((32, 2 * kw), dtype=np.float64)
        B = np.zeros((2 * kw, 32), dtype=np.float64)
        for half in range(2):
            A[:, kw * half:kw * half + kw] = a[32 * half:32 * half + 32]
            B[kw * half:kw * half + kw, :] = b[32 * half:32 * half + 32].T
        if args[3] == "0":
            C = np.zeros((32, 32), dtype=np.float32)
        else:
            clo, chi = vrange(args[3])
            if (clo, chi) != (dlo, dhi):
                self.err("srcC must be the destination (accumulation chain) or 0")
            rng = slice(clo, chi + 1)
            if self.pending[rng].any():
                self.err("srcC pending")
            if (self.slot - self.valu_w[rng] < 3).any():
                self.err("VALU result read as srcC within 2 wait states")
            for r in range(clo, chi + 1):
                w = self.mfma_dst.get(r)
                if self.slot - self.mfma_w[r] < self.mfma_need[r] and w != (dlo, dhi):
                    self.err(f"srcC from a different MFMA within {self.mfma_need[r]} wait states")
            C = self.acc_to_mat(self.v[clo:chi + 1])
        D = (A.astype(np.float64) @ B.astype(np.float64) + C).astype(np.float32)
        for r in (range(alo, ahi + 1)):
            self.mfma_rd[r] = self.n_mfma
        for r in (range(blo, bhi + 1)):
            self.mfma_rd[r] = self.n_mfma
        self.n_mfma += 1
        self.wr_v(dlo, dhi, "mfma")
        # a destination still counted by an earlier MFMA's result window is fine
        # only for the same accumulation chain
        for r in range(dlo, dhi + 1):
            if self.slot - self.mfma_w[r] < self.mfma_need[r] and self.mfma_dst.get(r) != (dlo, dhi):
                self.err(f"MFMA writes registers of a different MFMA within {self.mfma_need[r]} wait states")
        self.v[dlo:dhi + 1] = self.mat_to_acc(D)
        self.mfma_w[dlo:dhi + 1] = self.slot
        self.mfma_need[dlo:dhi + 1] = need
        for r in range(dlo, dhi + 1):
            self.mfma_dst[r] = (dlo, dhi)

    @staticmethod
    def acc_to_mat(regs):
        M = np.zeros((32, 32), dtype=np.float32)
        f = _f32(regs)
        for r in range(16):
            for lh in range(2):
                i = 8 * (r // 4) + 4 * lh + r % 4
                M[i, :] = f[r, 32 * lh:32 * lh + 32]
        return M

    @staticmethod
    def mat_to_acc(M):
        out = np.zeros((16, LANES), dtype=np.uint32)
        for r in range(16):
            for lh in range(2):
                i = 8 * (r // 4) + 4 * lh + r % 4
                out[r, 32 * lh:32 * lh + 32] = _u32(M[i, :])
        return out

    def ds_read(self, op, args):
        dlo, dhi = vrange(args[0])
        alo, _ = vrange(args[1].split()[0])
        m = re.search(r"offset:(\d+)", args[1])
        off = int(m.group(1)) if m else 0
        addr = self.rd_v(alo, alo)[0].astype(np.int64) + off
        nbytes = 16 if op == "ds_read_b128" else 8
        if dhi - dlo + 1 != nbytes // 4:
            self.err("destination size")
        self.wr_v(dlo, dhi, "load")
        raw = np.zeros((LANES, nbytes), dtype=np.uint8)
        for l in range(LANES):
            a = int(addr[l])
            if a < 0 or a + nbytes > self.emu.lds_size or a % 8:
                self.err(f"LDS read out of range or misaligned at {a}")
            self.emu.lds_read_check(a, nbytes, self)
            raw[l] = self.emu.lds[a:a + nbytes]
        if op == "ds_read_b128":
            data = raw.view(np.uint32).T.copy()            # (4, 64)
        elif op == "ds_read_b64_tr_b8":
            out = np.zeros((LANES, 8), dtype=np.uint8)
            for g in range(4):
                for i in range(16):
                    for e in range(8):
                        out[16 * g + i, e] = raw[16 * g + 2 * e + i // 8, i % 8]
            data = out.view(np.uint32).T.copy()            # (2, 64)
        else:
            el = raw.view(np.uint16)                        # (64, 4)
            out = np.zeros((LANES, 4), dtype=np.uint16)
            for g in range(4):
                for i in range(16):
                    for e in range(4):
                        out[16 * g + i, e] = el[16 * g + 4 * e + i // 4, i % 4]
            data = out.view(np.uint32).T.copy()            # (2, 64)
        self.pending[dlo:dhi + 1] = True
        self.lds_q.append(((dlo, dhi), data))

    def vgpr_load(self, args, line):
        """buffer_load_dwordx4 vD, vOff, s[desc], sOff offen offset:N: lane l
        reads 16 bytes at sOff + vOff[l] + N (zeros past the buffer)."""
        dlo, dhi = vrange(args[0])
        vlo, _ = vrange(args[1])
        blo, _ = srange(args[2])
        toks = args[3].split()
        soff = self.ssrc(toks[0])
        m = re.search(r"offset:(\d+)", args[3])
        off = int(m.group(1)) if m else 0
        if "offen" not in toks or dhi - dlo != 3:
            self.err("unsupported buffer load form")
        voff = self.rd_v(vlo, vlo)[0].astype(np.int64)
        buf = self.emu.buffers[self.s[blo]]
        data = np.zeros((LANES, 16), dtype=np.uint8)
        for l in range(LANES):
            g = soff + int(voff[l]) + off
            if g + 16 <= len(buf):
                data[l] = np.frombuffer(buf, dtype=np.uint8, count=16, offset=g)
        self.wr_v(dlo, dhi, "load")
        self.pending[dlo:dhi + 1] = True
        self.vm_q.append({"regs": (dlo, dhi), "data": data.view(np.uint32).T.copy()})

    def lds_copy(self, args, line):
        if "offen lds" not in line:
            self.err("only offen lds copies are supported")
        vlo, _ = vrange(args[0])
        dlo, _ = srange(args[1].split()[0])
        soff = self.ssrc(args[2].split()[0])
        if self.slot - self.m0_w < 2:
            self.err("M0 written within 1 wait state of an LDS copy")
        voff = self.rd_v(vlo, vlo)[0].astype(np.int64)
        buf = self.emu.buffers[self.s[dlo]]
        src = np.zeros((LANES, 16), dtype=np.uint8)
        for l in range(LANES):
            g = soff + int(voff[l])
            if g % 16:
                self.err("unaligned copy source")
            if g < 0 or g + 16 > len(buf):
                # the loops put the tile offset in soffset, which the range
                # check of a raw buffer does not cover: every copy must stay
                # inside the buffer by construction
                self.err(f"copy source {g} outside the buffer of {len(buf)} bytes")
            src[l] = np.frombuffer(buf, dtype=np.uint8, count=16, offset=g)
        dst = self.m0
        if dst < 0 or dst + 1024 > self.emu.lds_size or dst % 1024:
            self.err(f"LDS copy destination {dst} out of range")
        c = {"dst": dst, "data": src.reshape(-1), "issue": self.emu.phase, "wave": self.wid}
        self.emu.lds_copy_issue(c, self)
        self.vm_q.append(c)


class Emulator:
    """texts: the program of every wave of the workgroup."""

    def __init__(self, texts, lds_size, buffers, max_steps=200000, copies_may_continue=False):
        """copies_may_continue: a program may end with global->LDS copies in
        flight (the next program waits for them); they are completed at the
        end of the run."""
        self.copies_may_continue = copies_may_continue
        progs = {}
        for t in texts:
            if t not in progs:
                progs[t] = Program(t)
        self.lds_size = lds_size
        self.lds = np.zeros(lds_size, dtype=np.uint8)
        self.buffers = buffers
        self.max_steps = max_steps
        self.phase = 0
        g = lds_size // 8
        self.read_phase = np.full(g, -1)         # last phase a granule was read
        self.copy_pending = np.zeros(g, dtype=np.int64)   # copies in flight into a granule
        self.copy_done_phase = np.full(g, -1)    # phase a copy into the granule completed
        self.copy_issue_phase = np.full(g, -1)
        self.waves = [Wave(i, self, progs[t]) for i, t in enumerate(texts)]
        self.label_hits = {}     # branch target -> times taken

    def lds_read_check(self, a, n, w):
        g0, g1 = a // 8, (a + n - 1) // 8 + 1
        if (self.copy_pending[g0:g1] > 0).any():
            w.err(f"LDS read at {a} while a copy into it is in flight")
        if (self.copy_done_phase[g0:g1] >= self.phase).any():
            w.err(f"LDS read at {a} in the barrier phase in which a copy into it completed")
        if (self.copy_issue_phase[g0:g1] >= self.phase).any():
            w.err(f"LDS read at {a} in the barrier phase in which a copy into it was issued")
        self.read_phase[g0:g1] = self.phase

    def lds_copy_issue(self, c, w):
        g0, g1 = c["dst"] // 8, (c["dst"] + 1024) // 8
        if (self.read_phase[g0:g1] >= self.phase).any():
            w.err("copy into LDS bytes read by some wave in the same barrier phase")
        if (self.copy_pending[g0:g1] > 0).any():
            w.err("copy into LDS bytes with another copy in flight")
        self.copy_pending[g0:g1] += 1
        self.copy_issue_phase[g0:g1] = self.phase

    def lds_write(self, c, w):
        g0, g1 = c["dst"] // 8, (c["dst"] + 1024) // 8
        self.lds[c["dst"]:c["dst"] + 1024] = c["data"]
        self.copy_pending[g0:g1] -= 1
        self.copy_done_phase[g0:g1] = self.phase

    def run(self):
        while True:
            for w in self.waves:
                while not w.done and not w.at_barrier:
                    if w.pc >= len(w.prog.ins):
                        w.done = True
                        break
                    w.step()
            at = [w.at_barrier for w in self.waves]
            dn = [w.done for w in self.waves]
            if all(dn):
                break
            if not all(a or d for a, d in zip(at, dn)) or (any(at) and any(dn)):
                raise EmuError(f"barrier mismatch: at barrier {at}, finished {dn}")
            for w in self.waves:
                w.at_barrier = False
            self.phase += 1
        for w in self.waves:
            if w.lds_q or any("regs" in c for c in w.vm_q) or (w.vm_q and not self.copies_may_continue):
                raise EmuError(f"wave {w.wid} ends with loads in flight")
            w.complete_vm(0)
        return self.waves
