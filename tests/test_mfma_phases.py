"""Host checks of the hand-scheduled MFMA phase blocks (no GPU needed).

The blocks in exact_attention_63_amd/csrc/fa2_mfma_phases.inc are generated;
these tests pin the committed file to its generator and simulate every block:
each MFMA must read the buffer filled by its own operand read(s), those reads
must be complete under the preceding lgkmcnt wait (LDS reads complete in
order), and no buffer may be refilled before two further MFMAs were issued.
"""

import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_63_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_mfma_phases", os.path.join(CSRC, "gen_mfma_phases.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _blocks():
    text = open(os.path.join(CSRC, "fa2_mfma_phases.inc")).read()
    out = {}
    for name, body in re.findall(r'#define (FA2_ASM_(?:SCORES|PV)_(?:BF16|F16)_L\d+) "(.*)"', text):
        out[name] = body.split("\\n\\t")
    return out


def test_committed_file_matches_generator():
    gen = _gen()
    with open(gen.OUTPUT) as f:
        assert f.read() == gen.generate()


def simulate(body, pv):
    """Returns a list of problems found in one block."""
    problems = []
    writer = {}       # VGPR -> index of the read that last wrote it
    last_mfma = {}    # VGPR -> index of the last MFMA that read it
    nread = done = mf = 0
    for ins in body:
        if ins.startswith("ds_read"):
            lo, hi = map(int, re.search(r"v\[(\d+):(\d+)\]", ins).groups())
            for r in range(lo, hi + 1):
                if r in last_mfma and last_mfma[r] >= mf - 1:
                    problems.append(f"read {nread} refills v{r} one MFMA after its use")
                writer[r] = nread
            nread += 1
        elif ins.startswith("s_waitcnt"):
            done = max(done, nread - int(re.search(r"lgkmcnt\((\d+)\)", ins).group(1)))
        elif ins.startswith("v_mfma"):
            lo, hi = map(int, re.search(r"v\[(\d+):(\d+)\]", ins).groups())
            want = [2 * mf, 2 * mf + 1] if pv else [mf]
            got = sorted({writer.get(r, -1) for r in range(lo, hi + 1)})
            if got != want:
                problems.append(f"MFMA {mf} reads operands of reads {got}, expected {want}")
            if done < want[-1] + 1:
                problems.append(f"MFMA {mf} issued before its operand read completed")
            for r in range(lo, hi + 1):
                last_mfma[r] = mf
            mf += 1
    if mf != 16:
        problems.append(f"{mf} MFMAs, expected 16")
    if nread != (32 if pv else 16):
        problems.append(f"{nread} reads")
    if body[-3:] != ["s_nop 7", "s_nop 7", "s_nop 4"]:
        problems.append("block does not end with the MFMA-result hazard padding")
    return problems


@pytest.mark.parametrize("name", sorted(_blocks()))
def test_block_schedule(name):
    body = _blocks()[name]
    assert simulate(body, "_PV_" in name) == []


def test_simulator_catches_a_short_wait():
    """A planted mistake: one wait allows one read too many in flight."""
    name = sorted(n for n in _blocks() if "_SCORES_" in n)[0]
    body = list(_blocks()[name])
    i = next(k for k, ins in enumerate(body) if ins.startswith("s_waitcnt lgkmcnt(") and "(0)" not in ins)
    n = int(re.search(r"\((\d+)\)", body[i]).group(1))
    body[i] = f"s_waitcnt lgkmcnt({n + 1})"
    assert any("before its operand read completed" in p for p in simulate(body, False))


def test_simulator_catches_a_wrong_buffer():
    name = sorted(n for n in _blocks() if "_PV_" in n)[0]
    body = list(_blocks()[name])
    i = next(k for k, ins in enumerate(body) if ins.startswith("v_mfma"))
    j = next(k for k, ins in enumerate(body) if k > i and ins.startswith("v_mfma"))
    # swap the A operands of the first two MFMAs
    a_i = re.search(r"v\[\d+:\d+\]", body[i]).group(0)
    a_j = re.search(r"v\[\d+:\d+\]", body[j]).group(0)
    body[i] = body[i].replace(a_i, a_j, 1)
    body[j] = body[j].replace(a_j, a_i, 1)
    assert any("reads operands of reads" in p for p in simulate(body, True))
