"""Static checks on the compiled kernels (gfx950 assembly; no GPU needed).

The ring engines issue v_mfma_f32_16x16x32 as inline assembly with the
accumulator as an in-out AGPR operand, so that each accumulator stays in its
own registers. The compiler then treats those statements as opaque: it
inserts none of the wait states that separate an MFMA from VALU work on its
registers, and nothing but these checks would notice if a later change made
it copy or spill accumulators. The bf16 forward and backward units are
compiled to assembly here and every kernel in them is checked:

- every loop that holds MFMAs has no accumulator copy (v_accvgpr_mov), and
  the unrolled steady-state K loops have no scratch access;
- no VALU instruction writes a register that an inline-assembly MFMA reads
  as its A or B operand within the two wait states before it (the
  VALU-write to MFMA-read hazard);
- a VALU write of an accumulator (the zero fill) is at least 5 wait states
  before an inline-assembly MFMA that reads it, and such an MFMA's result is
  at least 19 wait states before a VALU read of it (the 16-pass bound,
  larger than any 16x16x32 needs). Wait states: one per instruction, N + 1
  per s_nop N, counted in program order. The builtin MFMAs of the other
  kernels are the compiler's to guard.
"""

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from backward_gate_up_amd import build as B

UNITS = {"bf16_fwd": ["-DSWIGLU_INST_DTYPE=0", "-DSWIGLU_INST_OP=0", "-DSWIGLU_INST_LIN=0"],
         "bf16_bwd": ["-DSWIGLU_INST_DTYPE=0", "-DSWIGLU_INST_OP=1", "-DSWIGLU_INST_LIN=0"]}


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="swiglu_isa_")
    try:
        def one(item):
            name, defs = item
            out = os.path.join(tmp, name + ".s")
            flags = [f for f in B.FLAGS if f != "-fPIC"]
            cmd = [B.HIPCC] + flags + defs + ["--cuda-device-only", "-S", "-o", out,
                                              os.path.join(B.CSRC, "instantiate.hip")]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            with open(out) as f:
                return name, f.read()

        with ThreadPoolExecutor(len(UNITS)) as ex:
            return dict(ex.map(one, UNITS.items()))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _kernels(text):
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w+):", text, re.M)]
    for i, (pos, name) in enumerate(starts):
        end = starts[i + 1][0] if i + 1 < len(starts) else len(text)
        yield name, text[pos:end]


def _instrs(body):
    """Instructions in program order, each with whether it came from an
    inline-assembly statement (between the ;;#ASMSTART / ;;#ASMEND markers
    the compiler writes around them)."""
    out, inline = [], False
    for ln in body.splitlines():
        s = ln.strip()
        if s.startswith(";;#ASMSTART"):
            inline = True
        elif s.startswith(";;#ASMEND"):
            inline = False
        t = ln.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        out.append((t, inline))
    return out


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(ins):
    parts = ins.split(None, 1)
    return [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []


def _wait_states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def test_mfma_loops_have_no_accumulator_copies_or_spills(asm):
    loops = steady = 0
    for unit, text in asm.items():
        for name, body in _kernels(text):
            lines = body.splitlines()
            labels = {}
            for i, ln in enumerate(lines):
                m = re.match(r"^(\.LBB\d+_\d+):", ln)
                if m:
                    labels[m.group(1)] = i
            for i, ln in enumerate(lines):
                m = re.search(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", ln)
                if not m or m.group(1) not in labels or labels[m.group(1)] >= i:
                    continue
                loop = "\n".join(lines[labels[m.group(1)]:i])
                if "v_mfma" not in loop:
                    continue
                loops += 1
                assert "v_accvgpr_mov" not in loop, (unit, name, m.group(1))
                # the unrolled steady-state loops (four 32-K steps, or five
                # 64-K stages); the last-stage loops select their LDS arrays
                # at run time and may load those pointers from scratch
                if loop.count("v_mfma") >= 256:
                    steady += 1
                    assert "scratch_" not in loop, (unit, name, m.group(1))
    assert loops > 0 and steady > 0


def _check_valu_to_mfma_source(unit, text):
    """Returns the number of inline-assembly MFMAs checked."""
    n = 0
    for name, body in _kernels(text):
        ins = _instrs(body)
        for i, (t, inline) in enumerate(ins):
            if not (inline and t.startswith("v_mfma_f32_16x16x32")):
                continue
            n += 1
            ops = _operands(t)
            src = _regs(ops[1]) | _regs(ops[2])
            states = 0
            for p, _ in reversed(ins[max(0, i - 4):i]):
                if states >= 2:
                    break
                if p.startswith("v_") and not p.startswith(("v_mfma", "v_accvgpr_read")):
                    ops_p = _operands(p)
                    assert not (ops_p and _regs(ops_p[0]) & src), (unit, name, p, t)
                states += _wait_states(p)
    return n


def _check_fences(unit, text):
    """VALU write -> MFMA read: >= 5 wait states; MFMA write -> VALU read:
    >= 19, in program order within each kernel."""
    for name, body in _kernels(text):
        recent_valu = []  # (position in wait states, AGPRs written)
        recent_mfma = []
        pos = 0
        for t, inline in _instrs(body):
            ops = _operands(t)
            if inline and t.startswith("v_mfma_f32_16x16x32"):
                srcc = _regs(ops[3]) if len(ops) > 3 else set()
                for p, regs in recent_valu:
                    assert pos - p >= 5 or not (regs & srcc), (unit, name, t)
                recent_mfma = [(p, r) for p, r in recent_mfma if pos - p < 19] + [(pos, _regs(ops[0]))]
            elif t.startswith("v_accvgpr_read"):
                src = _regs(ops[1]) if len(ops) > 1 else set()
                for p, regs in recent_mfma:
                    assert pos - p >= 19 or not (regs & src), (unit, name, t)
            elif t.startswith(("v_accvgpr_write", "v_accvgpr_mov")):
                recent_valu = [(p, r) for p, r in recent_valu if pos - p < 5] + [(pos, _regs(ops[0]))]
            pos += _wait_states(t)


def test_no_valu_write_right_before_an_mfma_source(asm):
    assert sum(_check_valu_to_mfma_source(u, t) for u, t in asm.items()) > 0


def test_accumulator_fences(asm):
    for u, t in asm.items():
        _check_fences(u, t)


_SNIPPET = """_Zk:
\tv_accvgpr_write_b32 a0, 0
\ts_nop {fill}
\t;;#ASMSTART
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[{b}:{b3}], a[0:3]
\t;;#ASMEND
\tv_mov_b32_e32 v20, 0
\ts_nop {drain}
\tv_accvgpr_read_b32 v1, a2
"""


@pytest.mark.parametrize("fill,b,drain,ok", [(4, 8, 17, True), (2, 8, 17, False), (4, 8, 10, False)])
def test_fence_checker_flags_short_fences(fill, b, drain, ok):
    text = _SNIPPET.format(fill=fill, b=b, b3=b + 3, drain=drain)
    if ok:
        _check_fences("snippet", text)
    else:
        with pytest.raises(AssertionError):
            _check_fences("snippet", text)


def test_source_checker_flags_a_valu_write_into_an_operand():
    text = _SNIPPET.format(fill=4, b=8, b3=11, drain=17).replace("\ts_nop 4\n", "\tv_mov_b32_e32 v9, 0\n")
    with pytest.raises(AssertionError):
        _check_valu_to_mfma_source("snippet", text)
    assert _check_valu_to_mfma_source("snippet", _SNIPPET.format(fill=4, b=8, b3=11, drain=17)) == 1
