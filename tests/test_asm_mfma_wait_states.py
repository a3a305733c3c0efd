"""Static check of the compiled kernels: wait states before every MFMA (CPU
only: hipcc, no GPU).

An MFMA that reads a register written by a VALU instruction (a VGPR operand,
or an AGPR accumulator zeroed by v_accvgpr_write) needs two wait states
between the two instructions; the compiler inserts them for the MFMAs it
issues, but the gradient kernel's dV^T/dK^T products are inline assembly, for
which the kernel supplies its own `s_nop`s.  This test compiles every kernel
source with the library's own flags and follows each function's control
flow, counting for each register the wait states since its last VALU write
(an `s_nop N` counts N + 1, any other instruction 1; at a join the smaller
count holds).  Every MFMA source register must have at least two.
"""
import re
import shutil
import os

import pytest

from test_asm_lds_reads import _blocks, _compile_to_asm, _functions

SOURCES = ["attn_bf16.hip", "attn_fp8.hip", "attn_bwd.hip"]
NEED = 2  # wait states between a VALU write and an MFMA read of the register

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(4), int(m.group(5))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return frozenset(out)


def _operands(s):
    return [o.strip() for o in s.split(None, 1)[1].split(",")] if " " in s else []


def _valu_dsts(s):
    """Registers a VALU instruction writes (none for MFMAs and compares)."""
    op = s.split()[0]
    if not op.startswith("v_") or op.startswith("v_mfma") or op.startswith("v_cmp"):
        return frozenset()
    ops = _operands(s)
    if not ops:
        return frozenset()
    if "swap" in op:  # v_permlane*_swap writes both operands
        return _regs(ops[0]) | _regs(ops[1] if len(ops) > 1 else "")
    return _regs(ops[0])


def _advance(state, n):
    return {r: c + n for r, c in state.items() if c + n < NEED}


def _step(state, s, report):
    op = s.split()[0]
    if op.startswith("v_mfma") and report is not None:
        srcs = frozenset().union(*(_regs(o) for o in _operands(s)[1:4]))
        close = sorted(r for r in srcs if r in state)
        if close:
            report.append((s, close[:4], min(state[r] for r in close)))
    m = re.match(r"s_nop\s+(\d+)", s)
    state = _advance(state, int(m.group(1)) + 1 if m else 1)
    for r in _valu_dsts(s):
        state[r] = 0
    return state


def _merge(a, b):
    out = dict(a)
    for r, c in b.items():
        out[r] = min(c, out.get(r, NEED))
    return out


def check_function(items):
    blocks, succ = _blocks(items)
    state = {0: {}}
    work = [0]
    while work:
        i = work.pop()
        st = dict(state[i])
        for s in blocks[i]:
            st = _step(st, s, None)
        for j in succ[i]:
            new = st if j not in state else _merge(state[j], st)
            if j not in state or new != state[j]:
                state[j] = new
                work.append(j)
    bad, mfmas = [], 0
    for i, b in enumerate(blocks):
        st = dict(state.get(i, {}))
        for s in b:
            if s.split()[0].startswith("v_mfma"):
                mfmas += 1
            st = _step(st, s, bad)
    return mfmas, bad


def test_checker_counts_wait_states():
    """The checker itself: an MFMA right after the VALU write of its B operand
    is reported, with `s_nop 1` in between it is not, and a write at the end
    of a loop body is seen by the MFMA at the loop's head."""
    close = [("inst", "v_cvt_pk_bf16_f32 v4, v0, v1"),
             ("inst", "v_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[4:7], a[0:15]"),
             ("inst", "s_endpgm")]
    n, bad = check_function(close)
    assert n == 1 and len(bad) == 1 and bad[0][2] == 0
    padded = [close[0], ("inst", "s_nop 1"), close[1], close[2]]
    assert check_function(padded)[1] == []
    loop = [("label", ".LBB0_1"),
            ("inst", "v_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[4:7], a[0:15]"),
            ("inst", "s_nop 3"), ("inst", "v_mov_b32 v5, v0"),
            ("inst", "s_cbranch_scc1 .LBB0_1"), ("inst", "s_endpgm")]
    _, bad = check_function(loop)
    assert len(bad) == 1  # v5, written one instruction before the back edge
    zero_then_use = [("inst", "v_accvgpr_write_b32 a3, 0"),
                     ("inst", "v_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[4:7], a[0:15]"),
                     ("inst", "s_endpgm")]
    assert len(check_function(zero_then_use)[1]) == 1


@pytest.mark.parametrize("src", SOURCES)
def test_mfma_sources_have_two_wait_states(src, tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    asm = _compile_to_asm(src, tmp_path)
    funcs = _functions(asm)
    assert funcs, "no kernel found in the listing"
    total, problems = 0, []
    for name, items in funcs:
        n, bad = check_function(items)
        total += n
        problems += [(name[:60],) + b for b in bad[:3]]
    assert total > 0
    assert not problems, problems[:6]
