"""Static check of the compiled attention kernels (CPU only: hipcc, no GPU).

Several LDS reads in the kernels are issued as inline assembly, so the
compiler's wait-count pass does not track them: their results are valid only
after an explicit ``s_waitcnt lgkmcnt`` that passes the registers through.
The compiler still treats an assembly output as written at once, so nothing
in the generated code may read, copy or overwrite such a destination register
(or reuse an address register) while the read is in flight.

This test compiles every kernel source that uses these reads to gfx950
assembly, with the library's own flags, and follows each function's control
flow: LDS reads complete in issue order, so after ``lgkmcnt(N)`` only the N
newest reads can still be in flight (scalar loads and LDS writes share the
counter, which only makes this model conservative).  At a join the in-flight
sets of the predecessors are merged.  Any instruction that names a register of
an in-flight read fails the test.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from exact_attention_74_amd import build as _build  # noqa: E402

SOURCES = ["attn_bf16.hip", "attn_fp8.hip", "attn_bwd.hip"]
MAXQ = 64  # in-flight reads tracked per path (more than the counter can hold)

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vregs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return frozenset(out)


def _functions(asm):
    """(name, [instruction or label lines]) for every kernel in the listing."""
    funcs, cur, name = [], None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if cur is not None:
                funcs.append((name, cur))
            name, cur = m.group(1), []
            continue
        if cur is None:
            continue
        if re.match(r"^\s*\.Lfunc_end", line):
            funcs.append((name, cur))
            cur = None
            continue
        s = line.split(";")[0].strip()
        if not s:
            continue
        if re.match(r"^\.LBB[\d_]+:$", s):
            cur.append(("label", s[:-1]))
        elif not s.startswith("."):
            cur.append(("inst", s))
    return funcs


def _blocks(items):
    """Basic blocks: lists of instructions, with successor indices."""
    blocks, labels, cur = [], {}, []

    def close():
        nonlocal cur
        if cur or not blocks:
            blocks.append(cur)
        cur = []

    for kind, s in items:
        if kind == "label":
            if cur:
                close()
            labels[s] = len(blocks)
            continue
        cur.append(s)
        op = s.split()[0]
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            close()
    if cur:
        close()
    succ = []
    for i, b in enumerate(blocks):
        out = []
        last = b[-1].split() if b else [""]
        op = last[0]
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = last[1]
            if tgt in labels:
                out.append(labels[tgt])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            out.append(i + 1)
        succ.append(out)
    # a label opens a new block even without a preceding branch: map label
    # positions recorded before the block list was final
    return blocks, succ


def _merge(a, b):
    """In-flight queues (oldest first), aligned at the newest entry."""
    n = max(len(a), len(b))
    a = [frozenset()] * (n - len(a)) + list(a)
    b = [frozenset()] * (n - len(b)) + list(b)
    return tuple(x | y for x, y in zip(a, b))[-MAXQ:]


def _step(q, s, report):
    op = s.split()[0]
    if op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", s)
        if m:
            k = int(m.group(1))
            q = q[len(q) - k:] if k < len(q) else q
            if k == 0:
                q = ()
        return q
    pending = frozenset().union(*q) if q else frozenset()
    operands = s.split(None, 1)[1] if " " in s else ""
    hit = _vregs(operands) & pending
    if hit and report is not None:
        report.append((s, sorted(hit)[:4]))
    if op.startswith("ds_read"):
        dst = _vregs(operands.split(",")[0])
        q = (q + (dst,))[-MAXQ:]
    return q


def check_function(items):
    blocks, succ = _blocks(items)
    state = {0: ()}
    work = [0]
    while work:
        i = work.pop()
        q = state[i]
        for s in blocks[i]:
            q = _step(q, s, None)
        for j in succ[i]:
            new = q if j not in state else _merge(state[j], q)
            if j not in state or new != state[j]:
                state[j] = new
                work.append(j)
    bad, reads = [], 0
    for i, b in enumerate(blocks):
        q = state.get(i, ())
        for s in b:
            if s.split()[0].startswith("ds_read"):
                reads += 1
            q = _step(q, s, bad)
    return reads, bad


def _compile_to_asm(src, tmp_path):
    hipcc = _build.hipcc()
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *_build.FLAGS, *_build.EXTRA.get(src, []), "-I", _build.INCLUDE,
           "-I", _build.CSRC, "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_checker_flags_a_use_before_the_wait():
    """The checker itself: a use of an in-flight destination is reported, the
    same use after the matching wait is not, and a wait on a loop back edge is
    seen on the path that takes it."""
    bad_fn = [("inst", "ds_read_b128 v[4:7], v1"), ("inst", "ds_read_b128 v[8:11], v1"),
              ("inst", "s_waitcnt lgkmcnt(1)"), ("inst", "v_mov_b32 v0, v4"),
              ("inst", "v_mov_b32 v0, v9"), ("inst", "s_endpgm")]
    reads, bad = check_function(bad_fn)
    assert reads == 2 and len(bad) == 1 and bad[0][1] == [9]
    loop = [("inst", "s_mov_b32 s0, 0"), ("label", ".LBB0_1"),
            ("inst", "ds_read_b64 v[2:3], v1"), ("inst", "s_cbranch_scc1 .LBB0_2"),
            ("inst", "s_waitcnt lgkmcnt(0)"), ("inst", "s_branch .LBB0_1"),
            ("label", ".LBB0_2"), ("inst", "v_mov_b32 v0, v2"), ("inst", "s_endpgm")]
    _, bad = check_function(loop)
    assert len(bad) == 1  # the exit path leaves the loop without the wait


@pytest.mark.parametrize("src", SOURCES)
def test_no_use_of_an_lds_read_in_flight(src, tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    asm = _compile_to_asm(src, tmp_path)
    funcs = _functions(asm)
    assert funcs, "no kernel found in the listing"
    total = 0
    for name, items in funcs:
        reads, bad = check_function(items)
        total += reads
        assert not bad, f"{name}: {len(bad)} uses of in-flight LDS read registers, e.g. {bad[:3]}"
    assert total > 100
