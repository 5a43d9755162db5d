"""Compiled-code checks of the split kernels (gfx950 assembly, no GPU).

1. A matrix-core read hazard.

A vector-ALU instruction that reads the result of a v_mfma must issue a
number of wait states after it.  The compiler pads this inside a basic block,
but a read placed right after a taken branch (for instance the uniform
ragged-block branch of the softmax) has been seen to get no padding and to
read a stale accumulator.  This test compiles the fused kernels to gfx950
assembly and checks every branch: MFMA results written in the instructions
before a branch must not be read at its target sooner than the distance the
compiler itself keeps within blocks.

2. Explicit load waits.  The query and register-staged mask loads are inline
assembly waited for with explicit vmcnt counts, because the compiler's own
wait for them would also wait for the block loads issued after them.  The
compiler therefore cannot protect their registers: this check follows the
in-order vmcnt queue through each kernel (along fall-through and forward
branches) and fails if any instruction touches a register whose load may
still be outstanding.
"""
import collections
import os
import re
import shutil
import subprocess

import pytest

from gqa_decode_attention_fr_amd import build as B

SRC = os.path.join(B.CSRC, "fr_fused.hip")


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _wait_states(line):
    m = re.match(r"s_nop (\d+)", line)
    return int(m.group(1)) + 1 if m else 1


def _sources(line):
    """VGPRs an instruction reads (destination dropped for ALU ops and loads)."""
    parts = line.split(None, 1)
    ops = parts[1].split(",") if len(parts) > 1 else []
    if line.startswith(("v_", "ds_read", "global_load", "buffer_load")):
        ops = ops[1:]
    return _regs(",".join(ops))


def _functions(asm):
    for name, body in re.findall(r"^(_ZN2fr\S*split_kernel\S*):[^\n]*\n(.*?)\.Lfunc_end", asm,
                                 re.S | re.M):
        lines = [l.strip() for l in body.splitlines()
                 if (l.startswith("\t") and not l.strip().startswith((".", ";")))
                 or l.startswith(".LBB")]
        yield name, lines


def _within_block_minimum(funcs):
    """Smallest distance the compiler leaves between an MFMA and a VALU read
    of its result inside one basic block."""
    seen = collections.Counter()
    for _, lines in funcs:
        for i, l in enumerate(lines):
            if not l.startswith("v_mfma"):
                continue
            dst = _regs(l.split()[1].rstrip(","))
            ws = 0
            for lk in lines[i + 1:i + 40]:
                if lk.startswith((".LBB", "s_cbranch", "s_branch")):
                    break
                if lk.startswith("v_") and not lk.startswith("v_mfma"):
                    if _sources(lk) & dst:
                        seen[ws] += 1
                        break
                    if _regs(lk.split(None, 1)[1].split(",")[0]) & dst:
                        break
                if lk.startswith("v_mfma") and _regs(lk.split()[1].rstrip(",")) & dst:
                    break
                ws += _wait_states(lk)
    return min(seen) if seen else None


def _violations(funcs, need):
    bad = []
    for name, lines in funcs:
        labels = {l.split(":")[0]: i for i, l in enumerate(lines) if l.startswith(".LBB")}
        for i, l in enumerate(lines):
            m = re.match(r"s_cbranch_\w+\s+(\.LBB\S+)|s_branch\s+(\.LBB\S+)", l)
            if not m:
                continue
            pend, ws = [], 0
            for j in range(i - 1, max(i - 24, -1), -1):
                if lines[j].startswith(".LBB"):
                    break
                if lines[j].startswith("v_mfma"):
                    pend.append((_regs(lines[j].split()[1].rstrip(",")), ws))
                ws += _wait_states(lines[j])
            if not pend:
                continue
            ws2 = 1  # the branch
            for lk in lines[labels[m.group(1) or m.group(2)] + 1:]:
                if lk.startswith(".LBB"):
                    continue
                if not lk.startswith(("v_mfma", "s_")):
                    src = _sources(lk)
                    for regs, w0 in pend:
                        if regs & src and w0 + ws2 < need:
                            bad.append(f"{name}: '{lk}' {w0 + ws2} wait states after its MFMA")
                ws2 += _wait_states(lk)
                if ws2 >= need:
                    break
    return bad


@pytest.fixture(scope="module")
def fused_asm(tmp_path_factory):
    cc = B.hipcc()
    if not shutil.which(cc) and not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "fr_fused.s"
    subprocess.run([cc, *B.compile_flags(), "--cuda-device-only", "-S", SRC, "-o", str(out)],
                   check=True, capture_output=True)
    return out.read_text()


def test_no_mfma_result_read_right_after_a_branch(fused_asm):
    funcs = list(_functions(fused_asm))
    assert len(funcs) >= 9, "split kernels not found in the assembly"
    need = _within_block_minimum(funcs)
    if need is None:
        # every read of an MFMA result follows a branch (the scores' reads sit
        # after the uniform ragged-block branches of the accumulator start):
        # take the distance the compiler keeps inside blocks for these 4-pass
        # MFMAs where such a pair exists, 8 wait states
        need = 8
    assert need >= 4
    bad = _violations(funcs, need)
    assert not bad, "\n".join(bad[:10])


def _step(queue, l, bad, name):
    """One instruction of the in-order vmcnt queue (destination register sets of
    the outstanding vector-memory operations, oldest first)."""
    op = l.split()[0]
    m = re.match(r"s_waitcnt.*vmcnt\((\d+)\)", l)
    if m:
        del queue[:max(0, len(queue) - int(m.group(1)))]
        return
    ops = l.split(None, 1)[1] if len(l.split(None, 1)) > 1 else ""
    pending = set().union(*queue) if queue else set()
    if op.startswith(("global_load", "buffer_load")) and "lds" not in op:
        if _regs(ops) & pending:
            bad.append(f"{name}: '{l}'")
        queue.append(_regs(ops.split(",")[0]))
    elif op.startswith(("global_load_lds", "global_store", "buffer_store", "global_atomic")):
        if _regs(ops) & pending:
            bad.append(f"{name}: '{l}'")
        queue.append(set())
    elif op.startswith(("v_", "ds_")) and _regs(ops) & pending:
        bad.append(f"{name}: '{l}'")


def _merge(a, b):
    """Queues reaching one point along two paths, aligned at their newest entry."""
    n = max(len(a), len(b))
    out = []
    for k in range(n, 0, -1):
        s = set()
        if k <= len(a):
            s |= a[-k]
        if k <= len(b):
            s |= b[-k]
        out.append(s)
    return out


def _outstanding_register_uses(funcs):
    """Walks each kernel in layout order, along the fall-through path (the
    waits the kernels take under complementary uniform conditions, such as
    "the next block, or all", sit on consecutive fall-through blocks).  A block
    that can only be entered by a jump (it follows an unconditional branch)
    starts from the merged queues of the earlier forward branches to it, or
    empty.  Loop back edges are not followed."""
    bad = []
    for name, lines in funcs:
        queue = []
        at_label = {}   # label -> merged queue of the forward branches seen to it
        falls = True    # the previous instruction can fall through
        for l in lines:
            if l.startswith(".LBB"):
                lab = l.split(":")[0]
                seen = at_label.get(lab)
                if not falls:
                    queue = [set(x) for x in seen] if seen is not None else []
                falls = True
                continue
            op = l.split()[0]
            m = re.match(r"s_c?branch\w*\s+(\.LBB\S+)", l)
            if m:
                lab = m.group(1)
                prev = at_label.get(lab)
                at_label[lab] = [set(x) for x in queue] if prev is None else _merge(prev, queue)
                falls = op != "s_branch"
                continue
            if op == "s_endpgm":
                falls = False
                continue
            _step(queue, l, bad, name)
    return bad


def test_no_register_use_before_its_load_wait(fused_asm):
    funcs = list(_functions(fused_asm))
    bad = _outstanding_register_uses(funcs)
    assert not bad, "\n".join(bad[:10])
