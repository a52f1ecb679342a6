"""The v_dot2_f32_bf16 result hazard, checked on the compiled gfx950 code.

The library issues v_dot2_f32_bf16 from inline assembly (`dot2_bf16` in
csrc/common.h).  The hardware does not interlock its result: another VALU
instruction that reads the result register, other than as the accumulator of
the next v_dot2 of a chain, must come at least three instructions later, and
the compiler does not insert those wait states for an instruction it only sees
as inline assembly.  A read one instruction later was seen to return the value
from before the dot.

This test compiles every source that uses `dot2_bf16` to gfx950 assembly with
the library's own flags (cached under `_build/asm_scan`, redone when a source
or csrc/common.h changes) and walks, from each v_dot2, every path through the
following instructions (fall-through and branch targets) until the result
register is overwritten, chained as an accumulator, or three instructions have
passed.  Any earlier read fails the test.  It needs only the compiler.
"""

import hashlib
import os
import re
import subprocess

import pytest

from block_sparse_spatiotemporal_build_amd import build as bb

WAIT_STATES = 3
CACHE = os.path.join(bb.BUILD_DIR, "asm_scan")


def _dot_sources():
    out = []
    for src in bb.sources():
        with open(src) as f:
            if "dot2_bf16(" in f.read():
                out.append(src)
    return out


def _asm(src):
    h = hashlib.sha256()
    for p in (src, os.path.join(bb.CSRC, "common.h"), os.path.join(bb.CSRC, "launch.h")):
        if os.path.exists(p):
            with open(p, "rb") as f:
                h.update(f.read())
    h.update(" ".join(bb.FLAGS).encode())
    os.makedirs(CACHE, exist_ok=True)
    path = os.path.join(CACHE, f"{os.path.basename(src)[:-4]}_{h.hexdigest()[:16]}.s")
    if not os.path.exists(path):
        tmp = path + ".tmp"
        cmd = [bb.HIPCC, *bb.FLAGS, "--cuda-device-only", "-S", src, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        os.replace(tmp, path)
    with open(path) as f:
        return f.read()


def _parse(text):
    """Instructions (mnemonic, operand list, source line) and label -> index."""
    insts, labels = [], {}
    for n, raw in enumerate(text.split("\n"), 1):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            labels[line[:-1]] = len(insts)
            continue
        if line.startswith("."):
            continue
        op, _, rest = line.partition(" ")
        ops = [o.strip() for o in rest.split(",")] if rest else []
        insts.append((op, ops, n))
    return insts, labels


def _regs(operand):
    """VGPR indices an operand names (v7, v[4:7])."""
    m = re.fullmatch(r"v(\d+)", operand.split()[0] if operand else "")
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand.split()[0] if operand else "")
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _writes_and_reads(op, ops):
    if not op.startswith(("v_", "ds_", "buffer_", "global_", "flat_", "scratch_")):
        return set(), set().union(*[_regs(o) for o in ops]) if ops else set()
    if op.startswith(("ds_write", "buffer_store", "global_store", "flat_store", "scratch_store")) or op.startswith("v_cmp"):
        return set(), set().union(*[_regs(o) for o in ops]) if ops else set()
    dst = _regs(ops[0]) if ops else set()
    src = set().union(*[_regs(o) for o in ops[1:]]) if len(ops) > 1 else set()
    return dst, src


def _violations(text):
    insts, labels = _parse(text)
    bad = []
    for i, (op, ops, line) in enumerate(insts):
        if op != "v_dot2_f32_bf16":
            continue
        reg = _regs(ops[0])
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, dist = stack.pop()
            if dist >= WAIT_STATES or j >= len(insts) or (j, dist) in seen:
                continue
            seen.add((j, dist))
            op2, ops2, line2 = insts[j]
            if op2 == "s_nop":
                stack.append((j + 1, dist + int(ops2[0], 0) + 1))
                continue
            if op2 == "v_dot2_f32_bf16" and _regs(ops2[-1]) == reg and not (reg & (_regs(ops2[1]) | _regs(ops2[2]))):
                continue  # chained as the accumulator
            w, r = _writes_and_reads(op2, ops2)
            if reg & r:
                bad.append((line, line2, dist, f"{op} {', '.join(ops)}", f"{op2} {', '.join(ops2)}"))
                continue
            if reg <= w:
                continue  # overwritten
            if op2 in ("s_endpgm", "s_setpc_b64"):
                continue
            if op2.startswith("s_cbranch") or op2 == "s_branch":
                tgt = labels.get(ops2[0])
                if tgt is not None:
                    stack.append((tgt, dist + 1))
                if op2 == "s_branch":
                    continue
            stack.append((j + 1, dist + 1))
    return bad


def test_scanner_flags_a_read_that_comes_too_soon():
    text = "\n".join([
        "k:",
        "\tv_dot2_f32_bf16 v10, v1, v2, v3",
        "\tv_dot2_f32_bf16 v10, v4, v2, v10",  # accumulator chain: fine
        "\ts_nop 0",
        "\tv_add_f32_e32 v11, v11, v10",       # one wait state after the chain's last dot
        "\tv_dot2_f32_bf16 v12, v1, v2, v3",
        "\ts_nop 2",
        "\tv_add_f32_e32 v11, v11, v12",       # three: fine
        "\tv_dot2_f32_bf16 v13, v1, v2, v3",
        "\ts_cbranch_scc1 L",
        "\tv_mov_b32_e32 v14, v13",            # fall-through, distance 1
        "L:",
        "\tv_mov_b32_e32 v15, v13",            # branch target, distance 1
        "\ts_endpgm",
    ])
    bad = _violations(text)
    assert sorted((b[2], b[4].split()[0]) for b in bad) == [(1, "v_add_f32_e32"), (1, "v_mov_b32_e32"),
                                                           (1, "v_mov_b32_e32")]


@pytest.mark.parametrize("src", _dot_sources(), ids=os.path.basename)
def test_no_dot2_result_read_too_soon(src):
    bad = _violations(_asm(src))
    assert not bad, "\n".join(f"line {a} -> {b} at distance {d}: {x}  ->  {y}" for a, b, d, x, y in bad[:10])
