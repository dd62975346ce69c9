"""Static check of the resident interpreter's compiled code (gfx950 ISA).

The weight slices are loaded by inline assembly into registers the compiler
does not allocate (v168 and up: the kernel's occupancy target caps the
compiler below them), and the compiler does not track those loads. Reading a
slot register while its load is in flight would return stale data, so the
code must satisfy, and this check proves on the assembly of every kernel:

1. no compiler-generated instruction names a register at or above the slot
   base; the only instructions that do are the slice loads (marked
   `slot_load`) and the slot copies (`slot_take`);
2. every `slot_take` copy is preceded, on every path from the loads, by a
   `slot_wait` (an s_waitcnt vmcnt) -- checked locally: each run of copies
   follows a wait in the same basic block with no label in between;
3. the kernel descriptor allocates the slot registers;
4. the slice loops (the innermost loops around each slot_wait, found by the
   compiler's loop annotations) hold no compiler-inserted vmcnt wait:
   the compiler does not see the slice loads, so any wait it places there
   for its own loads (a spill reload, say) is a vmcnt(0) that drains every
   slice in flight.

Usage: python -m persistent_megakernel_decode_cu_amd.check_isa file.s ...
"""
from __future__ import annotations

import re
import sys

SLOT_VGPR0 = 168
_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _kernels(lines):
    name, body = None, None
    for l in lines:
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", l)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if l.strip().startswith(".Lfunc_end"):
            yield name, body
            name = None
            continue
        body.append(l)


def check_kernel(body):
    problems = []
    waited = False   # a slot_wait seen in this basic block
    n_load = n_take = 0
    max_compiler = -1
    top_slot = -1
    for i, l in enumerate(body):
        code, _, comment = l.partition(";")
        code = code.strip()
        if re.match(r"^\.LBB\S+:", l) or code.startswith("s_branch") or code.startswith("s_cbranch"):
            waited = False
            continue
        if not code or code.startswith("."):
            continue
        regs = _regs(code)
        if "slot_wait" in comment:
            waited = True
            continue
        if "slot_load" in comment:
            n_load += 1
            top_slot = max([top_slot] + list(_regs(code.split(",")[0])))
            if not code.startswith("buffer_load_dwordx4") or min(_regs(code.split(",")[0])) < SLOT_VGPR0:
                problems.append(f"line {i}: malformed slot load '{code}'")
            continue
        if "slot_take" in comment:
            n_take += 1
            src = _regs(code.split(",", 1)[1])
            if not code.startswith("v_mov_b64") or min(src) < SLOT_VGPR0:
                problems.append(f"line {i}: malformed slot copy '{code}'")
            if not waited:
                problems.append(f"line {i}: slot copy without a preceding slot_wait in its block: '{code}'")
            continue
        if regs:
            hi = max(regs)
            if hi >= SLOT_VGPR0:
                problems.append(f"line {i}: compiler instruction names a slot register: '{code}'")
            max_compiler = max(max_compiler, hi)
    return problems, n_load, n_take, max_compiler, top_slot


def _innermost_header(body, i):
    for j in range(i, -1, -1):
        m = re.search(r"Loop: Header=(BB\S+) Depth=\d+", body[j])
        if m:
            return m.group(1)
        m = re.match(r"^\.L(BB\S+):.*Loop Header: Depth=\d+", body[j])
        if m:
            return m.group(1)
    return None


def slice_loop_waits(body):
    """(loop headers, lines in those loops, [compiler vmcnt waits in them]) for
    every innermost loop that holds a slot_wait (the slice loops)."""
    hdrs = {_innermost_header(body, i) for i, l in enumerate(body) if "slot_wait" in l}
    hdrs.discard(None)
    if not hdrs:
        return None, 0, []
    inloop, n, bad = False, 0, []
    for i, l in enumerate(body):
        m = re.match(r"^\.L(BB\S+):(.*)$", l)
        if m:
            inloop = m.group(1) in hdrs or any(f"Header={h} " in m.group(2) for h in hdrs)
            continue
        if re.match(r"^; %bb\.\d+:", l):
            inloop = any(f"Header={h} " in l for h in hdrs)
            continue
        if inloop:
            n += 1
            if "s_waitcnt" in l and "vmcnt" in l and "slot_wait" not in l:
                bad.append(f"line {i}: compiler vmcnt wait in a slice loop: '{l.strip()}'")
    return sorted(hdrs), n, bad


def _usage(txt):
    """{kernel name: {metadata key: int}} from the code object metadata of an
    assembly file (SGPR count, scratch bytes per lane, ...)."""
    out = {}
    for block in re.split(r"\n\s+- \.", txt):
        m = re.search(r"\.name:\s+(\S+)", block)
        if not m:
            continue
        vals = {k: int(v) for k, v in re.findall(r"\.(\w+):\s+(\d+)\s*$", block, re.M)}
        out[m.group(1)] = vals
    return out


def main(paths):
    bad = 0
    for p in paths:
        txt = open(p).read()
        lines = txt.split("\n")
        counts = {m.group(1): int(m.group(2))
                  for m in re.finditer(r"\.name:\s+(\S+)[\s\S]*?\.vgpr_count:\s+(\d+)", txt)}
        usage = _usage(txt)
        for name, body in _kernels(lines):
            pr, n_load, n_take, mx, top = check_kernel(body)
            _, _, loop_waits = slice_loop_waits(body)
            vg = counts.get(name)
            if n_load and (vg is None or vg <= top):
                pr.append(f"kernel allocates {vg} VGPRs, not covering slot register v{top}")
            u = usage.get(name, {})
            n_spill = sum(1 for l in body if re.match(r"^\s+scratch_(load|store)", l))
            print(f"{p}: {name}: {n_load} slot loads, {n_take} slot copies, compiler VGPRs <= v{mx}, "
                  f"{vg} allocated: {len(pr)} problems, {len(loop_waits)} slice-loop waits; "
                  f"{u.get('sgpr_count', '?')} SGPRs, {u.get('private_segment_fixed_size', '?')} bytes of scratch "
                  f"per lane, {n_spill} spill instructions")
            for x in pr[:10]:
                print("   ", x)
            bad += len(pr)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
