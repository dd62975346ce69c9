"""Independent checks of an encoded schedule (test helper, CPU only).

Written from the meaning of the queues, not from the C++ builder. In the
resident interpreter an instruction waits until every activation element it
reads carries the step's tag; each element is written once per step by one
producer (a tile, or the elected last finisher of a merge event). So:

* ``decode``: reads the [S, Q, 32] int32 queues and the merge-event table.
* ``validate``: every op's rows are covered exactly once per layer (so every
  element has exactly one producer), every attention tile exists once, the
  merge events have the right members and slots, each queue is a
  subsequence of one global order, and every element an instruction reads is
  produced earlier in that order -- which rules out deadlock: the earliest
  unfinished instruction always heads its compute unit's queue and has all
  its inputs.
* ``simulate``: runs the queues over many steps with randomised interleavings
  of the compute units (readiness only, no math) and reports a deadlock with
  the blocked compute units and instructions.

The queue word layout is read from the library's own header (mk_isa.h),
which defines the encoding.
"""
from __future__ import annotations

import os
import random
import re
from collections import defaultdict

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_ISA = os.path.join(ROOT, "persistent_megakernel_decode_cu_amd", "csrc", "mk_isa.h")


def _isa_constants():
    txt = open(_ISA).read()
    consts = {}
    for name, val in re.findall(r"\b([A-Z][A-Z0-9_]+)\s*=\s*(-?\d+)", txt):
        consts[name] = int(val)
    return consts


ISA = _isa_constants()


class Instr:
    __slots__ = ("cu", "pc", "op", "layer", "r0", "r1", "b", "g", "c", "nch", "flags", "merge", "slot", "nslot",
                 "seq")

    def __repr__(self):
        return f"Instr(cu={self.cu}, pc={self.pc}, op={self.op}, layer={self.layer}, seq={self.seq})"


def decode(queue: np.ndarray):
    out = []
    S, Q, _ = queue.shape
    for cu in range(S):
        for pc in range(Q):
            w = queue[cu, pc]
            if w[ISA["W_OP"]] == ISA["OP_END"]:
                break
            i = Instr()
            i.cu, i.pc = cu, pc
            i.op = int(w[ISA["W_OP"]])
            i.layer = int(w[ISA["W_LAYER"]])
            i.r0, i.r1 = int(w[ISA["W_R0"]]), int(w[ISA["W_R1"]])
            i.b, i.g, i.c, i.nch = (int(w[ISA[k]]) for k in ("W_B", "W_G", "W_C", "W_NCH"))
            i.flags = int(w[ISA["W_FLAGS"]])
            i.merge = int(w[ISA["W_MERGE"]])
            i.slot, i.nslot = int(w[ISA["W_SLOT"]]), int(w[ISA["W_NSLOT"]])
            i.seq = int(w[ISA["W_SEQ"]])
            out.append(i)
    return out


class ScheduleError(AssertionError):
    pass


class Deadlock(AssertionError):
    pass


def _req(cond, msg):
    if not cond:
        raise ScheduleError(msg)


def _cover(intervals, n, what):
    iv = sorted(intervals)
    at = 0
    for lo, hi in iv:
        _req(lo == at, f"{what}: gap or overlap at row {at} (next range starts at {lo})")
        _req(hi > lo, f"{what}: empty range")
        at = hi
    _req(at == n, f"{what}: rows end at {at}, expected {n}")


def _shape(shape):
    L, H, F = shape.n_layers, shape.hidden, shape.ffn
    nq, nkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    return L, H, F, nq, nkv, d, nq // nkv, nq * d, (nq + 2 * nkv) * d


def dependencies(shape, batch: int, ins):
    """Producer nodes of each instruction's inputs, by the data it reads.

    A node is ("i", seq) for a tile or ("m", event) for a merge event's
    elected finisher. Returns {seq: set(nodes)} and the merge members
    {event: [instr]}."""
    I = ISA
    L, H, F, nq, nkv, d, G, QD, QKV = _shape(shape)
    members = defaultdict(list)
    for i in ins:
        if i.merge >= 0:
            members[i.merge].append(i)
    # writers of each buffer region: buffer -> list of (lo, hi, node)
    writers = defaultdict(list)
    for i in ins:
        node = ("i", i.seq)
        for b in range(batch):
            if i.op == I["OP_QKV"]:
                writers[("qkv", i.layer)].append((b * QKV + i.r0, b * QKV + i.r1, node))
            elif i.op == I["OP_OPROJ"]:
                writers[("x", 2 * i.layer + 1)].append((b * H + i.r0, b * H + i.r1, node))
            elif i.op == I["OP_UPGATE"]:
                writers[("act", i.layer)].append((b * F + i.r0, b * F + i.r1, node))
            elif i.op == I["OP_DOWN"]:
                writers[("x", 2 * i.layer + 2)].append((b * H + i.r0, b * H + i.r1, node))
        if i.op == I["OP_ATTN"]:  # one softmax state per (kv head, tile)
            lo = i.g * i.nch + i.c
            writers[("opart", i.layer)].append((lo, lo + 1, node))
        if i.op == I["OP_AMERGE"]:  # the merged outputs of (request, kv head)
            lo = i.b * QD + i.g * G * d
            writers[("o", i.layer)].append((lo, lo + G * d, node))
    for k in writers:
        writers[k].sort()

    def producers(buf, lo, hi):
        out = set()
        covered = lo
        for wlo, whi, node in writers.get(buf, []):
            if whi <= lo or wlo >= hi:
                continue
            _req(wlo <= covered, f"{buf}[{covered}] is read but never written")
            covered = max(covered, whi)
            out.add(node)
        _req(covered >= hi, f"{buf}[{covered}] is read but never written")
        return out

    deps = {}
    for i in ins:
        first = (i.flags & I["F_X_FROM_INPUT"]) != 0
        need = set()
        for b in range(batch):
            if i.op == I["OP_QKV"]:
                if not first:
                    need |= producers(("x", 2 * i.layer), b * H, (b + 1) * H)
            elif i.op == I["OP_ATTN"]:
                # the split decides on the device which request a tile
                # serves: any request's queries and K/V entry of head g
                g = i.g
                for lo, n in ((g * G * d, G * d), (QD + g * d, d), (QD + nkv * d + g * d, d)):
                    need |= producers(("qkv", i.layer), b * QKV + lo, b * QKV + lo + n)
            elif i.op == I["OP_AMERGE"]:  # its request's tiles: any of head g's
                if b != i.b:
                    continue
                need |= producers(("opart", i.layer), i.g * i.nch, (i.g + 1) * i.nch)
            elif i.op == I["OP_OPROJ"]:  # the merged outputs of the request
                need |= producers(("o", i.layer), b * QD, (b + 1) * QD)
                if not first:
                    need |= producers(("x", 2 * i.layer), b * H + i.r0, b * H + i.r1)
            elif i.op == I["OP_UPGATE"]:
                need |= producers(("x", 2 * i.layer + 1), b * H, (b + 1) * H)
            elif i.op == I["OP_DOWN"]:
                need |= producers(("act", i.layer), b * F, (b + 1) * F)
                need |= producers(("x", 2 * i.layer + 1), b * H + i.r0, b * H + i.r1)
            elif i.op == I["OP_LMHEAD"]:
                need |= producers(("x", 2 * L), b * H, (b + 1) * H)
        deps[i.seq] = need
    return deps, members


def validate(shape, batch: int, queue: np.ndarray, events: np.ndarray, attn_chunks: int, max_kv_len: int = 0):
    """Raises ScheduleError on the first violation; returns the decoded list."""
    I = ISA
    ins = decode(queue)
    _req(len(ins) > 0, "empty schedule")
    seqs = sorted(i.seq for i in ins)
    _req(seqs == list(range(len(ins))), "W_SEQ values are not a permutation of 0..n-1")
    by_cu = defaultdict(list)
    for i in ins:
        by_cu[i.cu].append(i)
    for cu, lst in by_cu.items():
        for a, b in zip(lst, lst[1:]):
            _req(a.seq < b.seq, f"queue of CU {cu} is not a subsequence of the global order")
    L, H, F, nq, nkv, d, G, QD, QKV = _shape(shape)
    rows = defaultdict(list)
    attn = defaultdict(list)
    merges = defaultdict(list)
    for i in ins:
        if i.op == I["OP_ATTN"]:
            attn[i.layer].append((i.g, i.c))
            _req(i.nch == batch * attn_chunks, "ATTN instruction with a different tile count")
        elif i.op == I["OP_AMERGE"]:
            merges[i.layer].append((i.b, i.g))
            _req(i.nch == batch * attn_chunks, "AMERGE instruction with a different tile count")
        else:
            rows[(i.op, i.layer)].append((i.r0, i.r1))
    for l in range(L):
        _cover(rows[(I["OP_QKV"], l)], QKV, f"QKV layer {l}")
        _cover(rows[(I["OP_OPROJ"], l)], H, f"OPROJ layer {l}")
        _cover(rows[(I["OP_UPGATE"], l)], F, f"UPGATE layer {l}")
        _cover(rows[(I["OP_DOWN"], l)], H, f"DOWN layer {l}")
        want = sorted((g, c) for g in range(nkv) for c in range(batch * attn_chunks))
        _req(sorted(attn[l]) == want, f"attention tiles of layer {l} incomplete or duplicated")
        want_m = sorted((b, g) for b in range(batch) for g in range(nkv))
        _req(sorted(merges[l]) == want_m, f"attention merges of layer {l} incomplete or duplicated")
    if shape.has_embed:
        _cover(rows[(I["OP_LMHEAD"], L)], shape.vocab, "LMHEAD")
    # merge events
    ne = events.shape[0]
    deps, members = dependencies(shape, batch, ins)
    for e in range(ne):
        _req(int(events[e, I["EV_KIND"]]) == I["EVK_MERGE"], f"event {e} is not a merge event")
        need = int(events[e, I["EV_NEED"]])
        mem = members[e]
        _req(len(mem) == need, f"merge event {e}: need {need} but {len(mem)} members")
        _req(all(m.nslot == need for m in mem), f"merge event {e}: slot count mismatch")
        _req(sorted(m.slot for m in mem) == list(range(need)), f"merge event {e}: slots not 0..n-1")
        ops = {m.op for m in mem}
        _req(len(ops) == 1, f"merge event {e} mixes ops")
        _req(I["OP_ATTN"] not in ops, f"merge event {e} on attention tiles (the O projection merges chunks)")
    for i in ins:
        _req(i.merge < ne, "merge of an unknown event")
        if i.op == I["OP_ATTN"]:
            _req(i.merge < 0, "attention tiles publish their states without a merge event")
            _req(batch <= i.nch <= ISA["MAX_ATTN_TILES"], "attention tile count out of range")
        if i.op == I["OP_LMHEAD"]:
            _req(i.merge >= 0, "LM-head tiles need the argmax merge")
    # every input is produced earlier in the global order
    last_member = {e: max(m.seq for m in mem) for e, mem in members.items()}
    for i in ins:
        for kind, v in deps[i.seq]:
            at = v if kind == "i" else last_member[v]
            _req(at < i.seq, f"instruction {i.seq} (op {i.op}, layer {i.layer}) reads data produced at {at}")
    return ins


def simulate(shape, batch: int, queue: np.ndarray, events: np.ndarray, steps: int, seed: int = 0,
             need_override=None, drop=None):
    """Runs `steps` steps; at every tick one compute unit whose head
    instruction has all its inputs is picked at random and runs it. A merge
    event's output exists once its counter reaches need (per step). `drop`
    names an instruction seq whose outputs are never written (fault
    injection). Raises Deadlock naming the blocked compute units. Returns the
    merge counters after the last step (epoch-style: need * steps)."""
    I = ISA
    ins = decode(queue)
    deps, members = dependencies(shape, batch, ins)
    by_seq = {i.seq: i for i in ins}
    per_cu = defaultdict(list)
    for i in ins:
        per_cu[i.cu].append(i)
    need = events[:, I["EV_NEED"]].astype(np.int64).copy() if len(events) else np.zeros(0, np.int64)
    if need_override:
        for e, v in need_override.items():
            need[e] = v
    dependents = defaultdict(list)   # node -> seqs that read it
    for seq, nodes in deps.items():
        for n in nodes:
            dependents[n].append(seq)
    rng = random.Random(seed)
    counters = np.zeros(max(len(need), 1), dtype=np.int64)
    cus = list(per_cu)
    for step in range(1, steps + 1):
        missing = {seq: len(nodes) for seq, nodes in deps.items()}
        pc = {cu: 0 for cu in cus}
        step_count = defaultdict(int)
        ready = [cu for cu in cus if missing[per_cu[cu][0].seq] == 0]
        in_ready = set(ready)
        remaining = len(ins)

        def complete(node):
            for seq in dependents.get(node, ()):
                missing[seq] -= 1
                if missing[seq] == 0:
                    j = by_seq[seq]
                    if pc[j.cu] < len(per_cu[j.cu]) and per_cu[j.cu][pc[j.cu]].seq == seq and j.cu not in in_ready:
                        ready.append(j.cu)
                        in_ready.add(j.cu)

        while remaining:
            if not ready:
                stuck = [(cu, per_cu[cu][pc[cu]].pc, per_cu[cu][pc[cu]].op) for cu in cus
                         if pc[cu] < len(per_cu[cu])]
                raise Deadlock(f"step {step}: no compute unit can move; blocked (cu, pc, op): {stuck[:8]}")
            k = rng.randrange(len(ready))
            ready[k], ready[-1] = ready[-1], ready[k]
            cu = ready.pop()
            in_ready.discard(cu)
            i = per_cu[cu][pc[cu]]
            pc[cu] += 1
            remaining -= 1
            if i.seq != drop:
                complete(("i", i.seq))
                if i.merge >= 0:
                    counters[i.merge] += 1
                    step_count[i.merge] += 1
                    if step_count[i.merge] == need[i.merge]:
                        complete(("m", i.merge))
            if pc[cu] < len(per_cu[cu]) and missing[per_cu[cu][pc[cu]].seq] == 0 and cu not in in_ready:
                ready.append(cu)
                in_ready.add(cu)
    return counters
