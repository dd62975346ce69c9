"""Independent checks of an encoded schedule (test helper, CPU only).

Written from the meaning of the queues, not from the C++ builder:

* ``decode``: reads the [S, Q, 32] int32 queues and the event table.
* ``validate``: every op's rows are covered exactly once per layer, every
  attention chunk exists once, each queue is a subsequence of one global
  order, event counts equal their producer counts, and every read-after-
  write, write-after-read and write-after-write pair on every buffer region
  of the step is ordered by the event graph (the instruction that must come
  second transitively waits for the first).
* ``simulate``: runs the queues over many steps with randomised interleavings
  of the compute units against epoch counters (counts only, no math) and
  reports a deadlock with the blocked compute unit and instruction.

The queue word and event layout are read from the library's own header
(mk_isa.h), which defines the encoding.
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
    __slots__ = ("cu", "pc", "op", "layer", "r0", "r1", "b", "g", "c", "nch", "flags", "waits", "pubs", "merge",
                 "slot", "nslot", "seq")

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
            nw, npub = int(w[ISA["W_NWAIT"]]), int(w[ISA["W_NPUB"]])
            i.waits = [int(x) for x in w[ISA["W_WAIT"]: ISA["W_WAIT"] + nw]]
            i.pubs = [int(x) for x in w[ISA["W_PUB"]: ISA["W_PUB"] + npub]]
            i.merge = int(w[ISA["W_MERGE"]])
            i.slot, i.nslot = int(w[ISA["W_SLOT"]]), int(w[ISA["W_NSLOT"]])
            i.seq = int(w[ISA["W_SEQ"]])
            out.append(i)
    return out


class ScheduleError(AssertionError):
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


def validate(shape, batch: int, queue: np.ndarray, events: np.ndarray, attn_chunks: int, max_kv_len: int):
    """Raises ScheduleError on the first violation; returns the decoded list."""
    I = ISA
    ins = decode(queue)
    _req(len(ins) > 0, "empty schedule")
    # global order
    seqs = sorted(i.seq for i in ins)
    _req(seqs == list(range(len(ins))), "W_SEQ values are not a permutation of 0..n-1")
    by_cu = defaultdict(list)
    for i in ins:
        by_cu[i.cu].append(i)
    for cu, lst in by_cu.items():
        for a, b in zip(lst, lst[1:]):
            _req(a.seq < b.seq, f"queue of CU {cu} is not a subsequence of the global order")
    L, H, F = shape.n_layers, shape.hidden, shape.ffn
    nq, nkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    G, QD, QKV = nq // nkv, nq * d, (nq + 2 * nkv) * d
    # coverage
    rows = defaultdict(list)
    attn = defaultdict(list)
    for i in ins:
        if i.op == I["OP_ATTN"]:
            attn[i.layer].append((i.b, i.g, i.c))
            _req(i.nch == attn_chunks, "ATTN instruction with a different chunk count")
        else:
            rows[(i.op, i.layer)].append((i.r0, i.r1))
    for l in range(L):
        _cover(rows[(I["OP_QKV"], l)], QKV, f"QKV layer {l}")
        _cover(rows[(I["OP_OPROJ"], l)], H, f"OPROJ layer {l}")
        _cover(rows[(I["OP_UPGATE"], l)], F, f"UPGATE layer {l}")
        _cover(rows[(I["OP_DOWN"], l)], H, f"DOWN layer {l}")
        want = sorted((b, g, c) for b in range(batch) for g in range(nkv) for c in range(attn_chunks))
        _req(sorted(attn[l]) == want, f"attention tiles of layer {l} incomplete or duplicated")
    if shape.has_embed:
        _cover(rows[(I["OP_LMHEAD"], L)], shape.vocab, "LMHEAD")
    # event producer counts
    ne = events.shape[0]
    producers = defaultdict(set)   # event -> producer node ids ("i<seq>" or "m<event>")
    merge_members = defaultdict(list)
    for i in ins:
        if i.merge >= 0:
            merge_members[i.merge].append(i)
    for i in ins:
        for e in i.pubs:
            _req(0 <= e < ne, "publication of an unknown event")
            producers[e].add(("m", i.merge) if i.merge >= 0 else ("i", i.seq))
    for e in range(ne):
        kind, need = int(events[e, I["EV_KIND"]]), int(events[e, I["EV_NEED"]])
        if kind == I["EVK_MERGE"]:
            mem = merge_members[e]
            _req(len(mem) == need, f"merge event {e}: need {need} but {len(mem)} members")
            _req(all(m.nslot == need for m in mem), f"merge event {e}: slot count mismatch")
            _req(sorted(m.slot for m in mem) == list(range(need)), f"merge event {e}: slots not 0..n-1")
        else:
            _req(len(producers[e]) == need, f"event {e}: need {need} but {len(producers[e])} producers")
    for i in ins:
        for e in i.waits:
            _req(int(events[e, I["EV_KIND"]]) == I["EVK_WAIT"], "instruction waits on a merge counter")
    # reachability over the event graph; merge nodes come after their members
    order = []
    for i in sorted(ins, key=lambda x: x.seq):
        order.append(("i", i.seq, i))
    merge_pos = {m: max(x.seq for x in mem) for m, mem in merge_members.items()}
    nodes = sorted(order + [("m", merge_pos[m] + 0.5, m) for m in merge_members], key=lambda x: x[1])
    node_index = {}
    for k, n in enumerate(nodes):
        node_index[(n[0], n[2].seq if n[0] == "i" else n[2])] = k
    reach = [0] * len(nodes)
    ev_reach = {}

    def event_reach(e):
        if e not in ev_reach:
            r = 0
            for p in producers[e]:
                k = node_index[p]
                r |= reach[k] | (1 << k)
            ev_reach[e] = r
        return ev_reach[e]

    by_seq = {i.seq: i for i in ins}
    for k, n in enumerate(nodes):
        if n[0] == "i":
            r = 0
            for e in n[2].waits:
                r |= event_reach(e)
            reach[k] = r
        else:
            r = 0
            for m in merge_members[n[2]]:
                kk = node_index[("i", m.seq)]
                r |= reach[kk] | (1 << kk)
            reach[k] = r
    # accesses in program order
    accesses = []  # (node_k, buffer, lo, hi, is_write)

    def acc(k, buf, lo, hi, w):
        accesses.append((k, buf, lo, hi, w))

    for k, n in enumerate(nodes):
        if n[0] == "i":
            i = n[2]
            op = i.op
            first = (i.flags & I["F_X_FROM_INPUT"]) != 0
            for b in range(batch):
                if op == I["OP_QKV"]:
                    if first:
                        acc(k, "tokens", b, b + 1, False)
                    else:
                        acc(k, "x", b * H, (b + 1) * H, False)
                    acc(k, "qkv", b * QKV + i.r0, b * QKV + i.r1, True)
                elif op == I["OP_ATTN"]:
                    if b != i.b:
                        continue
                    g = i.g
                    acc(k, "kvlens", b, b + 1, False)
                    for lo in (g * G * d, QD + g * d, QD + nkv * d + g * d):
                        hi = lo + (G * d if lo == g * G * d else d)
                        acc(k, "qkv", b * QKV + lo, b * QKV + hi, False)
                    key = (b * nkv + g) * attn_chunks + i.c
                    acc(k, "part", key, key + 1, True)
                elif op == I["OP_OPROJ"]:
                    acc(k, "o", b * QD, (b + 1) * QD, False)
                    if first:
                        acc(k, "tokens", b, b + 1, False)
                    else:
                        acc(k, "x", b * H + i.r0, b * H + i.r1, False)
                    acc(k, "x", b * H + i.r0, b * H + i.r1, True)
                elif op == I["OP_UPGATE"]:
                    acc(k, "x", b * H, (b + 1) * H, False)
                    acc(k, "act", b * F + i.r0, b * F + i.r1, True)
                elif op == I["OP_DOWN"]:
                    acc(k, "act", b * F, (b + 1) * F, False)
                    acc(k, "x", b * H + i.r0, b * H + i.r1, False)
                    acc(k, "x", b * H + i.r0, b * H + i.r1, True)
                elif op == I["OP_LMHEAD"]:
                    acc(k, "x", b * H, (b + 1) * H, False)
                    acc(k, "lmpart", i.slot * batch + b, i.slot * batch + b + 1, True)
        else:
            m = n[2]
            mem = merge_members[m]
            i0 = mem[0]
            if i0.op == I["OP_ATTN"]:
                b, g = i0.b, i0.g
                base = (b * nkv + g) * attn_chunks
                acc(k, "part", base, base + attn_chunks, False)
                acc(k, "o", b * QD + g * G * d, b * QD + (g + 1) * G * d, True)
            elif i0.op == I["OP_LMHEAD"]:
                acc(k, "lmpart", 0, i0.nslot * batch, False)
                acc(k, "tokens", 0, batch, True)
                acc(k, "kvlens", 0, batch, True)
            elif i0.op == I["OP_DOWN"]:
                acc(k, "kvlens", 0, batch, True)
    # sweep per buffer: sorted segments [start) with (last writer, readers since)
    import bisect
    BIG = 1 << 40
    starts = defaultdict(lambda: [0])
    state = defaultdict(lambda: [[None, set()]])

    def split(buf, x):
        st, sv = starts[buf], state[buf]
        j = bisect.bisect_right(st, x) - 1
        if st[j] != x:
            st.insert(j + 1, x)
            sv.insert(j + 1, [sv[j][0], set(sv[j][1])])

    def ordered(a, b):
        return a is None or a == b or (reach[b] >> a) & 1

    for (k, buf, lo, hi, w) in accesses:
        split(buf, lo)
        split(buf, hi)
        st, sv = starts[buf], state[buf]
        j0 = bisect.bisect_left(st, lo)
        j1 = bisect.bisect_left(st, hi)
        for j in range(j0, j1):
            seg = sv[j]
            if not ordered(seg[0], k):
                raise ScheduleError(f"{buf}[{st[j]}]: access by node {k} not ordered after writer {seg[0]}")
            if w:
                for r in seg[1]:
                    if not ordered(r, k):
                        raise ScheduleError(f"{buf}[{st[j]}]: write by node {k} not ordered after reader {r}")
                seg[0] = k
                seg[1] = set()
            else:
                seg[1].add(k)
    # the block holding the new position belongs to the last chunk
    nb = (max_kv_len + 1 + 15) // 16
    last_blk = nb - 1
    c_last = attn_chunks - 1
    _req((c_last * nb) // attn_chunks <= last_blk < ((c_last + 1) * nb) // attn_chunks,
         "the new K/V position is not in the last chunk")
    return ins


class Deadlock(AssertionError):
    pass


def simulate(queue: np.ndarray, events: np.ndarray, steps: int, seed: int = 0, need_override=None,
             drop_pub=None):
    """Runs `steps` epochs with a random ready-instruction choice at every
    tick. Raises Deadlock naming the blocked compute units when no unit can
    move while some still have work."""
    I = ISA
    ins = decode(queue)
    S = queue.shape[0]
    per_cu = defaultdict(list)
    for i in ins:
        per_cu[i.cu].append(i)
    need = events[:, I["EV_NEED"]].astype(np.int64).copy()
    if need_override:
        for e, v in need_override.items():
            need[e] = v
    ctr_of = events[:, I["EV_CTR"]]
    rng = random.Random(seed)
    counters = np.zeros(int(ctr_of.max()) + 1 if len(ctr_of) else 1, dtype=np.int64)
    for epoch in range(1, steps + 1):
        pc = {cu: 0 for cu in per_cu}
        waiting = defaultdict(list)   # counter -> CUs blocked on it
        ready = []

        def blocked_on(cu):
            lst = per_cu[cu]
            if pc[cu] >= len(lst):
                return None
            for e in lst[pc[cu]].waits:
                if counters[ctr_of[e]] < need[e] * epoch:
                    return e
            return -1

        for cu in per_cu:
            e = blocked_on(cu)
            if e == -1:
                ready.append(cu)
            elif e is not None:
                waiting[ctr_of[e]].append(cu)
        remaining = sum(len(v) for v in per_cu.values())
        while remaining:
            if not ready:
                stuck = []
                for cu in per_cu:
                    if pc[cu] < len(per_cu[cu]):
                        i = per_cu[cu][pc[cu]]
                        stuck.append((cu, pc[cu], [e for e in i.waits if counters[ctr_of[e]] < need[e] * epoch]))
                raise Deadlock(f"step {epoch}: no compute unit can move; blocked (cu, pc, events): {stuck[:8]}")
            k = rng.randrange(len(ready))
            ready[k], ready[-1] = ready[-1], ready[k]
            cu = ready.pop()
            i = per_cu[cu][pc[cu]]
            bumped = []
            if i.merge >= 0:
                c = ctr_of[i.merge]
                counters[c] += 1
                if counters[c] == need[i.merge] * epoch:
                    bumped = [e for e in i.pubs if (i.seq, e) != drop_pub]
            else:
                bumped = [e for e in i.pubs if (i.seq, e) != drop_pub]
            for e in bumped:
                counters[ctr_of[e]] += 1
            pc[cu] += 1
            remaining -= 1
            st = blocked_on(cu)
            if st == -1:
                ready.append(cu)
            elif st is not None:
                waiting[ctr_of[st]].append(cu)
            for e in bumped:
                c = ctr_of[e]
                if waiting[c]:
                    again = waiting.pop(c)
                    for w in again:
                        st = blocked_on(w)
                        if st == -1:
                            ready.append(w)
                        elif st is not None:
                            waiting[ctr_of[st]].append(w)
    return counters
