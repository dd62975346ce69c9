"""Per-layer timeline of one traced decode step of the resident interpreter.

A schedule built with trace = 1 makes every instruction record device-clock
stamps (the 100 MHz wall clock): start, inputs staged (ready), end, first and
last wave done. `timeline` aggregates them over the compute units that run
each op of one layer, and over the whole step, into a short text table:
medians and extremes of when an op's tiles became ready and ended, relative
to the step's first stamp, and the tail, the spread between the first and
the last compute unit to finish the step.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np

CLOCK_MHZ = 100.0  # wall_clock64 ticks per microsecond
TR_START, TR_READY, TR_END, TR_FIRST, TR_LAST = 0, 1, 2, 3, 4
# queue encoding of csrc/mk_isa.h: the words a timeline needs, and the op names
W_OP, W_LAYER = 0, 1
OP_END = 0
OP_NAMES = {1: "QKV", 2: "ATTN", 3: "OPROJ", 4: "UPGATE", 5: "DOWN", 6: "LMHEAD", 7: "AMERGE"}


class Instr(NamedTuple):
    cu: int
    pc: int
    op: int
    layer: int


def decode_queue(queue: np.ndarray) -> list:
    """Instructions of encoded queues [n_cus, Q, 32] int32, up to each
    queue's END word."""
    out = []
    for cu in range(queue.shape[0]):
        for pc in range(queue.shape[1]):
            op = int(queue[cu, pc, W_OP])
            if op == OP_END:
                break
            out.append(Instr(cu, pc, op, int(queue[cu, pc, W_LAYER])))
    return out


def timeline(trace: np.ndarray, instrs, layer: int, op_names: dict = OP_NAMES) -> str:
    """trace: int64 [n_cus, Q, words]; instrs: decoded instructions (cu, pc,
    op, layer); op_names: opcode -> name."""
    rows = {}
    stamps = []
    last_end = {}
    for i in instrs:
        s = trace[i.cu, i.pc].astype(np.int64)
        if s[TR_START] <= 0:
            continue
        stamps.append(s[TR_START])
        last_end[i.cu] = max(last_end.get(i.cu, 0), int(s[TR_END]))
        if i.layer == layer:
            rows.setdefault(i.op, []).append(s)
    if not stamps:
        return "no stamps recorded\n"
    t0 = min(stamps)

    def us(x):
        return (float(x) - t0) / CLOCK_MHZ

    out = [f"layer {layer}: times in us from the step's first stamp (medians over the op's tiles)",
           f"{'op':8s} {'tiles':>5s} {'ready min':>10s} {'ready med':>10s} {'ready max':>10s} "
           f"{'end med':>10s} {'end max':>10s} {'ready->first':>13s}"]
    order = sorted(rows, key=lambda op: np.median([r[TR_READY] for r in rows[op]]))
    for op in order:
        a = np.stack(rows[op])
        rd, en, fi = a[:, TR_READY], a[:, TR_END], a[:, TR_FIRST]
        out.append(f"{op_names.get(op, str(op)):8s} {len(a):5d} {us(rd.min()):10.1f} {us(np.median(rd)):10.1f} "
                   f"{us(rd.max()):10.1f} {us(np.median(en)):10.1f} {us(en.max()):10.1f} "
                   f"{np.median(fi - rd) / CLOCK_MHZ:13.2f}")
    ends = np.array(sorted(last_end.values()), dtype=np.int64)
    out.append(f"step: last stamp {us(ends.max()):.1f} us; compute units finish between "
               f"{us(ends.min()):.1f} and {us(ends.max()):.1f} us (tail {(ends.max() - ends.min()) / CLOCK_MHZ:.1f} us, "
               f"median {us(np.median(ends)):.1f})")
    return "\n".join(out) + "\n"
