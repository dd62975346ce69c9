"""Latency of one grid-wide dependency hop, the measurement behind the
resident interpreter's choice of data-tagged exchanges over fenced counters.

A cooperative grid of one one-wave workgroup per compute unit runs R rounds;
in each, every workgroup waits for every other's previous round, exchanges
its share of a vector and signals. Kernel time / R is one hop on the
critical path. Three protocols:

  fenced counter     a shared counter per round; agent-scope release fence
                     before the increment, acquire fence after the wait
                     (the page's counter protocol: "Inference MegaKernel",
                     section "hand-written whole-model MegaKernel /
                     principle, schedule and dataflow");
  counter, no fences the same with device-coherent data accesses instead
                     of the fences;
  tagged words       no counter: every value travels with its round number
                     in one 64-bit word and readers poll the data itself.

    python -m persistent_megakernel_decode_cu_amd.hop_latency [--rounds N]
"""
from __future__ import annotations

import argparse
import sys

import torch

from . import _mk


def _time(fn, rounds):
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / rounds


def measure(n_cus: int, rounds: int, reps: int = 3) -> list:
    lib = _mk.lib()
    groups = (n_cus + 15) // 16
    ctr_words = max((rounds + 1) * 32, (17 + groups) * 1024)
    x_floats = 2 * ((n_cus * 8 + 31) // 32) * 1024
    rows = []
    for name, variant, per in (("fenced counter, 8 floats/WG", 0b000100, 8),
                               ("counter without fences, 8 floats/WG", 0b000111, 8),
                               ("tagged words, 8 floats/WG", None, 8),
                               ("tagged words, 32 floats/WG", None, 32)):
        best = None
        for _ in range(reps):
            res = torch.zeros(4, dtype=torch.int32, device="cuda")
            if variant is not None:
                ctr = torch.zeros(ctr_words, dtype=torch.int32, device="cuda")
                xb = torch.zeros(x_floats, dtype=torch.float32, device="cuda")
                us = _time(lambda: _mk._check(lib.mk_debug_hop_probe(ctr.data_ptr(), ctr_words, xb.data_ptr(),
                                                                     x_floats, n_cus, rounds, variant,
                                                                     res.data_ptr())), rounds)
            else:
                words = 2 * n_cus * per
                buf = torch.zeros(words, dtype=torch.int64, device="cuda")
                us = _time(lambda: _mk._check(lib.mk_debug_ll_probe(buf.data_ptr(), words, n_cus, per, 1, rounds,
                                                                    res.data_ptr())), rounds)
            if int(res.cpu()[0]) != 0:
                raise RuntimeError(f"{name}: {int(res.cpu()[0])} watchdog expiries")
            best = us if best is None else min(best, us)
        rows.append((name, best))
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--rounds", type=int, default=2000)
    args = ap.parse_args(argv)
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"grid-wide hop latency, {n_cus} one-wave workgroups (cooperative launch), {args.rounds} rounds, "
          f"best of 3")
    for name, us in measure(n_cus, args.rounds):
        print(f"  {name:40s} {us:7.2f} us per hop")
    return 0


if __name__ == "__main__":
    sys.exit(main())
