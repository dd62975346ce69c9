#!/usr/bin/env python3
"""Benchmark of one decode step of the 16-layer Llama-3.2-1B-shaped decoder
at batch 1 (random weights, K/V cache prefilled to 1024 positions), run as
the resident megakernel on one MI355X.

A step is one pass of the whole path: embedding row, 16 x (RMSNorm, QKV,
RoPE + K/V append, GQA attention, O projection + residual, RMSNorm, SiLU-
gated up/gate, down + residual), final norm, tied LM head and greedy argmax.
The timed steps form one greedy chain: each step's token and length feed the
next on the device, with no host synchronisation inside the timed region.

Prints one JSON line. `value` is microseconds per decode step (lower is
better); `roofline` gives the achieved algorithmic HBM bandwidth of the
megakernel launch against the 8 TB/s peak; `cpu_baseline` times the CPU
oracle on one full step of the same workload; `unfused` times the
one-kernel-per-op baseline on the same chain.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0


def algorithmic_bytes(cfg, kv_lens) -> int:
    """Bytes a step must move at least once: every weight, every cached K/V
    entry it attends to (positions 0..len_b, the new one included), and the
    appended entry."""
    L, H, F, d = cfg.n_layers, cfg.hidden, cfg.ffn, cfg.head_dim
    nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
    per_layer = 2 * ((nq + 2 * nkv) * d * H + nq * d * H + 3 * H * F) + 4 * H
    total = L * per_layer
    if cfg.has_embed:
        total += 2 * cfg.vocab * H + 2 * H + 2 * H * len(kv_lens)
    for n in kv_lens:
        total += L * (int(n) + 1) * 4 * nkv * d
    total += len(kv_lens) * L * 4 * nkv * d
    return total


def time_chain(dec, ds, cfg, steps, warmup, torch):
    """Runs warmup + steps chained greedy steps; returns ms per timed step
    (device events around the timed region on the launch stream)."""
    stream = torch.cuda.current_stream()
    tokens = ds.tokens
    kv = ds.kv_lens

    def one():
        dec.step(kv_lens=kv, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=tokens, tokens_out=tokens, kv_lens_out=kv, stream=stream.cuda_stream)

    for _ in range(warmup):
        one()
    dec.sync(stream.cuda_stream)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        one()
    t1.record(stream)
    torch.cuda.synchronize()
    dec.sync(stream.cuda_stream)
    return t0.elapsed_time(t1) / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="1b-kv1024")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="megakernel", choices=["megakernel", "unfused"])
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run the plain copy kernel three times over this many bytes "
                         "(the reference for the rocprofv3 FETCH_SIZE / WRITE_SIZE scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample: consecutive decode steps until this much time has passed")
    ap.add_argument("--trace-layer", type=int, default=-1,
                    help="after timing, run three untimed steps of a traced megakernel schedule and print the "
                         "per-op timeline of this layer to stderr")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the decode step is measured on one MI355X); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    from tests import gpu_util as gu

    cfg = synthetic.workload(args.workload)
    chain = args.steps + args.warmup
    if cfg.batch != 1 or chain > cfg.steps:
        print(f"workload {cfg.name}: batch {cfg.batch}, {cfg.steps}-step chain; need batch 1 and "
              f"warmup + steps <= {cfg.steps}", file=sys.stderr)
        sys.exit(2)
    t = time.time()
    model = synthetic.make_model(cfg)
    st0 = synthetic.make_state(cfg)
    print(f"# inputs generated in {time.time() - t:.1f} s", file=sys.stderr, flush=True)
    wdev = gu.upload_model(model)
    ds = gu.DevState(st0)
    max_len = int(st0.kv_lens.max()) + chain
    dec = gu.make_decoder(model, st0, wdev)

    result_modes = {}
    modes = [args.mode] + ([] if args.no_unfused or args.mode == "unfused" else ["unfused"])
    for mode in modes:
        info = dec.build_schedule(1, mode=mode, max_kv_len=max_len)
        ds.kv_lens.copy_(torch.from_numpy(st0.kv_lens))
        ds.tokens.copy_(torch.from_numpy(st0.tokens))
        ms = time_chain(dec, ds, cfg, args.steps, args.warmup, torch)
        result_modes[mode] = (ms, info)
        print(f"# {mode}: {ms * 1000:.1f} us/step", file=sys.stderr, flush=True)

    ms, info = result_modes[args.mode]
    lens_timed = [int(st0.kv_lens[0]) + args.warmup + s for s in range(args.steps)]
    bytes_avg = float(np.mean([algorithmic_bytes(cfg, [n]) for n in lens_timed]))
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    if args.copy_bytes > 0:
        from persistent_megakernel_decode_cu_amd import _mk
        n = args.copy_bytes // 16 * 16
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            _mk.mk_debug_copy_probe(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        del src, dst
    # HBM traffic per launch, measured with rocprofv3 counters (see the summary
    # file); reported only while the kernel sources are the ones it was taken on
    traffic = None
    if args.mode == "megakernel":
        from persistent_megakernel_decode_cu_amd import profile_summary
        rec = profile_summary.read_traffic(os.path.join(ROOT, "profiles", f"traffic_megakernel_{cfg.name}.txt"))
        if rec is not None and rec[1] == profile_summary.digest():
            traffic = int(rec[0])
    out = {
        "metric": "us/decode-step and achieved HBM GB/s (% of peak), 1B-shape batch 1",
        "value": round(ms * 1000.0, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights, fp32 compute",
        "data": "synthetic (seeded random-init weights and K/V cache)",
        "config": {"workload": f"{cfg.name}: 16-layer Llama-3.2-1B shape (H 2048, 32q/8kv x 64, F 8192, "
                               f"V 128256, tied), batch 1, K/V length {int(st0.kv_lens[0])}, greedy chain",
                   "mode": args.mode, "n_cus": info["n_cus"], "launches_per_step": info["launches_per_step"]},
        "hbm_gbps": round(achieved, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": int(bytes_avg)},
    }
    if "unfused" in result_modes and args.mode != "unfused":
        ums, uinfo = result_modes["unfused"]
        out["unfused"] = {"us_per_step": round(ums * 1000.0, 2), "launches_per_step": uinfo["launches_per_step"],
                          "hbm_gbps": round(bytes_avg / (ums * 1e-3) / 1e9, 1),
                          "speedup_of_megakernel": round(ums / ms, 3)}
    if args.trace_layer >= 0:
        # a separate traced schedule, outside the timed region
        from persistent_megakernel_decode_cu_amd import _mk, trace_summary
        from tests import sched_check
        tinfo = dec.build_schedule(1, mode="megakernel", max_kv_len=max_len, trace=True)
        ds.kv_lens.copy_(torch.from_numpy(st0.kv_lens))
        ds.tokens.copy_(torch.from_numpy(st0.tokens))
        for _ in range(3):
            gu.run_step(dec, ds, cfg, want_logits=False)
        plan = _mk.Plan(dec.cfg, _mk.MkScheduleDesc(1, tinfo["n_cus"], 0, max_len, 0, 1, 0, 0, 0))
        names = {v: k[3:] for k, v in sched_check.ISA.items() if k.startswith("OP_") and k not in ("OP_END", "OP_COUNT")}
        text = trace_summary.timeline(dec.trace(), sched_check.decode(plan.queue), names, args.trace_layer)
        for line in text.splitlines():
            print(f"# {line}", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        # the oracle as it stands (single-threaded fp64 C), on consecutive greedy
        # steps of the same workload until the sample time has passed
        from oracle import Oracle
        ora = Oracle("f64")
        ost = st0.copy()
        n, t = 0, time.time()
        while True:
            r = ora.decode_step(model, ost)
            assert r["rc"] == 0
            ost.tokens[:] = r["tokens"]
            ost.kv_lens += 1
            n += 1
            dt = time.time() - t
            if dt >= args.cpu_seconds or n >= 64:
                break
        out["cpu_baseline"] = {"value": round(dt / n * 1e6, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
                               "sample": f"{n} consecutive greedy decode steps of {cfg.name} from K/V length "
                                         f"{int(st0.kv_lens[0])} (same weights and cache), single-threaded fp64 C "
                                         f"oracle, {dt:.1f} s"}
    dec.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
