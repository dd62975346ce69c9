#!/usr/bin/env python3
"""Benchmark of one decode step of the 16-layer Llama-3.2-1B-shaped decoder
at batch 1 (random weights, K/V cache prefilled to 1024 positions), run as
the resident megakernel on one MI355X.

A step is one pass of the whole path: embedding row, 16 x (RMSNorm, QKV,
RoPE + K/V append, GQA attention, O projection + residual, RMSNorm, SiLU-
gated up/gate, down + residual), final norm, tied LM head and greedy argmax.
The timed steps form one greedy chain: each step's token and length feed the
next on the device, with no host synchronisation inside the timed region.

By default the chain runs as resident launches of up to 64 steps each (the
grid stays resident across a launch's steps, mk_decode_steps); the same
chain with one launch per step is timed beside it
(`megakernel_launch_per_step`).

Prints one JSON line. `value` is microseconds per decode step (lower is
better); `roofline` gives the achieved algorithmic HBM bandwidth of the
timed chain against the 8 TB/s peak; `step_us` the 10th, 50th and 90th
percentiles of the per-step time (of single steps with one launch per step;
of each launch's average with resident launches); `read_probe` the read rate
the interpreter's streaming shape reaches on a plain buffer, a second,
achievable peak; `cpu_baseline` times the CPU oracle on consecutive steps of
the same workload; `unfused` times the one-kernel-per-op baseline on the
same chain, and `unfused_graph` that baseline with one step captured in a
HIP graph and replayed per step.

`--workload 1b-layer-kv512` times one 1B-shaped layer instead (hidden
vector in and out): single steps, each after a write that evicts the
memory-side cache the layer's weights would otherwise sit in, with hot-cache
figures beside them.
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


def time_chain(dec, ds, cfg, steps, warmup, torch, per_step=None):
    """Runs warmup + steps chained greedy steps; returns ms per timed step
    (device events around the timed region on the launch stream). With a
    list `per_step`, also records an event between consecutive steps and
    appends each step's ms to it (no host synchronisation in between)."""
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
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps - 1)] if per_step is not None else []
    t0.record(stream)
    for k in range(steps):
        one()
        if marks and k < steps - 1:
            marks[k].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    dec.sync(stream.cuda_stream)
    if per_step is not None:
        bounds = [t0] + marks + [t1]
        per_step.extend(bounds[k].elapsed_time(bounds[k + 1]) for k in range(steps))
    return t0.elapsed_time(t1) / steps


def time_resident(dec, ds, cfg, steps, warmup, torch, per_launch=64, per_step=None):
    """The same greedy chain as resident launches (mk_decode_steps): the
    warmup steps in one untimed launch, then `steps` timed steps in launches
    of up to `per_launch` steps, each launch starting from the previous
    launch's last token (two token buffers alternate; no host
    synchronisation in the timed region). Returns ms per timed step; with a
    list `per_step`, appends each launch's ms per step."""
    stream = torch.cuda.current_stream()
    B = ds.tokens.shape[0]
    rows = max(per_launch, warmup, 1)
    bufs = [torch.zeros((rows, B), dtype=torch.int32, device="cuda") for _ in range(2)]
    bufs[1][rows - 1].copy_(ds.tokens)
    state = {"k": 0, "last": (1, rows - 1)}

    def launch(n):
        src, row = state["last"]
        out = bufs[state["k"] % 2]
        dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=bufs[src][row], tokens_out=out[:n] if n > 1 else out[0], kv_lens_out=ds.kv_lens,
                 n_steps=n, stream=stream.cuda_stream)
        state["last"] = (state["k"] % 2, n - 1)
        state["k"] += 1

    if warmup > 0:
        launch(warmup)
    dec.sync(stream.cuda_stream)
    sizes = [per_launch] * (steps // per_launch) + ([steps % per_launch] if steps % per_launch else [])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k, n in enumerate(sizes):
        launch(n)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    dec.sync(stream.cuda_stream)
    if per_step is not None:
        per_step.extend(ev[k].elapsed_time(ev[k + 1]) / n for k, n in enumerate(sizes))
    ds.tokens.copy_(bufs[state["last"][0]][state["last"][1]])
    return ev[0].elapsed_time(ev[-1]) / steps


def time_graph_chain(dec, ds, cfg, steps, warmup, torch):
    """The same greedy chain with one step captured in a HIP graph and the
    graph replayed per step (the schedule must be the one-kernel-per-op
    baseline: its launches have fixed arguments, and every step's inputs and
    outputs are the same device buffers). Returns ms per timed step."""
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=ds.tokens, tokens_out=ds.tokens, kv_lens_out=ds.kv_lens, stream=side.cuda_stream)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    dec.sync()
    del graph
    return t0.elapsed_time(t1) / steps


def read_probe_gbps(torch, nbytes: int) -> float:
    """Best of three passes of the register-slice read probe (one workgroup
    of 8 waves per compute unit, 4 slices of 4 KiB in flight per wave: the
    interpreter's own streaming shape) over `nbytes` of device memory."""
    from persistent_megakernel_decode_cu_amd import _mk
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = 0.0
    stream = torch.cuda.current_stream()
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        _mk.mk_debug_regstream_probe(src.data_ptr(), nbytes, n_cus, 512, 4, sink.data_ptr())
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, sink
    return best


def gpu_env(device: int = 0) -> dict | None:
    """Socket power, clocks, temperatures and throttle state of the GPU from
    `amd-smi metric --json` (None where the tool is missing or fails)."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", str(device), "--json"], capture_output=True, text=True,
                           timeout=60)
        d = json.loads(r.stdout)
    except Exception:
        return None
    g = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else (d[0] if isinstance(d, list) else d)

    def val(x):
        return x.get("value") if isinstance(x, dict) else None

    clk = g.get("clock", {})
    gfx = [val(v.get("clk")) for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)]
    gfx = [c for c in gfx if isinstance(c, (int, float))]
    first_gfx = next((v for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)), {})
    temp, power = g.get("temperature", {}), g.get("power", {})
    return {"socket_power_w": val(power.get("socket_power")),
            "gfx_clk_mhz_mean": round(sum(gfx) / len(gfx), 1) if gfx else None,
            "gfx_clk_max_mhz": val(first_gfx.get("max_clk")),
            "gfx_clk_locked": first_gfx.get("clk_locked"),
            "mem_clk_mhz": val(clk.get("mem_0", {}).get("clk")) if isinstance(clk.get("mem_0"), dict) else None,
            "hotspot_c": val(temp.get("hotspot")), "mem_c": val(temp.get("mem")),
            "throttle_status": power.get("throttle_status")}


def host_cpu() -> dict:
    """CPU model of the host and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def pct(v, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(v), q)) * 1000.0, 2)


def bench_layer(args, cfg, torch, np, gu, synthetic):
    """One 1B-shaped layer (hidden vector in, hidden vector out, no embedding
    or LM head): repeated single steps, each timed alone with device events.
    Its 123 MB fit in the 256 MB memory-side cache, so before every cold
    iteration a 512 MB scratch write evicts it; hot iterations (no flush)
    are reported beside them."""
    model = synthetic.make_model(cfg)
    st0 = synthetic.make_state(cfg)
    wdev = gu.upload_model(model)
    ds = gu.DevState(st0)
    dec = gu.make_decoder(model, st0, wdev)
    # one step per launch (a layer has no token to hand to a next step), so
    # the default resident mode times the megakernel's single launches
    mode = "megakernel" if args.mode == "resident" else args.mode
    info = dec.build_schedule(1, mode=mode, max_kv_len=int(st0.kv_lens.max()) + 1)
    stream = torch.cuda.current_stream()
    hidden = torch.empty((1, cfg.hidden), dtype=torch.float32, device="cuda")
    kv_out = torch.empty_like(ds.kv_lens)
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")

    def one():
        dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 hidden_in=ds.hidden_in, hidden_out=hidden, kv_lens_out=kv_out, stream=stream.cuda_stream)

    times = {"cold": [], "hot": []}
    for _ in range(args.warmup):
        one()
    for kind in ("cold", "hot"):
        for _ in range(args.steps):
            if kind == "cold":
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            one()
            e1.record(stream)
            torch.cuda.synchronize()
            times[kind].append(e0.elapsed_time(e1))
    dec.sync(stream.cuda_stream)
    dec.close()
    nbytes = algorithmic_bytes(cfg, [int(st0.kv_lens[0])])
    cold_us = pct(times["cold"], 50)
    achieved = nbytes / (cold_us * 1e-6) / 1e9
    out = {
        "metric": "us/decode-step and achieved HBM GB/s (% of peak), 1B-shape batch 1",
        "value": cold_us, "unit": "us/step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(cold_us / 1000.0, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 weights, fp32 compute",
        "data": "synthetic (seeded random-init weights, K/V cache and input vector)",
        "config": {"workload": f"{cfg.name}: one Llama-3.2-1B-shaped layer (H 2048, 32q/8kv x 64, F 8192), "
                               f"batch 1, K/V length {int(st0.kv_lens[0])}, no embedding or LM head; median of "
                               f"{args.steps} single steps, each after a 512 MB cache-evicting write",
                   "mode": mode, "n_cus": info["n_cus"], "launches_per_step": info["launches_per_step"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None, "bytes_per_launch": int(nbytes)},
        "step_us": {"p10": pct(times["cold"], 10), "p50": cold_us, "p90": pct(times["cold"], 90)},
        "hot_cache_step_us": {"p10": pct(times["hot"], 10), "p50": pct(times["hot"], 50),
                              "p90": pct(times["hot"], 90)},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="1b-kv1024")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="resident", choices=["resident", "megakernel", "unfused"],
                    help="resident: the megakernel with the grid resident across up to --per-launch steps "
                         "(mk_decode_steps); megakernel: one launch per step; unfused: one kernel per op")
    ap.add_argument("--per-launch", type=int, default=64, help="steps per resident launch")
    ap.add_argument("--no-gpu-env", action="store_true",
                    help="skip the amd-smi readings (a child process; for runs under a profiler, whose preloaded "
                         "library counts the child's program start as an exec after GPU initialisation)")
    ap.add_argument("--no-launch-per-step", action="store_true",
                    help="with --mode resident, skip the comparison chain of one launch per step")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run the plain copy kernel three times over this many bytes "
                         "(the reference for the rocprofv3 FETCH_SIZE / WRITE_SIZE scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample: consecutive decode steps until this much time has passed")
    ap.add_argument("--no-graph-baseline", action="store_true",
                    help="skip the one-kernel-per-op chain replayed from a captured HIP graph")
    ap.add_argument("--probe-bytes", type=int, default=2 << 30,
                    help="bytes the register-slice read probe streams for the achievable-read-rate figure (0: skip)")
    ap.add_argument("--attn-chunks", type=int, default=0,
                    help="attention tiles per request on average (each kv head gets batch x this many); 0 = auto")
    ap.add_argument("--attn-split", default="balanced", choices=["balanced", "per_request"],
                    help="how each step shares a kv head's attention tiles out over the requests")
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
    from persistent_megakernel_decode_cu_amd import devio as gu

    cfg = synthetic.workload(args.workload)
    if cfg.batch == 1 and not cfg.has_embed:
        bench_layer(args, cfg, torch, np, gu, synthetic)
        return
    chain = args.steps + args.warmup
    B = cfg.batch
    t = time.time()
    model = synthetic.make_model(cfg)
    # every request gets cache pages for the whole chain
    st0 = synthetic.make_state(cfg, extra_positions=max(cfg.steps, chain + 1))
    print(f"# inputs generated in {time.time() - t:.1f} s", file=sys.stderr, flush=True)
    wdev = gu.upload_model(model)
    ds = gu.DevState(st0)
    max_len = int(st0.kv_lens.max()) + chain
    dec = gu.make_decoder(model, st0, wdev)

    split = {"attn_chunks": args.attn_chunks, "attn_split": args.attn_split}
    result_modes = {}
    env = {}
    modes = [args.mode]
    if args.mode == "resident" and not args.no_launch_per_step:
        modes.append("megakernel")
    if not args.no_unfused and args.mode != "unfused":
        modes.append("unfused")
    for mode in modes:
        info = dec.build_schedule(B, mode="megakernel" if mode == "resident" else mode, max_kv_len=max_len, **split)
        ds.kv_lens.copy_(torch.from_numpy(st0.kv_lens))
        ds.tokens.copy_(torch.from_numpy(st0.tokens))
        per_step = []
        if mode == args.mode and not args.no_gpu_env:
            env["before"] = gpu_env()
        if mode == "resident":
            ms = time_resident(dec, ds, cfg, args.steps, args.warmup, torch, args.per_launch, per_step)
        else:
            ms = time_chain(dec, ds, cfg, args.steps, args.warmup, torch, per_step)
        if mode == args.mode and not args.no_gpu_env:
            env["after"] = gpu_env()
        result_modes[mode] = (ms, info, per_step)
        print(f"# {mode}: {ms * 1000:.1f} us/step", file=sys.stderr, flush=True)

    graph_ms = None
    if "unfused" in result_modes and not args.no_graph_baseline:
        dec.build_schedule(B, mode="unfused", max_kv_len=max_len, **split)
        ds.kv_lens.copy_(torch.from_numpy(st0.kv_lens))
        ds.tokens.copy_(torch.from_numpy(st0.tokens))
        graph_ms = time_graph_chain(dec, ds, cfg, args.steps, args.warmup, torch)
        print(f"# unfused, graph-captured: {graph_ms * 1000:.1f} us/step", file=sys.stderr, flush=True)
    ms, info, per_step = result_modes[args.mode]
    bytes_avg = float(np.mean([algorithmic_bytes(cfg, [int(n) + args.warmup + s for n in st0.kv_lens])
                               for s in range(args.steps)]))
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
    if args.mode in ("megakernel", "resident"):
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
        "dtype": ("bf16 weights, fp32 compute" if B <= 4 else
                  "bf16 weights; matvec inputs staged as binary16 and multiplied by packed fp16 dot products "
                  "accumulating in fp32 (padded batch 8); fp32 elsewhere"),
        "data": "synthetic (seeded random-init weights and K/V cache)",
        "config": {"workload": f"{cfg.name}: {cfg.n_layers}-layer Llama-3.2-1B shape (H {cfg.hidden}, "
                               f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}, F {cfg.ffn}, V {cfg.vocab}, "
                               f"tied), batch {B}, K/V length "
                               + (f"{int(st0.kv_lens[0])}" if B == 1 else
                                  f"{int(st0.kv_lens.min())}-{int(st0.kv_lens.max())} (paged)")
                               + ", greedy chain",
                   "mode": args.mode, "n_cus": info["n_cus"],
                   "launches_per_step": (round(1.0 / min(args.per_launch, args.steps), 4) if args.mode == "resident"
                                         else info["launches_per_step"]),
                   "steps_per_launch": min(args.per_launch, args.steps) if args.mode == "resident" else 1,
                   "lds_bytes_per_workgroup": info["lds_bytes"],
                   "attn_tiles_per_kv_head": B * info["attn_chunks"], "attn_split": args.attn_split},
        "hbm_gbps": round(achieved, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "bytes_per_step": int(bytes_avg),
                     "bytes_per_launch": int(bytes_avg * (min(args.per_launch, args.steps)
                                                          if args.mode == "resident" else 1))},
        "step_us": {"p10": pct(per_step, 10), "p50": pct(per_step, 50), "p90": pct(per_step, 90)},
    }
    if args.probe_bytes > 0:
        # the achievable read rate of the interpreter's streaming shape, a
        # second denominator beside the nominal peak
        pg = read_probe_gbps(torch, args.probe_bytes // 4096 * 4096)
        out["read_probe"] = {"gbps": round(pg, 1), "bytes": args.probe_bytes,
                             "frac_of_probe": round(achieved / pg, 4),
                             "shape": "1 workgroup x 8 waves per CU, 4 slices of 4 KiB in flight per wave"}
    if "megakernel" in result_modes and args.mode == "resident":
        mms, _, mper = result_modes["megakernel"]
        out["megakernel_launch_per_step"] = {"us_per_step": round(mms * 1000.0, 2),
                                             "hbm_gbps": round(bytes_avg / (mms * 1e-3) / 1e9, 1),
                                             "step_us": {"p10": pct(mper, 10), "p50": pct(mper, 50),
                                                         "p90": pct(mper, 90)},
                                             "speedup_of_resident": round(mms / ms, 3)}
    if "unfused" in result_modes and args.mode != "unfused":
        ums, uinfo, _ = result_modes["unfused"]
        out["unfused"] = {"us_per_step": round(ums * 1000.0, 2), "launches_per_step": uinfo["launches_per_step"],
                          "hbm_gbps": round(bytes_avg / (ums * 1e-3) / 1e9, 1),
                          "speedup_of_megakernel": round(ums / ms, 3)}
        if graph_ms is not None:
            out["unfused_graph"] = {"us_per_step": round(graph_ms * 1000.0, 2),
                                    "hbm_gbps": round(bytes_avg / (graph_ms * 1e-3) / 1e9, 1),
                                    "speedup_of_megakernel": round(graph_ms / ms, 3)}
    if args.trace_layer >= 0:
        # a separate traced schedule, outside the timed region
        from persistent_megakernel_decode_cu_amd import _mk, trace_summary
        tinfo = dec.build_schedule(B, mode="megakernel", max_kv_len=max_len, trace=True, **split)
        ds.kv_lens.copy_(torch.from_numpy(st0.kv_lens))
        ds.tokens.copy_(torch.from_numpy(st0.tokens))
        for _ in range(3):
            gu.run_step(dec, ds, cfg, want_logits=False)
        plan = _mk.Plan(dec.cfg, _mk.MkScheduleDesc(B, tinfo["n_cus"], 0, max_len, args.attn_chunks, 1, 0,
                                                    {"balanced": 0, "per_request": 1}[args.attn_split], 0))
        text = trace_summary.timeline(dec.trace(), trace_summary.decode_queue(plan.queue), args.trace_layer)
        for line in text.splitlines():
            print(f"# {line}", file=sys.stderr, flush=True)
    out["gpu_env"] = env
    out["host_cpu"] = host_cpu()
    # release the device objects in order while the runtime is intact: the
    # decoder's handle (its schedule buffers and pinned error word), then the
    # tensors it borrowed, then torch's cached blocks
    dec.close()
    del dec, ds, wdev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        # the oracle as it stands (single-threaded fp32 C) on one pinned core,
        # on consecutive greedy steps of the same workload until the sample
        # time has passed
        from oracle import Oracle
        ora = Oracle("f32")
        ost = st0.copy()
        saved = os.sched_getaffinity(0)
        core = min(saved)
        os.sched_setaffinity(0, {core})
        try:
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
        finally:
            os.sched_setaffinity(0, saved)
        hc = out["host_cpu"]
        out["cpu_baseline"] = {"value": round(dt / n * 1e6, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
                               "cpu": hc["model"], "host_cpus": hc["cpu_count"], "pinned_core": core,
                               "sample": f"{n} consecutive greedy decode steps of {cfg.name} from K/V length "
                                         f"{int(st0.kv_lens[0])} (same weights and cache), single-threaded fp32 C "
                                         f"oracle pinned to core {core} of {hc['cpu_count']} ({hc['model']}), "
                                         f"{dt:.1f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
