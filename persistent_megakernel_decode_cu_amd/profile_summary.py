"""Text summaries of rocprofv3 result databases (SQLite), for the figures the
benchmark reports: per-kernel launch statistics from a --kernel-trace run,
and HBM traffic per launch from two --pmc runs (FETCH_SIZE, WRITE_SIZE),
each scaled by what the same counter reads for the plain copy kernel
mk_copy_probe of a known size.

    python -m persistent_megakernel_decode_cu_amd.profile_summary stats DB --command "..."
    python -m persistent_megakernel_decode_cu_amd.profile_summary traffic --fetch DB --write DB \\
        --kernel mk_megakernel --copy-bytes N --command "..." --command "..."
    python -m persistent_megakernel_decode_cu_amd.profile_summary counters DB [DB ...] --command "..."

`digest()` fingerprints the kernel sources' code (comments and blank lines
left out, so that a comment edit does not disown a measurement); a traffic
summary records it, so that a reader can tell whether the kernels changed
after the counters were taken.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import os
import re
import sqlite3
import statistics
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)


def _code(text: str) -> str:
    """The source without its comments, trailing blanks and blank lines (the
    sources hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def digest() -> str:
    """sha256 over the code of the HIP/C++ sources and the public header, in
    name order, and the compiler flags that shape the kernels (without the
    include paths, which differ between machines)."""
    h = hashlib.sha256()
    if __package__:
        from . import build
    else:  # run as a script
        sys.path.insert(0, _ROOT)
        from persistent_megakernel_decode_cu_amd import build
    h.update(repr(([f for f in build.COMMON if not os.path.isabs(f)], sorted(build.EXTRA.items()))).encode())
    csrc = os.path.join(_HERE, "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".h", ".hip", ".cpp")))
    files.append(os.path.join(_ROOT, "include", "mk.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code(fh.read()).encode())
    return h.hexdigest()[:16]


def kernel_durations(db: str) -> dict:
    """{kernel name: [durations in ns]} of a --kernel-trace database."""
    con = sqlite3.connect(db)
    out = collections.defaultdict(list)
    for name, dur in con.execute("select name, duration from kernels"):
        out[name].append(int(dur))
    return out


def pmc_per_dispatch(db: str) -> dict:
    """{kernel name: [(dispatch id, {counter: value summed over instances})]}."""
    con = sqlite3.connect(db)
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for name, did, cn, cv in con.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        acc[did][cn] += float(cv)
        names[did] = name
    out = collections.defaultdict(list)
    for did in sorted(acc):
        out[names[did]].append((did, dict(acc[did])))
    return out


def _short(name: str) -> str:
    return name if len(name) <= 70 else name[:67] + "..."


def stats_text(db: str, command: str) -> str:
    d = kernel_durations(db)
    lines = [f"command: {command}", "",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_us':>12s}"]
    for name, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{_short(name):70s} {len(v):6d} {statistics.mean(v) / 1e3:10.1f} {min(v) / 1e3:10.1f} "
                     f"{max(v) / 1e3:10.1f} {sum(v) / 1e3:12.1f}")
    return "\n".join(lines) + "\n"


def _counter_bytes(db: str, counter: str, kernel: str, copy_kernel: str, skip: int):
    per = pmc_per_dispatch(db)
    mk = [v[counter] for name, lst in per.items() if kernel in name for _, v in lst[skip:] if counter in v]
    cp = [v[counter] for name, lst in per.items() if copy_kernel in name for _, v in lst if counter in v]
    if not mk or not cp:
        raise SystemExit(f"{db}: no {counter} values for '{kernel}' and '{copy_kernel}'")
    return statistics.mean(mk) * 1024.0, statistics.mean(cp) * 1024.0, len(mk)


def traffic_text(fetch_db: str, write_db: str, kernel: str, copy_kernel: str, copy_bytes: int, commands,
                 skip: int, steps_per_launch: int = 1) -> str:
    f_mk, f_cp, nf = _counter_bytes(fetch_db, "FETCH_SIZE", kernel, copy_kernel, skip)
    w_mk, w_cp, nw = _counter_bytes(write_db, "WRITE_SIZE", kernel, copy_kernel, skip)
    ff, fw = f_cp / copy_bytes, w_cp / copy_bytes
    fetch, write = f_mk / ff, w_mk / fw
    lines = [f"command (FETCH_SIZE): {commands[0]}", f"command (WRITE_SIZE): {commands[1]}", "",
             f"kernel: {kernel} ({nf} and {nw} dispatches averaged, first {skip} skipped)",
             f"copy_kernel: {copy_kernel}, {copy_bytes} bytes read and written",
             f"copy_fetch_factor: {ff:.4f}  (FETCH_SIZE bytes / bytes copied)",
             f"copy_write_factor: {fw:.4f}  (WRITE_SIZE bytes / bytes copied)",
             f"raw_fetch_bytes_per_launch: {f_mk:.0f}",
             f"raw_write_bytes_per_launch: {w_mk:.0f}",
             f"fetch_bytes_per_launch: {fetch:.0f}",
             f"write_bytes_per_launch: {write:.0f}",
             f"traffic_bytes_per_launch: {fetch + write:.0f}",
             f"steps_per_launch: {steps_per_launch}",
             f"traffic_bytes_per_step: {(fetch + write) / steps_per_launch:.0f}",
             f"source_digest: {digest()}"]
    return "\n".join(lines) + "\n"


def counters_text(dbs, kernel: str, commands, skip: int) -> str:
    """Per-dispatch averages (summed over counter instances) of every counter
    in the --pmc databases `dbs`, for the kernels whose name holds `kernel`;
    one line per counter, the first `skip` dispatches left out."""
    lines = [f"command: {c}" for c in commands] + ["", f"kernel: {kernel} (first {skip} dispatches skipped)",
                                                   f"{'counter':28s} {'dispatches':>10s} {'per dispatch':>16s}"]
    for db in dbs:
        per = pmc_per_dispatch(db)
        vals = collections.defaultdict(list)
        for name, lst in per.items():
            if kernel not in name:
                continue
            for _, v in lst[skip:]:
                for cn, cv in v.items():
                    vals[cn].append(cv)
        for cn in sorted(vals):
            lines.append(f"{cn:28s} {len(vals[cn]):10d} {statistics.mean(vals[cn]):16.6g}")
    lines.append(f"source_digest: {digest()}")
    return "\n".join(lines) + "\n"


def read_traffic(path: str):
    """(traffic bytes per decode step, source digest) of a traffic summary,
    or None (a launch of a resident run covers steps_per_launch steps)."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        k, _, v = line.partition(":")
        kv[k.strip()] = v.strip()
    try:
        steps = float(kv.get("steps_per_launch", "1").split()[0])
        return float(kv["traffic_bytes_per_launch"]) / steps, kv["source_digest"]
    except (KeyError, ValueError):
        return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("db")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", default="mk_megakernel")
    b.add_argument("--copy-kernel", default="mk_copy_probe")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--skip", type=int, default=1, help="leading dispatches of the kernel to leave out (warm-up)")
    b.add_argument("--steps-per-launch", type=int, default=1, help="decode steps one launch of the kernel runs")
    b.add_argument("--command", action="append", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--kernel", default="mk_megakernel")
    c.add_argument("--skip", type=int, default=1)
    c.add_argument("--command", action="append", required=True)
    sub.add_parser("digest")
    args = ap.parse_args(argv)
    if args.what == "stats":
        sys.stdout.write(stats_text(args.db, args.command))
    elif args.what == "traffic":
        if len(args.command) != 2:
            ap.error("give --command twice: the FETCH_SIZE run, then the WRITE_SIZE run")
        sys.stdout.write(traffic_text(args.fetch, args.write, args.kernel, args.copy_kernel, args.copy_bytes,
                                      args.command, args.skip, args.steps_per_launch))
    elif args.what == "counters":
        sys.stdout.write(counters_text(args.dbs, args.kernel, args.command, args.skip))
    else:
        print(digest())


if __name__ == "__main__":
    main()
