"""Writes tests/golden/chain_<workload>.json: the CPU oracle's 128-step
teacher-forced greedy chain of a 16-layer 1B-shaped workload.

Calls only the seeded generators (synthetic/) and the oracle (oracle/). For
each step s the oracle runs on its own cache (which keeps the entries the
earlier steps appended), at K/V length len0 + s, with the token the oracle
picked at step s - 1 (the workload's seeded token at s = 0). Stored per step:
the oracle's token and the gap between its two largest logits (binary32);
at a few steps also the logits at seeded sample indices and at the 64
largest, which the GPU test compares element by element. Those indices and
values are stored exactly, as base64 of little-endian int32 and binary32
arrays (`decode` reads them back).

The page "Inference MegaKernel" (shaojiemike.top) prints no numeric example;
these are the oracle's values, used to hold the GPU path to it over the whole
chain of the workload.

Run: python tests/golden/make_chains.py 1b-kv1024 [1b-kv8192]
"""
import base64
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synthetic  # noqa: E402
from oracle import Oracle  # noqa: E402

STEPS = 128
LOGIT_STEPS = (0, 1, 31, 63, 95, 127)
N_SAMPLE = 4096
N_TOP = 64


def top2_gap(row):
    f = row.astype(np.float32)
    i = int(np.argmax(f))
    return float(f[i] - np.max(np.delete(f, i)))


def _b64(a):
    return base64.b64encode(np.ascontiguousarray(a).tobytes()).decode("ascii")


def decode(rec):
    """(indices int32, logits float32) of one stored step."""
    idx = np.frombuffer(base64.b64decode(rec["index"]), dtype="<i4")
    val = np.frombuffer(base64.b64decode(rec["value"]), dtype="<f4")
    return idx, val


def make(name):
    cfg = synthetic.workload(name)
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg, extra_positions=STEPS + 1)
    ora = Oracle("f32")
    sample = np.sort(np.random.default_rng([cfg.cid, 100]).choice(cfg.vocab, N_SAMPLE, replace=False))
    out = {"workload": name, "oracle": "f32", "steps": STEPS, "token0": int(st.tokens[0]),
           "kv_len0": int(st.kv_lens[0]), "tokens": [], "gaps": [], "logits": {}}
    t = time.time()
    for s in range(STEPS):
        r = ora.decode_step(m, st)
        assert r["rc"] == 0
        row = r["logits"][0].astype(np.float32)
        out["tokens"].append(int(r["tokens"][0]))
        out["gaps"].append(top2_gap(row))
        if s in LOGIT_STEPS:
            top = np.argsort(-row, kind="stable")[:N_TOP]
            idx = np.unique(np.concatenate([sample, top]))
            out["logits"][str(s)] = {"index": _b64(idx.astype("<i4")), "value": _b64(row[idx].astype("<f4"))}
        st.tokens = r["tokens"].copy()
        st.kv_lens = st.kv_lens + 1
        print(f"{name} step {s}: token {out['tokens'][-1]} gap {out['gaps'][-1]:.4f} ({time.time() - t:.0f} s)",
              flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"chain_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f)


if __name__ == "__main__":
    for n in sys.argv[1:] or ["1b-kv1024", "1b-kv8192"]:
        make(n)
