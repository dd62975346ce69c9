"""GPU path over the whole 128-step greedy chains of the 16-layer 1B-shaped
batch-1 workloads (K/V length 1024 and 8192), against the CPU oracle's chain
stored in tests/golden/chain_<workload>.json (written by
tests/golden/make_chains.py, which calls only the seeded generators and the
oracle).

Protocol (teacher-forced): at step s both sides start from their own cache
(holding their own earlier appended entries) at length len0 + s, with the
oracle's token of step s - 1 as input. At every step the GPU's greedy token
must equal the oracle's wherever the oracle's top-2 gap exceeds 1e-2; at the
stored steps the GPU's logits at the stored indices (a seeded sample of the
vocabulary plus the oracle's 64 largest) must be within 5e-2 of the oracle's.
The length written by each step (kv_lens_out aliasing kv_lens) must be
len0 + s + 1.
"""
import base64
import json
import os

import numpy as np
import pytest
import torch

import synthetic
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
_models = {}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def fixture(name):
    with open(os.path.join(HERE, "golden", f"chain_{name}.json")) as f:
        return json.load(f)


def stored_logits(rec):
    """(indices, binary32 logits) of a stored step (base64 of little-endian
    int32 and binary32 arrays, as make_chains.py writes them)."""
    return (np.frombuffer(base64.b64decode(rec["index"]), dtype="<i4"),
            np.frombuffer(base64.b64decode(rec["value"]), dtype="<f4"))


def model_of(name):
    if name not in _models:
        _models.clear()
        cfg = synthetic.workload(name)
        _models[name] = (cfg, synthetic.make_model(cfg))
    return _models[name]


@pytest.mark.parametrize("name", ["1b-kv1024", "1b-kv8192"])
@pytest.mark.parametrize("mode", ["megakernel", "unfused"])
def test_128_step_chain_matches_oracle(name, mode):
    fx = fixture(name)
    steps = fx["steps"]
    cfg, m = model_of(name)
    st = synthetic.make_state(cfg, extra_positions=steps + 1)
    assert int(st.tokens[0]) == fx["token0"] and int(st.kv_lens[0]) == fx["kv_len0"]
    wdev = gu.upload_model(m)
    ds = gu.DevState(st)
    dec = gu.make_decoder(m, st, wdev)
    dec.build_schedule(1, mode=mode, max_kv_len=fx["kv_len0"] + steps)
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    tokens_out = torch.empty(1, dtype=torch.int32, device="cuda")
    worst, forced = 0.0, 0
    print(f"[{name} {mode}] {steps} teacher-forced steps", flush=True)
    for s in range(steps):
        tok_in = fx["token0"] if s == 0 else fx["tokens"][s - 1]
        ds.tokens.fill_(tok_in)
        dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=ds.tokens, tokens_out=tokens_out, kv_lens_out=ds.kv_lens, logits_out=logits)
        dec.sync()
        g_tok = int(tokens_out.cpu()[0])
        assert int(ds.kv_lens.cpu()[0]) == fx["kv_len0"] + s + 1, f"length after step {s}"
        if g_tok != fx["tokens"][s]:
            assert fx["gaps"][s] <= gu.TOP2_GAP, (
                f"step {s}: token {g_tok} against the oracle's {fx['tokens'][s]} with top-2 gap {fx['gaps'][s]}")
            forced += 1
        rec = fx["logits"].get(str(s))
        if rec is not None:
            idx, want = stored_logits(rec)
            got = logits.cpu().numpy()[0]
            assert np.all(np.isfinite(got)), f"step {s}: non-finite logits"
            d = float(np.max(np.abs(got[idx].astype(np.float64) - want.astype(np.float64))))
            worst = max(worst, d)
            assert d <= gu.LOGIT_TOL, f"step {s}: max |logit diff| {d}"
    dec.close()
    print(f"{name} {mode}: {steps} steps, max |dlogit| at stored steps {worst:.3g}, "
          f"{forced} allowed token differences", flush=True)
