"""Writes the stored fixtures of tests/golden/ from the seeded generators and
the CPU oracle only. The page "Inference MegaKernel" (shaojiemike.top) prints
no numeric worked example, so these are regression pins of the generator and
of the oracle, not values from the page.

Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synthetic  # noqa: E402
from oracle import Oracle  # noqa: E402


def main():
    out = {}
    for name in ("tiny-2l", "1b-layer-kv512"):
        cfg = synthetic.workload(name)
        m = synthetic.make_model(cfg)
        st = synthetic.make_state(cfg)
        out[name] = {
            "weights_sha256": synthetic.sha256_of(*[m.weights[k] for k in sorted(m.weights)]),
            "state_sha256": synthetic.sha256_of(st.tokens, st.kv_lens, st.k_pool, st.v_pool,
                                                st.page_table, st.hidden_in),
        }
        r = Oracle("f64").decode_step(m, st, want_hidden=True)
        if cfg.has_embed:
            out[name]["token"] = int(r["tokens"][0])
            out[name]["logits_head"] = [float(v) for v in r["logits"][0, :8]]
        out[name]["hidden_head"] = [float(v) for v in r["hidden"][0, :8]]
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_fixtures.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
