"""Regression pins of the seeded generators and of the oracle's outputs on
the two small workloads (fixtures written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

import synthetic

HERE = os.path.dirname(os.path.abspath(__file__))


def _fixtures():
    with open(os.path.join(HERE, "golden", "oracle_fixtures.json")) as f:
        return json.load(f)


def test_generators_are_deterministic():
    fx = _fixtures()
    for name, rec in fx.items():
        cfg = synthetic.workload(name)
        m = synthetic.make_model(cfg)
        st = synthetic.make_state(cfg)
        assert synthetic.sha256_of(*[m.weights[k] for k in sorted(m.weights)]) == rec["weights_sha256"]
        assert synthetic.sha256_of(st.tokens, st.kv_lens, st.k_pool, st.v_pool, st.page_table,
                                   st.hidden_in) == rec["state_sha256"]


def test_oracle_outputs_are_stable(oracle64):
    fx = _fixtures()
    for name, rec in fx.items():
        cfg = synthetic.workload(name)
        r = oracle64.decode_step(synthetic.make_model(cfg), synthetic.make_state(cfg), want_hidden=True)
        assert np.array_equal(r["hidden"][0, :8], np.array(rec["hidden_head"]))
        if cfg.has_embed:
            assert int(r["tokens"][0]) == rec["token"]
            assert np.array_equal(r["logits"][0, :8], np.array(rec["logits_head"]))


def test_workload_byte_budget():
    """Algorithmic weight bytes of the 1B-shaped layer and step."""
    c3 = synthetic.workload("1b-kv1024")
    per_layer = 2 * (3072 * 2048 + 2048 * 2048 + 3 * 2048 * 8192) + 4 * 2048
    assert c3.weight_bytes() == 16 * per_layer + 2 * 128256 * 2048 + 2 * 2048
    assert abs(per_layer / 1e6 - 121.64) < 0.01
