"""Several greedy decode steps in one resident launch (mk_decode_steps)
against the same steps run one launch each (mk_decode_step), through the C
ABI, and against the oracle's greedy chain.

Step s of the resident launch embeds the token that step s - 1 chose and
attends over kv_lens + s entries, with no kernel boundary in between: the
entries earlier steps appended are read back on other XCDs, the tagged
exchange words are rewritten with each step's tag, and the merge counters
run one epoch per step. The single-step chain feeds each step's greedy
token back by hand. Both run the same arithmetic, so every step's tokens,
the last step's logits and hidden output, the final lengths and both K/V
pools (every appended entry) must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import synthetic
from persistent_megakernel_decode_cu_amd import MkError
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(cfg, B, n):
    return {"tokens": torch.full((n, B) if n > 1 else (B,), -1, dtype=torch.int32, device="cuda"),
            "kv_lens": torch.zeros(B, dtype=torch.int32, device="cuda"),
            "logits": torch.full((B, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda"),
            "hidden": torch.full((B, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")}


def _single_chain(dec, st, cfg, n):
    """n launches of one step each, every step's greedy tokens fed back."""
    ds = gu.DevState(st)
    B = st.batch
    toks = []
    for s in range(n):
        out = _outputs(cfg, B, 1)
        dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=ds.tokens, tokens_out=out["tokens"], kv_lens_out=out["kv_lens"],
                 logits_out=out["logits"], hidden_out=out["hidden"])
        dec.sync()
        toks.append(out["tokens"].cpu().numpy())
        ds.tokens.copy_(out["tokens"])
        ds.kv_lens.copy_(out["kv_lens"])
    r = {"tokens": np.stack(toks), "kv_lens": ds.kv_lens.cpu().numpy(), "logits": out["logits"].cpu().numpy(),
         "hidden": out["hidden"].cpu().numpy(), "k_pool": ds.k_pool.cpu().numpy(),
         "v_pool": ds.v_pool.cpu().numpy()}
    return r


def _resident_chain(dec, st, cfg, n):
    """One launch of n steps."""
    ds = gu.DevState(st)
    out = _outputs(cfg, st.batch, n)
    dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
             tokens_in=ds.tokens, tokens_out=out["tokens"], kv_lens_out=out["kv_lens"], logits_out=out["logits"],
             hidden_out=out["hidden"], n_steps=n)
    dec.sync()
    r = {k: v.cpu().numpy() for k, v in out.items()}
    if n == 1:
        r["tokens"] = r["tokens"][None]
    r["k_pool"] = ds.k_pool.cpu().numpy()
    r["v_pool"] = ds.v_pool.cpu().numpy()
    return r


def _compare(cfg, n, st=None, m=None):
    m = m or synthetic.make_model(cfg)
    st = st or synthetic.make_state(cfg, extra_positions=n + 1)
    wdev = gu.upload_model(m)
    dec = gu.make_decoder(m, st, wdev)
    dec.build_schedule(st.batch, mode="megakernel", max_kv_len=int(st.kv_lens.max()) + n)
    print(f"[{cfg.name} batch {st.batch}] {n} steps: one resident launch against {n} launches", flush=True)
    a = _single_chain(dec, st, cfg, n)
    b = _resident_chain(dec, st, cfg, n)
    c = _resident_chain(dec, st, cfg, n)  # a second launch on the same handle: later tags and epochs
    dec.close()
    print(f"  tokens per step: {b['tokens'][:, 0].tolist()}")
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
        assert np.array_equal(c[key].view(np.uint8), b[key].view(np.uint8)), key
    assert np.array_equal(b["kv_lens"], st.kv_lens + n)
    assert np.all(b["tokens"] >= 0)
    return m, st, b


def test_resident_tiny_many_steps():
    _compare(synthetic.workload("tiny-2l"), 24)


def test_resident_batched_paged_against_single_steps_and_oracle(oracle32):
    cfg = synthetic.Workload(31, "tiny-b4-resident", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2,
                             head_dim=64, ffn=1024, vocab=4096, has_embed=True, batch=4, kv_len_range=(1, 300),
                             steps=6, paged_random=True)
    n = 6
    m, st, got = _compare(cfg, n)
    # the oracle's own greedy chain: equal tokens step by step while the
    # chains agree; a disagreement is allowed only where the oracle's top-2
    # gap is within the bar, and ends the comparison of that request
    ost = st.copy()
    live = np.ones(st.batch, bool)
    for s in range(n):
        o = oracle32.decode_step(m, ost, want_hidden=False)
        assert o["rc"] == 0
        for b in range(st.batch):
            if live[b] and got["tokens"][s, b] != o["tokens"][b]:
                gap = gu.top2_gap(o["logits"][b])
                assert gap <= gu.TOP2_GAP, f"step {s} request {b}: token differs with top-2 gap {gap}"
                live[b] = False
        ost.tokens = o["tokens"].copy()
        ost.kv_lens = ost.kv_lens + 1
    print(f"  requests still equal to the oracle's chain after {n} steps: {int(live.sum())} of {st.batch}")


def test_resident_1b_batch1():
    _compare(synthetic.workload("1b-kv1024"), 8)


def test_resident_1b_batch8():
    _compare(synthetic.workload("1b-b8-paged"), 3)


def test_resident_rejects_bad_requests():
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg, extra_positions=4)
    dec = gu.make_decoder(m, st, gu.upload_model(m))
    ds = gu.DevState(st)
    toks = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    args = dict(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                tokens_in=ds.tokens, tokens_out=toks)
    dec.build_schedule(1, mode="unfused", max_kv_len=int(st.kv_lens.max()) + 4)
    with pytest.raises(MkError):
        dec.step(n_steps=2, **args)
    dec.build_schedule(1, mode="megakernel", max_kv_len=int(st.kv_lens.max()) + 4)
    with pytest.raises(MkError):
        dec.step(n_steps=0, **{**args, "tokens_out": toks[0]})
    dec.close()
