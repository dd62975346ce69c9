"""GPU runtime properties of the resident interpreter, through the C ABI.

- Determinism and progress over a long chain: 10,000 consecutive steps of
  the tiny model with no host synchronisation between them. The inputs vary
  at every step: a seeded token sequence, and lengths that cycle through 512
  positions (so RoPE angles, attention lengths and the overwritten cache
  entries change from step to step). Run twice through the megakernel and
  once through the one-kernel-per-op baseline, the three runs must give the
  same tokens, lengths and, at sampled steps, the same logits bit for bit.
  Every step must finish without a watchdog or device error, which means no
  wait deadlocked. The baseline shares the op arithmetic and summation
  orders, so it gives the same bits.
- The per-instruction trace: every instruction of a traced step is stamped,
  and its stamps are ordered (start <= inputs staged <= end).
- The baseline captured in a HIP graph: replays of one captured step, fed a
  seeded token per replay, match the CPU oracle's logits and tokens.
- The tagged-word visibility protocol the interpreter relies on ("Inference
  MegaKernel", section "unified framework", obligation 1: a producer's data
  is visible before its completion is): writer and reader workgroups on
  different XCDs, the reader holding possibly stale copies in its caches,
  must never read a stale word through device-coherent loads.
- The debug copy of the last layer's activations agrees with the step's
  hidden output in both modes.
"""
import numpy as np
import pytest
import torch

import synthetic
from persistent_megakernel_decode_cu_amd import _mk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_STEPS = 10_000
CYCLE = 512
SAMPLED = (0, 1, 2, 777, 4096, 5000, 9998, 9999)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def forced_chain(mode, n_steps):
    """n_steps steps of the tiny model, step s reading token seq[s] at length
    len0 + s % CYCLE; returns tokens, lengths written and sampled logits."""
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg, extra_positions=CYCLE + 1)
    len0 = int(st.kv_lens[0])
    seq = np.random.default_rng([cfg.cid, 200]).integers(0, cfg.vocab, n_steps).astype(np.int32)
    lens = (len0 + np.arange(n_steps) % CYCLE).astype(np.int32)
    wdev = gu.upload_model(m)
    ds = gu.DevState(st)
    dec = gu.make_decoder(m, st, wdev)
    dec.build_schedule(1, mode=mode, max_kv_len=len0 + CYCLE - 1)
    d_seq = torch.from_numpy(seq).cuda()
    d_lens = torch.from_numpy(lens).cuda()
    d_tok = torch.full((n_steps,), -1, dtype=torch.int32, device="cuda")
    d_len = torch.full((n_steps,), -1, dtype=torch.int32, device="cuda")
    logits = torch.full((len(SAMPLED), cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    where = {s: k for k, s in enumerate(SAMPLED)}
    stream = torch.cuda.current_stream().cuda_stream
    print(f"[{mode}] {n_steps} chained steps", flush=True)
    for s in range(n_steps):
        k = where.get(s)
        dec.step(kv_lens=d_lens[s:s + 1], k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=d_seq[s:s + 1], tokens_out=d_tok[s:s + 1], kv_lens_out=d_len[s:s + 1],
                 logits_out=None if k is None else logits[k:k + 1], stream=stream)
    dec.sync()  # raises on a sticky device error (watchdog, range, NaN)
    out = d_tok.cpu().numpy(), d_len.cpu().numpy(), logits.cpu().numpy()
    dec.close()
    return out, lens


def test_ten_thousand_varying_steps_deterministic_and_deadlock_free():
    (ta, la, ga), lens = forced_chain("megakernel", N_STEPS)
    (tb, lb, gb), _ = forced_chain("megakernel", N_STEPS)
    (tu, lu, gu_), _ = forced_chain("unfused", N_STEPS)
    assert np.array_equal(la, lens + 1) and np.array_equal(lb, la) and np.array_equal(lu, la)
    assert np.all(ta >= 0), "a step did not write its token"
    assert np.array_equal(ta, tb), f"megakernel runs differ first at step {int(np.argmax(ta != tb))}"
    assert np.array_equal(ta, tu), f"megakernel and baseline differ first at step {int(np.argmax(ta != tu))}"
    assert np.all(np.isfinite(ga))
    assert np.array_equal(ga.view(np.uint32), gb.view(np.uint32)), "sampled logits differ between megakernel runs"
    assert np.array_equal(ga.view(np.uint32), gu_.view(np.uint32)), "sampled logits differ from the baseline"
    # the chain is not a fixed point: tokens and logits change along it
    assert len(np.unique(ta)) > 100, f"only {len(np.unique(ta))} distinct tokens"
    assert len({ga[k].tobytes() for k in range(len(SAMPLED))}) == len(SAMPLED)
    print(f"{N_STEPS} steps identical; {len(np.unique(ta))} distinct tokens")


def test_trace_stamps_every_instruction_in_order():
    from persistent_megakernel_decode_cu_amd import trace_summary
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg)
    wdev = gu.upload_model(m)
    ds = gu.DevState(st)
    dec = gu.make_decoder(m, st, wdev)
    info = dec.build_schedule(1, mode="megakernel", max_kv_len=int(st.kv_lens.max()) + 1, n_cus=16, trace=True)
    gu.run_step(dec, ds, cfg)
    tr = dec.trace()
    plan = _mk.Plan(dec.cfg, _mk.MkScheduleDesc(1, 16, 0, int(st.kv_lens.max()) + 1, 0, 1, 0, 0, 0))
    ins = trace_summary.decode_queue(plan.queue)
    assert len(ins) == info["n_instr"]
    for i in ins:
        start, ready, end = (int(x) for x in tr[i.cu, i.pc, :3])
        assert 0 < start <= ready <= end, (i.cu, i.pc, i.op, start, ready, end)
    dec.close()


def test_graph_captured_baseline_replays_match_oracle(oracle32):
    """The one-kernel-per-op baseline, one step captured in a HIP graph on a
    side stream (tokens and lengths read and written in place on the
    device) and replayed with a seeded token written before each replay,
    eager device work and synchronisations between replays. Every replay's
    logits and token must match the oracle run on the same inputs."""
    n = 6
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg, extra_positions=n + 1)
    seq = np.random.default_rng([cfg.cid, 201]).integers(0, cfg.vocab, n).astype(np.int32)
    wdev = gu.upload_model(m)
    ds = gu.DevState(st)
    dec = gu.make_decoder(m, st, wdev)
    dec.build_schedule(1, mode="unfused", max_kv_len=int(st.kv_lens.max()) + n)
    logits = torch.empty((1, cfg.vocab), dtype=torch.float32, device="cuda")
    tok_out = torch.empty(1, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=ds.tokens, tokens_out=tok_out, kv_lens_out=ds.kv_lens, logits_out=logits,
                 stream=side.cuda_stream)
    # the capture ran nothing: the device state is still the initial one
    ost = st.copy()
    scratch = torch.zeros(1 << 20, device="cuda")
    worst = 0.0
    for k in range(n):
        ds.tokens.fill_(int(seq[k]))
        ost.tokens[:] = seq[k]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_logits, g_tok = logits.cpu().numpy(), tok_out.cpu().numpy()
        assert int(ds.kv_lens.cpu()[0]) == int(ost.kv_lens[0]) + 1
        o = oracle32.decode_step(m, ost)
        assert o["rc"] == 0
        diff, _ = gu.check_logits(g_logits, o["logits"], g_tok, o["tokens"])
        worst = max(worst, diff)
        ost.kv_lens = ost.kv_lens + 1
        scratch.add_(float(k))  # eager work between replays
        torch.cuda.synchronize()
    dec.sync()
    del graph
    dec.close()
    print(f"{n} graph replays against the oracle: max |dlogit| {worst:.3g}", flush=True)


def test_tagged_word_protocol_never_reads_stale_across_xcds():
    """mk_debug_litmus in the interpreter's mode: 128 writer/reader pairs
    (workgroups 2k and 2k + 1, which the round-robin dispatch puts on
    different XCDs), 200 rounds of 1024 words; device-coherent stores, a
    completion wait before the flag, no fences. The reader first plants
    possibly stale copies with plain loads; its device-coherent reads after
    the flag must all return the round's value."""
    pairs, n_words, rounds = 128, 1024, 200
    data = torch.zeros(pairs * n_words, dtype=torch.int32, device="cuda")
    flags = torch.zeros(pairs * 64, dtype=torch.int32, device="cuda")
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    _mk._check(_mk.lib().mk_debug_litmus(pairs, n_words, rounds, 1, data.data_ptr(), flags.data_ptr(),
                                         res.data_ptr()))
    r = res.cpu().numpy()
    print(f"litmus: stale plain reads {r[0]}, stale device-coherent reads {r[1]}, timeouts {r[2]}", flush=True)
    assert r[2] == 0, "a litmus wait timed out"
    assert r[1] == 0, f"{r[1]} stale device-coherent reads"


@pytest.mark.parametrize("mode", ["megakernel", "unfused"])
def test_debug_copy_of_residual_stream_equals_hidden_output(mode):
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg)
    wdev = gu.upload_model(m)
    ds = gu.DevState(st)
    dec = gu.make_decoder(m, st, wdev)
    dec.build_schedule(1, mode=mode, max_kv_len=int(st.kv_lens.max()))
    g = gu.run_step(dec, ds, cfg, want_hidden=True)
    x = _mk.mk_debug_copy_scratch(dec.handle, "x", cfg.hidden)
    dec.close()
    assert np.array_equal(x.view(np.uint32), g["hidden"][0].view(np.uint32))
