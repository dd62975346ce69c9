"""GPU runtime properties of the resident interpreter, through the C ABI.

- Determinism and progress over a long greedy chain: 10,000 consecutive
  steps of the tiny model, with tokens and lengths fed back on the device
  and no host synchronisation between steps. Run twice through the
  megakernel and once through the one-kernel-per-op baseline, all three must
  produce the same token sequence bit for bit. Every step must finish
  without a watchdog or device error, which means no wait deadlocked. The
  baseline shares the op arithmetic and summation orders, so it gives the
  same sequence.
- The per-instruction trace: every instruction of a traced step is stamped,
  and its stamps are ordered (start <= inputs staged <= end).
- The baseline captured in a HIP graph: replays of one captured step form
  the same greedy chain as eager steps.
"""
import numpy as np
import pytest
import torch

import synthetic
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_STEPS = 10_000


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def greedy_chain(mode, n_steps):
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg, extra_positions=n_steps + 1)
    wdev = gu.upload_model(m)
    ds = gu.DevState(st)
    dec = gu.make_decoder(m, st, wdev)
    dec.build_schedule(1, mode=mode, max_kv_len=int(st.kv_lens.max()) + n_steps)
    seq = torch.full((n_steps + 1,), -1, dtype=torch.int32, device="cuda")
    seq[0:1].copy_(ds.tokens)
    lens = ds.kv_lens
    stream = torch.cuda.current_stream().cuda_stream
    print(f"[{mode}] {n_steps} chained steps", flush=True)
    for s in range(n_steps):
        dec.step(kv_lens=lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=seq[s:s + 1], tokens_out=seq[s + 1:s + 2], kv_lens_out=lens, stream=stream)
    dec.sync()  # raises on a sticky device error (watchdog, range, NaN)
    out = seq.cpu().numpy()
    final_len = int(lens.cpu().numpy()[0])
    dec.close()
    return out, final_len, int(st.kv_lens[0])


def test_ten_thousand_steps_deterministic_and_deadlock_free():
    a, len_a, len0 = greedy_chain("megakernel", N_STEPS)
    b, len_b, _ = greedy_chain("megakernel", N_STEPS)
    u, len_u, _ = greedy_chain("unfused", N_STEPS)
    assert len_a == len_b == len_u == len0 + N_STEPS
    assert np.all(a >= 0), "a step did not write its token"
    assert np.array_equal(a, b), f"megakernel runs differ first at step {int(np.argmax(a != b))}"
    assert np.array_equal(a, u), f"megakernel and baseline differ first at step {int(np.argmax(a != u))}"
    print(f"{N_STEPS} steps identical; {len(np.unique(a))} distinct tokens")


def test_trace_stamps_every_instruction_in_order():
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg)
    wdev = gu.upload_model(m)
    ds = gu.DevState(st)
    dec = gu.make_decoder(m, st, wdev)
    info = dec.build_schedule(1, mode="megakernel", max_kv_len=int(st.kv_lens.max()) + 1, n_cus=16, trace=True)
    gu.run_step(dec, ds, cfg)
    tr = dec.trace()
    from persistent_megakernel_decode_cu_amd import _mk
    from tests import sched_check
    plan = _mk.Plan(dec.cfg, _mk.MkScheduleDesc(1, 16, 0, int(st.kv_lens.max()) + 1, 0, 1, 0, 0, 0))
    ins = sched_check.decode(plan.queue)
    assert len(ins) == info["n_instr"]
    for i in ins:
        start, ready, end = (int(x) for x in tr[i.cu, i.pc, :3])
        assert 0 < start <= ready <= end, (i.cu, i.pc, i.op, start, ready, end)
    dec.close()


def test_graph_captured_baseline_replays_match_eager():
    """The one-kernel-per-op baseline, one step captured in a HIP graph on a
    side stream and replayed as a greedy chain (tokens and lengths updated in
    place on the device): every replay must give the token and length of the
    eager chain's step, with eager device work and synchronisations between
    the replays."""
    n = 6
    cfg = synthetic.workload("tiny-2l")
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg, extra_positions=n + 1)
    wdev = gu.upload_model(m)

    def fresh():
        ds = gu.DevState(st)
        dec = gu.make_decoder(m, st, wdev)
        dec.build_schedule(1, mode="unfused", max_kv_len=int(st.kv_lens.max()) + n)
        return ds, dec

    def step(dec, ds, stream):
        dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
                 tokens_in=ds.tokens, tokens_out=ds.tokens, kv_lens_out=ds.kv_lens, stream=stream)

    ds, dec = fresh()
    eager = []
    for _ in range(n):
        step(dec, ds, torch.cuda.current_stream().cuda_stream)
        dec.sync()
        eager.append((int(ds.tokens.cpu()[0]), int(ds.kv_lens.cpu()[0])))
    dec.close()

    ds, dec = fresh()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        step(dec, ds, side.cuda_stream)
    replayed = []
    scratch = torch.zeros(1 << 20, device="cuda")
    for k in range(n):
        graph.replay()
        torch.cuda.synchronize()
        replayed.append((int(ds.tokens.cpu()[0]), int(ds.kv_lens.cpu()[0])))
        scratch.add_(float(k))  # eager work between replays
        torch.cuda.synchronize()
    dec.sync()
    del graph
    dec.close()
    print(f"eager {eager}; replayed {replayed}", flush=True)
    assert replayed == eager
    assert eager[-1][1] == int(st.kv_lens[0]) + n
