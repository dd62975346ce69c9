"""Host scheduler: the encoded queues of every workload pass the
independent validator (coverage, event counts, hazard ordering) and the
randomised simulator (no deadlock over many steps); injected faults are
caught and name the blocked compute unit."""
import numpy as np
import pytest

import synthetic
from persistent_megakernel_decode_cu_amd import _mk
from tests import sched_check
from tests.test_abi import cfg_of


def plan_for(name, n_cus, batch=None, max_kv_len=None, chunks=0):
    w = synthetic.workload(name)
    B = batch or w.batch
    if w.kv_len_range:
        maxlen = w.kv_len_range[1] + w.steps
        pages = (maxlen + 16) // 16 + 1
    else:
        maxlen = w.kv_len + w.steps - 1
        pages = (w.kv_len + w.steps + 15) // 16
    if max_kv_len is not None:
        maxlen = max_kv_len
    cfg = cfg_of(w, max_batch=max(B, 1), pages=pages)
    p = _mk.Plan(cfg, _mk.MkScheduleDesc(B, n_cus, 0, maxlen, chunks, 0, 0, 0, 0))
    return w, B, maxlen, p


@pytest.mark.parametrize("name,n_cus", [("tiny-2l", 256), ("tiny-2l", 7), ("tiny-2l", 32),
                                        ("1b-layer-kv512", 256), ("1b-layer-kv512", 19),
                                        ("1b-kv1024", 256), ("1b-kv8192", 256)])
def test_plans_validate(name, n_cus):
    w, B, maxlen, p = plan_for(name, n_cus)
    sched_check.validate(w, B, p.queue, p.events, p.info.attn_chunks, maxlen)
    assert p.info.n_cus == n_cus
    assert p.info.lds_bytes <= 160 * 1024


def test_tiny_batched_plan_validates():
    w, B, maxlen, p = plan_for("tiny-2l", 16, batch=4)
    sched_check.validate(w, 4, p.queue, p.events, p.info.attn_chunks, maxlen)


def test_streamed_bytes_match_the_byte_model():
    w, B, maxlen, p = plan_for("1b-kv1024", 256)
    kv = w.n_layers * 8 * ((maxlen + 1 + 15) // 16) * 4096
    weights = w.weight_bytes() - 2 * w.hidden * (2 * w.n_layers + 1)  # norms are read, not streamed
    assert p.info.stream_bytes_total == weights + kv
    # balanced: no compute unit streams more than 2% above the mean
    assert p.info.stream_bytes_max_cu <= 1.02 * p.info.stream_bytes_total / 256


@pytest.mark.parametrize("name,n_cus,steps", [("tiny-2l", 8, 10000), ("tiny-2l", 256, 200),
                                              ("1b-layer-kv512", 64, 200), ("1b-kv1024", 256, 2)])
def test_simulator_no_deadlock(name, n_cus, steps):
    w, B, maxlen, p = plan_for(name, n_cus)
    ctr = sched_check.simulate(p.queue, p.events, steps, seed=n_cus)
    need = p.events[:, sched_check.ISA["EV_NEED"]]
    assert np.array_equal(ctr[p.events[:, 0]], need * steps)


def test_simulator_reports_injected_deadlocks():
    w, B, maxlen, p = plan_for("tiny-2l", 8)
    ins = sched_check.decode(p.queue)
    waited = next(i for i in ins if i.waits)
    e = waited.waits[0]
    need = int(p.events[e, sched_check.ISA["EV_NEED"]])
    with pytest.raises(sched_check.Deadlock) as ex:
        sched_check.simulate(p.queue, p.events, 3, need_override={e: need + 1})
    assert "blocked" in str(ex.value)
    producer = next(i for i in ins if i.pubs and i.merge < 0)
    with pytest.raises(sched_check.Deadlock):
        sched_check.simulate(p.queue, p.events, 3, drop_pub=(producer.seq, producer.pubs[0]))


def test_validator_catches_a_missing_edge():
    w, B, maxlen, p = plan_for("tiny-2l", 8)
    q = p.queue.copy()
    I = sched_check.ISA
    # drop the wait of the first UPGATE instruction: its norm input is unordered
    for cu in range(q.shape[0]):
        for pc in range(q.shape[1]):
            if q[cu, pc, I["W_OP"]] == I["OP_UPGATE"]:
                q[cu, pc, I["W_NWAIT"]] = 0
                with pytest.raises(sched_check.ScheduleError):
                    sched_check.validate(w, B, q, p.events, p.info.attn_chunks, maxlen)
                return
    pytest.fail("no UPGATE instruction")
