"""Host scheduler: the encoded queues of every workload pass the independent
validator (coverage, merge events, every input produced earlier in the global
order) and the randomised simulator (no deadlock over many steps); injected
faults are caught and name the blocked compute unit."""
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


@pytest.mark.parametrize("batch,n_cus,chunks", [(4, 16, 0), (2, 8, 3), (3, 5, 1)])
def test_tiny_batched_plans_validate(batch, n_cus, chunks):
    w, B, maxlen, p = plan_for("tiny-2l", n_cus, batch=batch, chunks=chunks)
    sched_check.validate(w, batch, p.queue, p.events, p.info.attn_chunks, maxlen)


def test_1b_batch4_and_batch8_fit():
    # at a padded batch of 8 the down projection's input is staged as binary16
    for batch in (4, 8):
        w, B, maxlen, p = plan_for("1b-kv1024", 256, batch=batch)
        sched_check.validate(w, batch, p.queue, p.events, p.info.attn_chunks, maxlen)
        assert p.info.lds_bytes <= 160 * 1024


def test_streamed_bytes_match_the_byte_model():
    w, B, maxlen, p = plan_for("1b-kv1024", 256)
    kv = w.n_layers * 8 * ((maxlen + 1 + 15) // 16) * 4096
    weights = w.weight_bytes() - 2 * w.hidden * (2 * w.n_layers + 1)  # norms are read, not streamed
    assert p.info.stream_bytes_total == weights + kv
    # balanced: no compute unit streams more than 2% above the mean
    assert p.info.stream_bytes_max_cu <= 1.02 * p.info.stream_bytes_total / 256


def test_auto_chunks_about_one_block_per_wave():
    # attention is spread so that about one 16-position K/V block goes to
    # each of half a tile's 8 waves (one wave per SIMD), up to a chunk cap
    # that halves above batch 2, where there are also no more attention
    # tiles than compute units; long K/V at batch <= 2 goes to two blocks per
    # wave, up to one tile per compute unit
    for name in ("tiny-2l", "1b-kv1024", "1b-kv8192", "1b-b8-paged"):
        w, B, maxlen, p = plan_for(name, 256)
        nb = (maxlen + 1 + 15) // 16
        cap = sched_check.ISA["AUTO_ATTN_CHUNKS"] // (1 if B <= 2 else 2)
        want = min(cap, max(1, -(-nb // 4)))
        if B <= 2:
            want = max(want, min(sched_check.ISA["MAX_ATTN_CHUNKS"], -(-nb // 16), max(1, 256 // (B * w.n_kv_heads))))
        if B > 2:
            want = min(want, max(1, 256 // (B * w.n_kv_heads)))
        want = min(want, nb)
        assert p.info.attn_chunks == want, (name, p.info.attn_chunks, want)
        if B > 2:
            assert B * p.info.attn_chunks * w.n_kv_heads <= 256


def test_attention_chunks_above_the_limit_are_rejected():
    with pytest.raises(_mk.MkError) as ex:
        plan_for("1b-kv1024", 256, chunks=sched_check.ISA["MAX_ATTN_CHUNKS"] + 1)
    assert ex.value.code == _mk.MK_EINVAL
    # batch 8: the per-request cap is allowed, but not more tiles per kv head
    # than the split's tables hold
    with pytest.raises(_mk.MkError) as ex:
        plan_for("1b-b8-paged", 256, chunks=sched_check.ISA["MAX_ATTN_TILES"] // 8 + 1)
    assert ex.value.code == _mk.MK_EINVAL
    w, B, maxlen, p = plan_for("1b-b8-paged", 256, chunks=sched_check.ISA["MAX_ATTN_TILES"] // 8)
    assert p.info.attn_chunks * B <= sched_check.ISA["MAX_ATTN_TILES"]


@pytest.mark.parametrize("name,n_cus,steps", [("tiny-2l", 8, 2000), ("tiny-2l", 256, 50),
                                              ("1b-layer-kv512", 64, 20), ("1b-kv1024", 256, 1)])
def test_simulator_no_deadlock(name, n_cus, steps):
    w, B, maxlen, p = plan_for(name, n_cus)
    ctr = sched_check.simulate(w, B, p.queue, p.events, steps, seed=n_cus)
    if len(p.events):
        assert np.array_equal(ctr[: len(p.events)], p.events[:, sched_check.ISA["EV_NEED"]] * steps)


def test_simulator_reports_injected_deadlocks():
    w, B, maxlen, p = plan_for("tiny-2l", 8, chunks=2)
    ins = sched_check.decode(p.queue)
    I = sched_check.ISA
    # an attention chunk whose softmax state never arrives: the O projection waits on it
    chunk = next(i for i in ins if i.op == I["OP_ATTN"] and i.layer == 0)
    with pytest.raises(sched_check.Deadlock) as ex:
        sched_check.simulate(w, B, p.queue, p.events, 3, drop=chunk.seq)
    assert "blocked" in str(ex.value)
    # a producer whose rows never arrive
    producer = next(i for i in ins if i.op == I["OP_UPGATE"])
    with pytest.raises(sched_check.Deadlock):
        sched_check.simulate(w, B, p.queue, p.events, 3, drop=producer.seq)


def test_validator_catches_an_out_of_order_consumer():
    w, B, maxlen, p = plan_for("tiny-2l", 8)
    q = p.queue.copy()
    I = sched_check.ISA
    # move the first UPGATE before every O projection in the global order
    ups = [(cu, pc) for cu in range(q.shape[0]) for pc in range(q.shape[1]) if q[cu, pc, I["W_OP"]] == I["OP_UPGATE"]]
    cu, pc = ups[0]
    q[cu, pc, I["W_SEQ"]], q[cu, pc - 1, I["W_SEQ"]] = q[cu, pc - 1, I["W_SEQ"]], q[cu, pc, I["W_SEQ"]]
    with pytest.raises(sched_check.ScheduleError):
        sched_check.validate(w, B, q, p.events, p.info.attn_chunks, maxlen)


def test_validator_catches_a_coverage_gap():
    w, B, maxlen, p = plan_for("tiny-2l", 8)
    q = p.queue.copy()
    I = sched_check.ISA
    for cu in range(q.shape[0]):
        for pc in range(q.shape[1]):
            if q[cu, pc, I["W_OP"]] == I["OP_DOWN"] and q[cu, pc, I["W_R1"]] - q[cu, pc, I["W_R0"]] > 1:
                q[cu, pc, I["W_R1"]] -= 1
                with pytest.raises(sched_check.ScheduleError):
                    sched_check.validate(w, B, q, p.events, p.info.attn_chunks, maxlen)
                return
    pytest.fail("no DOWN instruction with two rows")


def test_trace_decoder_follows_the_queue_encoding():
    """The package's queue decoder (used by the benchmark's trace timeline)
    reads the words and opcodes mk_isa.h defines."""
    from persistent_megakernel_decode_cu_amd import trace_summary as ts
    from tests.sched_check import ISA
    assert (ts.W_OP, ts.W_LAYER, ts.OP_END) == (ISA["W_OP"], ISA["W_LAYER"], ISA["OP_END"])
    ops = {v: k[3:] for k, v in ISA.items() if k.startswith("OP_") and k not in ("OP_END", "OP_COUNT")}
    assert ts.OP_NAMES == ops


@pytest.mark.parametrize("name", ["1b-kv1024", "1b-kv8192", "tiny-2l"])
def test_batch1_tile_multiplier_divides_exactly(name):
    """A single request's attention tile t of T covers blocks [t nb / T,
    (t + 1) nb / T); the interpreter divides by T as the high word of
    n ceil(2^32 / T), the multiplier the queue carries in the R1 word of each
    attention instruction. The multiplier is checked against its definition,
    and the quotient against integer division for every n the device can
    form (n <= T x 65536 blocks)."""
    w, B, maxlen, p = plan_for(name, 256)
    assert B == 1
    q = p.queue.reshape(-1, sched_check.ISA["INSTR_WORDS"])
    attn = q[q[:, sched_check.ISA["W_OP"]] == sched_check.ISA["OP_ATTN"]]
    T = int(attn[0, sched_check.ISA["W_NCH"]])
    assert T == p.info.attn_chunks and np.all(attn[:, sched_check.ISA["W_NCH"]] == T)
    mult = attn[:, sched_check.ISA["W_R1"]].astype(np.uint32)
    want = 0 if T == 1 else -(-(1 << 32) // T)
    assert np.all(mult == np.uint32(want))
    if T > 1:
        n = np.arange(0, T * 65536 + 1, dtype=np.uint64)
        assert np.array_equal((n * np.uint64(want)) >> np.uint64(32), n // np.uint64(T))
