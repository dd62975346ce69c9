"""The allocation-free step (mk_decode_step_static, for callers that cannot
allocate) against mk_decode_step, through the C ABI.

Both run the same resident interpreter on the same inputs; only where the
exchange words and counters live differs (the device's static scratch, or
the handle's own buffers), so every output must agree bit for bit: tokens,
lengths, logits, the hidden output and both K/V pools. Two calls in a row on
different schedules, the second smaller than the first, so the second reads
a static scratch the first left behind; then a schedule whose exchange
buffers exceed the static scratch is rejected with MK_ECAPACITY before any
launch.
"""
import numpy as np
import pytest
import torch

import synthetic
from persistent_megakernel_decode_cu_amd import _mk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _one(dec, m, st, cfg, static):
    ds = gu.DevState(st)
    B = st.batch
    out = {"tokens": torch.full((B,), -1, dtype=torch.int32, device="cuda"),
           "kv_lens": torch.zeros(B, dtype=torch.int32, device="cuda"),
           "logits": torch.full((B, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda"),
           "hidden": torch.full((B, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")}
    dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
             tokens_in=ds.tokens, tokens_out=out["tokens"], kv_lens_out=out["kv_lens"], logits_out=out["logits"],
             hidden_out=out["hidden"], static_scratch=static)
    dec.sync()
    r = {k: v.cpu().numpy() for k, v in out.items()}
    r["k_pool"] = ds.k_pool.cpu().numpy()
    r["v_pool"] = ds.v_pool.cpu().numpy()
    return r


def _compare(cfg, batch):
    m = synthetic.make_model(cfg)
    st = synthetic.make_state(cfg, extra_positions=2)
    wdev = gu.upload_model(m)
    dec = gu.make_decoder(m, st, wdev)
    dec.build_schedule(batch, mode="megakernel", max_kv_len=int(st.kv_lens.max()))
    print(f"[{cfg.name} batch {batch}] static-scratch step against the handle's", flush=True)
    a = _one(dec, m, st, cfg, static=True)
    b = _one(dec, m, st, cfg, static=False)
    c = _one(dec, m, st, cfg, static=True)  # the handle stays usable both ways
    dec.close()
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
        assert np.array_equal(c[key].view(np.uint8), b[key].view(np.uint8)), key
    assert np.all(a["tokens"] >= 0) and np.array_equal(a["kv_lens"], st.kv_lens + 1)


def test_static_scratch_step_equals_handle_step_twice_then_smaller():
    big = synthetic.Workload(21, "static-b4", n_layers=3, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64,
                             ffn=1024, vocab=3000, has_embed=True, batch=4, kv_len_range=(5, 700), steps=2,
                             paged_random=True)
    _compare(big, 4)
    _compare(synthetic.workload("tiny-2l"), 1)


def test_static_scratch_rejects_a_schedule_beyond_its_size():
    # 96 layers of the 1B shape at batch 2 with 16 attention chunks need
    # about 79 MB of exchange buffers; no kernel runs (the weights are never
    # read), so one small tensor stands in for every weight
    L, B = 96, 2
    dummy = torch.zeros(1 << 20, dtype=torch.int16, device="cuda")
    mc = _mk.MkConfig(L, 2048, 32, 8, 64, 8192, 128256, 1, 1e-5, 10000.0, B, 16, 20, 0)
    layers = (_mk.MkLayerWeights * L)()
    for lw in layers:
        for f, _ in _mk.MkLayerWeights._fields_:
            setattr(lw, f, dummy.data_ptr())
    import ctypes
    w = _mk.MkWeights(dummy.data_ptr(), dummy.data_ptr(), ctypes.cast(layers, ctypes.POINTER(_mk.MkLayerWeights)))
    h = _mk.mk_create(mc, w)
    try:
        _mk.mk_build_schedule(h, _mk.MkScheduleDesc(B, 0, 0, 300, 16, 0, 0, 0, 0))
        io = _mk.MkStepIO(dummy.data_ptr(), None, dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), 1,
                          dummy.data_ptr(), dummy.data_ptr(), None, None, None)
        with pytest.raises(_mk.MkError) as e:
            _mk.mk_decode_step_static(h, io, torch.cuda.current_stream().cuda_stream)
        assert e.value.code == _mk.MK_ECAPACITY
        assert "static scratch" in str(e.value)
        torch.cuda.synchronize()
    finally:
        _mk.mk_destroy(h)
