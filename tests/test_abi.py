"""The C-ABI library loads, exports every call declared in include/*.h, and
its argument checks and host-only planning work without a GPU."""
import ctypes
import dataclasses
import glob
import os
import re

import pytest

from persistent_megakernel_decode_cu_amd import _mk
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(mk_\w+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"mk_create", "mk_build_schedule", "mk_decode_step", "mk_destroy"} <= set(names)
    lib = ctypes.CDLL(_mk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(_mk._SIGS), "binding misses a declared call"


def cfg_of(w, max_batch=1, pages=None, device=0):
    pages = pages or ((w.kv_len or 4096) + w.steps + 15) // 16
    return _mk.MkConfig(w.n_layers, w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ffn, w.vocab,
                        int(w.has_embed), w.rms_eps, w.rope_theta, max_batch, 16, pages, device)


def test_null_and_invalid_arguments_without_gpu():
    L = _mk.lib()
    assert L.mk_create(None, None, None) == _mk.MK_EINVAL
    assert L.mk_build_schedule(None, None) == _mk.MK_EINVAL
    assert L.mk_decode_step(None, None, None) == _mk.MK_EINVAL
    assert L.mk_sync_status(None, None) == _mk.MK_EINVAL
    L.mk_destroy(None)  # no-op
    assert isinstance(_mk.mk_last_error(), str) and _mk.mk_last_error()


@pytest.mark.parametrize("field,value", [("head_dim", 128), ("n_kv_heads", 3), ("hidden", 300),
                                         ("page_tokens", 8), ("max_batch", 9)])
def test_shape_checks(field, value):
    w = synthetic.workload("tiny-2l")
    cfg = cfg_of(w)
    setattr(cfg, field, value)
    desc = _mk.MkScheduleDesc(1, 8, 0, 0, 0, 0, 0, 0, 0)
    with pytest.raises(_mk.MkError) as e:
        _mk.Plan(cfg, desc)
    assert e.value.code == _mk.MK_EINVAL


def test_capacity_checks():
    w = synthetic.workload("tiny-2l")
    cfg = cfg_of(w, pages=5)
    with pytest.raises(_mk.MkError) as e:
        _mk.Plan(cfg, _mk.MkScheduleDesc(1, 8, 0, 80, 0, 0, 0, 0, 0))   # 80 >= 5 * 16
    assert e.value.code == _mk.MK_ECAPACITY
    with pytest.raises(_mk.MkError) as e:
        _mk.Plan(cfg_of(w, max_batch=2), _mk.MkScheduleDesc(3, 8, 0, 0, 0, 0, 0, 0, 0))  # batch > max_batch
    assert e.value.code == _mk.MK_EINVAL
    big = synthetic.workload("1b-b8-paged")
    # batch 8 of the 1B shape fits (the down projection's input is staged as binary16)
    _mk.Plan(cfg_of(big, max_batch=8, pages=258), _mk.MkScheduleDesc(8, 256, 0, 0, 0, 0, 0, 0, 0))
    wide = dataclasses.replace(big, ffn=32768)
    with pytest.raises(_mk.MkError) as e:   # 8 activation rows of 32768 do not fit in the LDS
        _mk.Plan(cfg_of(wide, max_batch=8, pages=258), _mk.MkScheduleDesc(8, 256, 0, 0, 0, 0, 0, 0, 0))
    assert e.value.code == _mk.MK_ECAPACITY
    # the one-kernel-per-op mode has no such limit
    _mk.Plan(cfg_of(wide, max_batch=8, pages=258), _mk.MkScheduleDesc(8, 256, 1, 0, 0, 0, 0, 0, 0))
    with pytest.raises(_mk.MkError) as e:   # reserved field
        _mk.Plan(cfg_of(w), _mk.MkScheduleDesc(1, 8, 0, 0, 0, 0, 0, 0, 1))
    assert e.value.code == _mk.MK_EINVAL
    with pytest.raises(_mk.MkError) as e:   # unknown attention split
        _mk.Plan(cfg_of(w), _mk.MkScheduleDesc(1, 8, 0, 0, 0, 0, 0, 2, 0))
    assert e.value.code == _mk.MK_EINVAL
    _mk.Plan(cfg_of(w), _mk.MkScheduleDesc(1, 8, 0, 0, 0, 0, 0, 1, 0))  # per-request split


def test_head_grouping_of_the_resident_interpreter():
    w = synthetic.workload("tiny-2l")
    cfg = cfg_of(w)
    cfg.n_q_heads, cfg.n_kv_heads = 24, 8   # 3 q heads per kv head: no interpreter variant
    with pytest.raises(_mk.MkError) as e:
        _mk.Plan(cfg, _mk.MkScheduleDesc(1, 8, 0, 0, 0, 0, 0, 0, 0))
    assert e.value.code == _mk.MK_EINVAL
    _mk.Plan(cfg, _mk.MkScheduleDesc(1, 8, 1, 0, 0, 0, 0, 0, 0))  # the unfused path takes any grouping


def test_create_reports_hip_error_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    w = synthetic.workload("tiny-2l")
    cfg = cfg_of(w)
    layers = (_mk.MkLayerWeights * w.n_layers)()
    for l in range(w.n_layers):
        for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            setattr(layers[l], k, 0x1000)
    weights = _mk.MkWeights(0x1000, 0x1000, ctypes.cast(layers, ctypes.POINTER(_mk.MkLayerWeights)))
    with pytest.raises(_mk.MkError) as e:
        _mk.mk_create(cfg, weights)
    assert e.value.code in (_mk.MK_EHIP, _mk.MK_EINVAL)
