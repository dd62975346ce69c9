"""ctypes binding of the C ABI declared in include/mk.h (argument marshalling
only; every step of the decode runs in the HIP library libmk.so).

The names mirror the C calls: mk_create, mk_build_schedule, mk_decode_step,
mk_destroy, mk_last_error, mk_sync_status, mk_get_schedule_info,
mk_read_trace, and the host-only mk_plan_* calls. Structures mirror the C
structs field by field.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_OK, MK_EINVAL, MK_ENOSCHED, MK_ECAPACITY, MK_ERESOURCE, MK_EHIP, MK_ETIMEOUT, MK_EDEVICE = range(8)
STATUS_NAMES = {0: "MK_OK", 1: "MK_EINVAL", 2: "MK_ENOSCHED", 3: "MK_ECAPACITY", 4: "MK_ERESOURCE",
                5: "MK_EHIP", 6: "MK_ETIMEOUT", 7: "MK_EDEVICE"}
MK_MODE_MEGAKERNEL, MK_MODE_UNFUSED = 0, 1

i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class MkConfig(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("hidden", i32), ("n_q_heads", i32), ("n_kv_heads", i32),
                ("head_dim", i32), ("ffn", i32), ("vocab", i32), ("has_embed", i32),
                ("rms_eps", f32), ("rope_theta", f32), ("max_batch", i32), ("page_tokens", i32),
                ("max_pages_per_req", i32), ("device", i32)]


class MkLayerWeights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class MkWeights(ctypes.Structure):
    _fields_ = [("embed", vp), ("final_norm", vp), ("layers", ctypes.POINTER(MkLayerWeights))]


class MkScheduleDesc(ctypes.Structure):
    _fields_ = [("batch", i32), ("n_cus", i32), ("mode", i32), ("max_kv_len", i32),
                ("attn_chunks", i32), ("trace", i32), ("watchdog_spins", i64), ("attn_split", i32),
                ("reserved1", i32)]


class MkStepIO(ctypes.Structure):
    _fields_ = [("tokens_in", vp), ("hidden_in", vp), ("kv_lens", vp), ("k_pool", vp), ("v_pool", vp),
                ("n_pages", i32), ("page_table", vp), ("tokens_out", vp), ("kv_lens_out", vp),
                ("logits_out", vp), ("hidden_out", vp)]


class MkScheduleInfo(ctypes.Structure):
    _fields_ = [("n_cus", i32), ("queue_len", i32), ("n_instr", i32), ("n_events", i32),
                ("n_counters", i32), ("attn_chunks", i32), ("prefetch_slices", i32), ("lds_bytes", i32),
                ("block_threads", i32), ("stream_bytes_max_cu", i64), ("stream_bytes_total", i64),
                ("launches_per_step", i32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "mk_create": (i32, [ctypes.POINTER(MkConfig), ctypes.POINTER(MkWeights), ctypes.POINTER(vp)]),
    "mk_build_schedule": (i32, [vp, ctypes.POINTER(MkScheduleDesc)]),
    "mk_decode_step": (i32, [vp, ctypes.POINTER(MkStepIO), vp]),
    "mk_decode_step_static": (i32, [vp, ctypes.POINTER(MkStepIO), vp]),
    "mk_decode_steps": (i32, [vp, ctypes.POINTER(MkStepIO), i32, vp]),
    "mk_destroy": (None, [vp]),
    "mk_last_error": (ctypes.c_char_p, []),
    "mk_sync_status": (i32, [vp, vp]),
    "mk_get_schedule_info": (i32, [vp, ctypes.POINTER(MkScheduleInfo)]),
    "mk_read_trace": (i32, [vp, ctypes.POINTER(ctypes.c_int64), ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]),
    "mk_debug_copy_scratch": (i32, [vp, i32, vp, ctypes.c_size_t]),
    "mk_debug_copy_probe": (i32, [vp, vp, ctypes.c_size_t, vp]),
    "mk_debug_litmus": (i32, [i32, i32, i32, i32, vp, vp, vp]),
    "mk_debug_attn_split": (i32, [vp, i32, i32, i32, i32, i32, vp]),
    "mk_debug_hop_probe": (i32, [vp, ctypes.c_size_t, vp, ctypes.c_size_t, i32, i32, i32, vp]),
    "mk_debug_ll_probe": (i32, [vp, ctypes.c_size_t, i32, i32, i32, i32, vp]),
    "mk_debug_regstream_probe": (i32, [vp, ctypes.c_size_t, i32, i32, i32, vp]),
    "mk_plan_create": (i32, [ctypes.POINTER(MkConfig), ctypes.POINTER(MkScheduleDesc), ctypes.POINTER(vp)]),
    "mk_plan_destroy": (None, [vp]),
    "mk_plan_info": (i32, [vp, ctypes.POINTER(MkScheduleInfo)]),
    "mk_plan_queue": (i32, [vp, ctypes.POINTER(ctypes.c_int32), ctypes.c_size_t]),
    "mk_plan_events": (i32, [vp, ctypes.POINTER(ctypes.c_int32), ctypes.c_size_t]),
}


def lib():
    """The loaded HIP library. Raises if it has not been built: there is no
    fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m persistent_megakernel_decode_cu_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def mk_last_error() -> str:
    return lib().mk_last_error().decode()


def _check(rc: int):
    if rc != MK_OK:
        raise MkError(rc, mk_last_error())


def mk_create(cfg: MkConfig, weights: MkWeights) -> int:
    h = vp()
    _check(lib().mk_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h)))
    return h.value


def mk_build_schedule(handle: int, desc: MkScheduleDesc) -> None:
    _check(lib().mk_build_schedule(handle, ctypes.byref(desc)))


def mk_decode_step(handle: int, io: MkStepIO, stream: int = 0) -> None:
    _check(lib().mk_decode_step(handle, ctypes.byref(io), stream))


def mk_decode_step_static(handle: int, io: MkStepIO, stream: int = 0) -> None:
    _check(lib().mk_decode_step_static(handle, ctypes.byref(io), stream))


def mk_decode_steps(handle: int, io: MkStepIO, n_steps: int, stream: int = 0) -> None:
    _check(lib().mk_decode_steps(handle, ctypes.byref(io), n_steps, stream))


def mk_destroy(handle: int) -> None:
    lib().mk_destroy(handle)


def mk_sync_status(handle: int, stream: int = 0) -> None:
    _check(lib().mk_sync_status(handle, stream))


def mk_get_schedule_info(handle: int) -> MkScheduleInfo:
    info = MkScheduleInfo()
    _check(lib().mk_get_schedule_info(handle, ctypes.byref(info)))
    return info


def mk_read_trace(handle: int) -> np.ndarray:
    info = mk_get_schedule_info(handle)
    cap = info.n_cus * info.queue_len * TRACE_WORDS
    buf = np.zeros(cap, dtype=np.int64)
    n = ctypes.c_size_t()
    _check(lib().mk_read_trace(handle, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), cap, ctypes.byref(n)))
    return buf.reshape(info.n_cus, info.queue_len, TRACE_WORDS)


TRACE_WORDS = 8  # MK_TRACE_WORDS

SCRATCH = {"x": 0, "qkv": 1, "o": 2, "act": 3}


def mk_debug_copy_scratch(handle: int, which: str, n_floats: int) -> np.ndarray:
    out = np.zeros(n_floats, dtype=np.float32)
    _check(lib().mk_debug_copy_scratch(handle, SCRATCH[which], out.ctypes.data, out.nbytes))
    return out


def mk_debug_copy_probe(src_ptr: int, dst_ptr: int, nbytes: int, stream: int = 0) -> None:
    _check(lib().mk_debug_copy_probe(src_ptr, dst_ptr, nbytes, stream))


def mk_debug_attn_split(kv_lens_ptr: int, n_cases: int, batch: int, tiles: int, mode: int, capacity: int,
                        out_ptr: int) -> None:
    _check(lib().mk_debug_attn_split(kv_lens_ptr, n_cases, batch, tiles, mode, capacity, out_ptr))


def mk_debug_regstream_probe(src_ptr: int, nbytes: int, blocks: int, threads: int, depth: int, out_ptr: int) -> None:
    _check(lib().mk_debug_regstream_probe(src_ptr, nbytes, blocks, threads, depth, out_ptr))


class Plan:
    """Host-only schedule (no GPU needed): encoded queues and event table."""

    def __init__(self, cfg: MkConfig, desc: MkScheduleDesc):
        h = vp()
        _check(lib().mk_plan_create(ctypes.byref(cfg), ctypes.byref(desc), ctypes.byref(h)))
        self._h = h.value
        info = MkScheduleInfo()
        _check(lib().mk_plan_info(self._h, ctypes.byref(info)))
        self.info = info
        q = np.zeros(max(1, info.n_cus * info.queue_len * 32), dtype=np.int32)
        if info.n_instr:
            _check(lib().mk_plan_queue(self._h, q.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), q.size))
        self.queue = q[: info.n_cus * info.queue_len * 32].reshape(info.n_cus, info.queue_len, 32)
        e = np.zeros(max(1, info.n_events * 16), dtype=np.int32)
        if info.n_events:
            _check(lib().mk_plan_events(self._h, e.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), e.size))
        self.events = e[: info.n_events * 16].reshape(info.n_events, 16)

    def close(self):
        if self._h:
            lib().mk_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
