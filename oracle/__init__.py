"""CPU oracle for one decode step of a Llama-style dense decoder.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``persistent_megakernel_decode_cu_amd``) never imports it, and the two share
no code: this package wraps ``oracle.c`` (plain single-threaded C, sequential
sums in index order) through ctypes.

What it computes follows the page "Inference MegaKernel" (shaojiemike.top),
sections "why conventional inference still has bubbles" (the op chain of a
decode step) and "hand-written whole-model MegaKernel / principle, schedule
and dataflow" (the op bodies and the object table). The per-function
citations and the readings of what the page leaves open are in oracle.c.

Two builds of the same source exist: ``liboracle_f32.so`` (single
precision throughout: the plain single-threaded fp32 forward pass that GPU
parity, the stored chain fixtures, the smoke check and the CPU baseline use)
and ``liboracle_f64.so`` (double; the pins run on both builds, and the f32
build tracks the f64 one to 1e-4 on logits).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, special cases that reduce to a library routine, and
brute force on tiny inputs. The full decode step has no printed example on
the page; it is pinned through those decompositions only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")


def lib_path(precision: str) -> str:
    return os.path.join(_HERE, f"liboracle_{precision}.so")


def build(force: bool = False) -> None:
    """Compile both oracle variants with gcc (no fast-math, no contraction)."""
    for prec, defs in (("f64", []), ("f32", ["-DORACLE_REAL_FLOAT"])):
        out = lib_path(prec)
        if not force and os.path.exists(out) and os.path.getmtime(out) >= max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
        ):
            continue
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", *defs, _SRC, "-o", out + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


class Dims(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("has_embed", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32), ("max_pages_per_req", ctypes.c_int32),
        ("n_pages", ctypes.c_int32),
        ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double),
    ]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "embed", "final_norm", "attn_norm", "wqkv", "wo", "mlp_norm",
        "w_gate", "w_up", "w_down")]


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """ctypes front of one oracle build. ``precision`` is "f64" or "f32"."""

    def __init__(self, precision: str = "f64"):
        path = lib_path(precision)
        if not os.path.exists(path):
            build()
        self.precision = precision
        self.real = np.float64 if precision == "f64" else np.float32
        self._lib = ctypes.CDLL(path)
        L = self._lib
        vp, i32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_rmsnorm.argtypes = [vp, vp, i32, f64, vp]
        L.oracle_matvec.argtypes = [vp, i32, i32, vp, vp]
        L.oracle_rope.argtypes = [vp, i32, i32, i32, f64]
        rtype = ctypes.c_double if precision == "f64" else ctypes.c_float
        L.oracle_silu.argtypes = [rtype]
        L.oracle_silu.restype = rtype
        L.oracle_argmax.argtypes = [vp, i32]
        L.oracle_argmax.restype = i32
        L.oracle_attention.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, i32, vp]
        L.oracle_decode_step.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                         vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_decode_step.restype = i32

    # ---- helpers
    def _real(self, a):
        return np.ascontiguousarray(a, dtype=self.real)

    @staticmethod
    def _u16(a):
        a = np.ascontiguousarray(a)
        assert a.dtype == np.uint16
        return a

    # ---- bf16
    def bf16_to_f32(self, h: int) -> float:
        return float(self._lib.oracle_bf16_to_f32(int(h)))

    def f32_to_bf16(self, f: float) -> int:
        return int(self._lib.oracle_f32_to_bf16(float(np.float32(f))))

    # ---- ops
    def rmsnorm(self, x, w, eps):
        x = self._real(x)
        w = self._u16(w)
        out = np.empty_like(x)
        self._lib.oracle_rmsnorm(_ptr(x), _ptr(w), x.size, float(eps), _ptr(out))
        return out

    def matvec(self, W, x):
        W = self._u16(W)
        x = self._real(x)
        rows, cols = W.shape
        assert x.size == cols
        y = np.empty(rows, dtype=self.real)
        self._lib.oracle_matvec(_ptr(W), rows, cols, _ptr(x), _ptr(y))
        return y

    def rope(self, v, n_heads, head_dim, pos, theta):
        v = self._real(v).copy()
        assert v.size == n_heads * head_dim
        self._lib.oracle_rope(_ptr(v), n_heads, head_dim, int(pos), float(theta))
        return v

    def silu(self, z):
        return float(self._lib.oracle_silu(float(z)))

    def argmax(self, v):
        v = self._real(v)
        return int(self._lib.oracle_argmax(_ptr(v), v.size))

    def attention(self, dims: Dims, q, k_layer, v_layer, page_row, pos):
        q = self._real(q)
        out = np.empty_like(q)
        pr = np.ascontiguousarray(page_row, dtype=np.int32)
        self._lib.oracle_attention(ctypes.byref(dims), _ptr(q), _ptr(self._u16(k_layer)),
                                   _ptr(self._u16(v_layer)), _ptr(pr), int(pos), _ptr(out))
        return out

    # ---- whole step
    def decode_step(self, model, state, want_logits=True, want_hidden=False):
        """Run one decode step in place on ``state`` (its K/V pools receive
        the new entries). ``model`` and ``state`` are the objects built by
        ``synthetic.make_model`` / ``synthetic.make_state``. Returns a dict
        with ``rc``, ``tokens``, ``logits`` [B, V] and ``hidden`` [B, H]."""
        cfg = model.cfg
        dims = dims_of(cfg, state)
        w = model.weights
        W = Weights(*[_ptr(w.get(n)) for n in (
            "embed", "final_norm", "attn_norm", "wqkv", "wo", "mlp_norm",
            "w_gate", "w_up", "w_down")])
        B = state.batch
        logits = np.zeros((B, cfg.vocab), dtype=self.real) if (want_logits and cfg.has_embed) else None
        hidden = np.zeros((B, cfg.hidden), dtype=self.real) if (want_hidden or not cfg.has_embed) else None
        tokens = np.full(B, -1, dtype=np.int32)
        hidden_in = None if state.hidden_in is None else self._real(state.hidden_in)
        rc = self._lib.oracle_decode_step(
            ctypes.byref(dims), ctypes.byref(W), _ptr(state.k_pool), _ptr(state.v_pool),
            _ptr(state.page_table), B, _ptr(state.tokens), _ptr(hidden_in),
            _ptr(state.kv_lens), _ptr(logits), _ptr(hidden), _ptr(tokens))
        return {"rc": int(rc), "tokens": tokens, "logits": logits, "hidden": hidden}


def dims_of(cfg, state) -> Dims:
    return Dims(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                cfg.ffn, cfg.vocab, int(cfg.has_embed), cfg.page_tokens,
                state.page_table.shape[1], state.n_pages, cfg.rms_eps, cfg.rope_theta)


if __name__ == "__main__":  # pragma: no cover
    build(force="--force" in sys.argv)
