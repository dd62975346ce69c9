"""Persistent decode megakernel for AMD Instinct MI355X (gfx950).

One decode step of a Llama-style dense decoder runs as one resident grid of
one workgroup per compute unit (see include/mk.h for the C ABI and the page
it follows). This package is the thin Python front: ``_mk`` binds the C ABI
with ctypes, and ``Decoder`` marshals torch device tensors into its structs.
PyTorch provides device memory and streams only; every step of the decode
runs in the HIP kernels of ``libmk.so``. There is no fallback path: if the
library is not built, or the device is not gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
from typing import Mapping, Optional

from . import _mk
from ._mk import (MK_MODE_MEGAKERNEL, MK_MODE_UNFUSED, MkConfig, MkError, MkLayerWeights,  # noqa: F401
                  MkScheduleDesc, MkStepIO, MkWeights, Plan, mk_build_schedule, mk_create, mk_decode_step,
                  mk_decode_step_static, mk_decode_steps,
                  mk_destroy, mk_get_schedule_info, mk_last_error, mk_read_trace, mk_sync_status)

_MODES = {"megakernel": MK_MODE_MEGAKERNEL, "unfused": MK_MODE_UNFUSED}
_SPLITS = {"balanced": 0, "per_request": 1}  # MK_SPLIT_BALANCED, MK_SPLIT_PER_REQUEST
_LAYER_KEYS = ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def make_config(shape, max_batch: int, max_pages_per_req: int, device: int = 0) -> MkConfig:
    """MkConfig from any object with the model-shape attributes (n_layers,
    hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, has_embed, rms_eps,
    rope_theta, page_tokens)."""
    return MkConfig(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                    shape.ffn, shape.vocab, int(bool(shape.has_embed)), float(shape.rms_eps),
                    float(shape.rope_theta), int(max_batch), int(shape.page_tokens), int(max_pages_per_req),
                    int(device))


def _ptr(t, what, nbytes_elem=None, shape=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if nbytes_elem is not None and t.element_size() != nbytes_elem:
        raise ValueError(f"{what} must have {nbytes_elem}-byte elements, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


class Decoder:
    """A bound model: torch device tensors in, C-ABI handle out.

    ``weights`` maps "embed", "final_norm" (None without an embedding) and the
    stacked per-layer tensors "attn_norm" [L, H], "wqkv" [L, QKV, H], "wo"
    [L, H, nq d], "mlp_norm" [L, H], "w_gate" [L, F, H], "w_up" [L, F, H],
    "w_down" [L, H, F]; any 2-byte dtype holding bf16 patterns. The tensors are
    borrowed: keep them alive while the Decoder lives.
    """

    def __init__(self, shape, weights: Mapping[str, object], max_batch: int, max_pages_per_req: int,
                 device: int = 0):
        self.shape = shape
        self.cfg = make_config(shape, max_batch, max_pages_per_req, device)
        L, H, F = shape.n_layers, shape.hidden, shape.ffn
        QD = shape.n_q_heads * shape.head_dim
        QKV = (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim
        dims = {"attn_norm": (L, H), "wqkv": (L, QKV, H), "wo": (L, H, QD), "mlp_norm": (L, H),
                "w_gate": (L, F, H), "w_up": (L, F, H), "w_down": (L, H, F)}
        self._keep = dict(weights)
        layers = (MkLayerWeights * L)()
        for k in _LAYER_KEYS:
            t = weights[k]
            _ptr(t, k, 2, dims[k])
            stride = t[0].numel() * 2
            for l in range(L):
                setattr(layers[l], k, t.data_ptr() + l * stride)
        embed = final_norm = None
        if shape.has_embed:
            embed = _ptr(weights["embed"], "embed", 2, (shape.vocab, H))
            final_norm = _ptr(weights["final_norm"], "final_norm", 2, (H,))
        self._layers = layers
        self._w = MkWeights(embed, final_norm, ctypes.cast(layers, ctypes.POINTER(MkLayerWeights)))
        self.handle = mk_create(self.cfg, self._w)
        self.batch = 0

    def build_schedule(self, batch: int, mode: str = "megakernel", max_kv_len: int = 0, attn_chunks: int = 0,
                       n_cus: int = 0, trace: bool = False, watchdog_spins: int = 0,
                       attn_split: str = "balanced") -> dict:
        desc = MkScheduleDesc(batch, n_cus, _MODES[mode], max_kv_len, attn_chunks, int(trace), watchdog_spins,
                              _SPLITS[attn_split], 0)
        mk_build_schedule(self.handle, desc)
        self.batch = batch
        self.mode = mode
        return self.info()

    def step(self, *, kv_lens, k_pool, v_pool, page_table, tokens_in=None, hidden_in=None, tokens_out=None,
             kv_lens_out=None, logits_out=None, hidden_out=None, stream: Optional[int] = None,
             static_scratch: bool = False, n_steps: int = 1) -> None:
        """One step (mk_decode_step), or with ``static_scratch`` the
        allocation-free mk_decode_step_static, or with ``n_steps`` > 1 that
        many greedy steps in one resident launch (mk_decode_steps; tokens_out
        is then [n_steps, B])."""
        import torch
        s = self.shape
        B = self.batch
        pool_shape = (s.n_layers, k_pool.shape[1], s.n_kv_heads, s.page_tokens, s.head_dim)
        io = MkStepIO(
            _ptr(tokens_in, "tokens_in", 4, (B,)), _ptr(hidden_in, "hidden_in", 4, (B, s.hidden)),
            _ptr(kv_lens, "kv_lens", 4, (B,)), _ptr(k_pool, "k_pool", 2, pool_shape),
            _ptr(v_pool, "v_pool", 2, pool_shape), int(k_pool.shape[1]),
            _ptr(page_table, "page_table", 4, (B, self.cfg.max_pages_per_req)),
            _ptr(tokens_out, "tokens_out", 4, (n_steps, B) if n_steps > 1 else (B,)),
            _ptr(kv_lens_out, "kv_lens_out", 4, (B,)),
            _ptr(logits_out, "logits_out", 4, (B, s.vocab)), _ptr(hidden_out, "hidden_out", 4, (B, s.hidden)))
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        if n_steps != 1:  # the library checks the count
            if static_scratch:
                raise ValueError("the allocation-free entry point runs one step per call")
            mk_decode_steps(self.handle, io, int(n_steps), stream)
        else:
            (mk_decode_step_static if static_scratch else mk_decode_step)(self.handle, io, stream)

    def sync(self, stream: Optional[int] = None) -> None:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        mk_sync_status(self.handle, stream)

    def info(self) -> dict:
        return mk_get_schedule_info(self.handle).as_dict()

    def trace(self):
        return mk_read_trace(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            mk_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
