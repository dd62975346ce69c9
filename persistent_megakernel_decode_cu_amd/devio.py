"""Device plumbing around ``Decoder`` for callers that hold their model and
step state as host arrays: upload bf16 weight patterns and the step state
(K/V pools, page table, lengths, tokens) as torch device tensors, and run one
step into freshly allocated device outputs. Argument marshalling only; the
step itself runs in libmk.so.

``model`` is any object with ``cfg`` (the shape attributes ``make_config``
reads) and ``weights`` (name -> uint16 array of bf16 patterns, or None);
``state`` any object with ``kv_lens``, ``k_pool``, ``v_pool``,
``page_table``, ``tokens`` and ``hidden_in`` arrays.
"""
from __future__ import annotations

import numpy as np
import torch

from . import Decoder


def u16_to_dev(a: np.ndarray) -> torch.Tensor:
    """bf16 patterns (uint16) as a 2-byte device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def upload_model(model) -> dict:
    return {k: (None if v is None else u16_to_dev(v)) for k, v in model.weights.items()}


class DevState:
    """Device copies of one step's state."""

    def __init__(self, st):
        self.kv_lens = torch.from_numpy(st.kv_lens.copy()).cuda()
        self.k_pool = u16_to_dev(st.k_pool)
        self.v_pool = u16_to_dev(st.v_pool)
        self.page_table = torch.from_numpy(st.page_table.copy()).cuda()
        self.tokens = torch.from_numpy(st.tokens.copy()).cuda()
        self.hidden_in = None if st.hidden_in is None else torch.from_numpy(st.hidden_in.copy()).cuda()


def make_decoder(model, st, wdev, max_batch=None) -> Decoder:
    return Decoder(model.cfg, wdev, max_batch=max_batch or st.batch, max_pages_per_req=st.page_table.shape[1])


def run_step(dec: Decoder, ds: DevState, cfg, want_logits=True, want_hidden=False) -> dict:
    """One step on the current stream, synchronised; outputs as host arrays
    (tokens, kv_lens, and logits / hidden when asked for)."""
    B = ds.kv_lens.shape[0]
    out = {"tokens": torch.full((B,), -1, dtype=torch.int32, device="cuda"),
           "kv_lens": torch.zeros(B, dtype=torch.int32, device="cuda")}
    if want_logits and cfg.has_embed:
        out["logits"] = torch.full((B, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    if want_hidden or not cfg.has_embed:
        out["hidden"] = torch.full((B, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
    dec.step(kv_lens=ds.kv_lens, k_pool=ds.k_pool, v_pool=ds.v_pool, page_table=ds.page_table,
             tokens_in=ds.tokens if cfg.has_embed else None, hidden_in=ds.hidden_in,
             tokens_out=out["tokens"] if cfg.has_embed else None, kv_lens_out=out["kv_lens"],
             logits_out=out.get("logits"), hidden_out=out.get("hidden"))
    dec.sync()
    return {k: v.cpu().numpy() for k, v in out.items()}
