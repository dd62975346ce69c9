"""Seeded generators (see the package docstring for the recipe)."""
from __future__ import annotations

import hashlib
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from .configs import Workload

_CHUNK = 1 << 24
_ONE_BF16 = np.uint16(0x3F80)


def _rng(cid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cid, stream])


def _fill_normal_bf16(rng: np.random.Generator, out: np.ndarray, sigma: float) -> None:
    """Fill a uint16 array with bf16 patterns of N(0, sigma) draws: binary32
    draws, scaled in binary32, truncated to their upper 16 bits."""
    flat = out.reshape(-1)
    s = np.float32(sigma)
    for i in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - i)
        x = rng.standard_normal(n, dtype=np.float32)
        if sigma != 1.0:
            x *= s
        flat[i:i + n] = (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Model:
    cfg: Workload
    weights: Dict[str, Optional[np.ndarray]]

    def layer(self, name: str, l: int) -> np.ndarray:
        return self.weights[name][l]


@dataclass
class State:
    batch: int
    tokens: np.ndarray          # int32 [B]
    kv_lens: np.ndarray         # int32 [B]
    k_pool: np.ndarray          # uint16 [L, n_pages, nkv, page_tokens, d]
    v_pool: np.ndarray
    page_table: np.ndarray      # int32 [B, max_pages_per_req]
    n_pages: int
    hidden_in: Optional[np.ndarray]  # float32 [B, H] for models without embedding

    def copy(self) -> "State":
        return State(self.batch, self.tokens.copy(), self.kv_lens.copy(), self.k_pool.copy(),
                     self.v_pool.copy(), self.page_table.copy(), self.n_pages,
                     None if self.hidden_in is None else self.hidden_in.copy())


def make_model(cfg: Workload, sigma: float = 0.02) -> Model:
    rng = _rng(cfg.cid, 0)
    L, H, F, d = cfg.n_layers, cfg.hidden, cfg.ffn, cfg.head_dim
    nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
    w: Dict[str, Optional[np.ndarray]] = {}
    w["embed"] = None
    if cfg.has_embed:
        w["embed"] = np.empty((cfg.vocab, H), dtype=np.uint16)
        _fill_normal_bf16(rng, w["embed"], sigma)
    w["attn_norm"] = np.empty((L, H), dtype=np.uint16)
    w["wqkv"] = np.empty((L, cfg.qkv_rows, H), dtype=np.uint16)
    w["wo"] = np.empty((L, H, nq * d), dtype=np.uint16)
    w["mlp_norm"] = np.empty((L, H), dtype=np.uint16)
    w["w_gate"] = np.empty((L, F, H), dtype=np.uint16)
    w["w_up"] = np.empty((L, F, H), dtype=np.uint16)
    w["w_down"] = np.empty((L, H, F), dtype=np.uint16)
    for l in range(L):
        w["attn_norm"][l] = _ONE_BF16
        _fill_normal_bf16(rng, w["wqkv"][l, : nq * d], sigma)              # Wq
        _fill_normal_bf16(rng, w["wqkv"][l, nq * d:(nq + nkv) * d], sigma)  # Wk
        _fill_normal_bf16(rng, w["wqkv"][l, (nq + nkv) * d:], sigma)        # Wv
        _fill_normal_bf16(rng, w["wo"][l], sigma)
        w["mlp_norm"][l] = _ONE_BF16
        _fill_normal_bf16(rng, w["w_gate"][l], sigma)
        _fill_normal_bf16(rng, w["w_up"][l], sigma)
        _fill_normal_bf16(rng, w["w_down"][l], sigma)
    w["final_norm"] = np.full(H, _ONE_BF16, dtype=np.uint16) if cfg.has_embed else None
    return Model(cfg, w)


def make_state(cfg: Workload, extra_positions: Optional[int] = None) -> State:
    """Prefilled cache, lengths, page table and inputs. Each request gets
    pages for its length plus ``extra_positions`` (default: the workload's
    step count) new positions."""
    B, L, T = cfg.batch, cfg.n_layers, cfg.page_tokens
    extra = cfg.steps if extra_positions is None else extra_positions
    if cfg.kv_len_range:
        lo, hi = cfg.kv_len_range
        lens = _rng(cfg.cid, 3).integers(lo, hi, endpoint=True, size=B).astype(np.int32)
    else:
        lens = np.full(B, cfg.kv_len, dtype=np.int32)
    pages_per_req = [(int(n) + extra + T - 1) // T for n in lens]
    max_pages = max(pages_per_req)
    n_pages = int(sum(pages_per_req))
    if cfg.paged_random:
        perm = _rng(cfg.cid, 4).permutation(n_pages).astype(np.int32)
    else:
        perm = np.arange(n_pages, dtype=np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        page_table[b, : pages_per_req[b]] = perm[at: at + pages_per_req[b]]
        at += pages_per_req[b]
    shape = (L, n_pages, cfg.n_kv_heads, T, cfg.head_dim)
    rng = _rng(cfg.cid, 1)
    k_pool = np.empty(shape, dtype=np.uint16)
    v_pool = np.empty(shape, dtype=np.uint16)
    _fill_normal_bf16(rng, k_pool, 1.0)
    _fill_normal_bf16(rng, v_pool, 1.0)
    tokens = np.zeros(B, dtype=np.int32)
    hidden_in = None
    if cfg.has_embed:
        tokens = _rng(cfg.cid, 2).integers(0, cfg.vocab, size=B).astype(np.int32)
    else:
        hidden_in = _rng(cfg.cid, 5).standard_normal((B, cfg.hidden), dtype=np.float32)
    return State(B, tokens, lens, k_pool, v_pool, page_table, n_pages, hidden_in)


def sha256_of(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is None:
            h.update(b"none")
        else:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
