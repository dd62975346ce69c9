"""Seeded synthetic inputs for the decode step: model shapes, random-init
weights, prefilled K/V caches, page tables, tokens and lengths.

This module holds none of the decode arithmetic. Both the CPU oracle (in the
tests) and the HIP library (through its Python binding) receive the same
bytes from here. Nothing here is a trained model or a dataset: the page
"Inference MegaKernel" (shaojiemike.top), section "hand-written whole-model
MegaKernel / effects and applicability", measures on Llama-3.2-1B at batch 1;
these generators stand in for it with random weights of the same shape.

Recipe (per workload id `cid`, numpy PCG64 seeded with ``[cid, stream]``):

* stream 0, weights, in this order: embedding [V, H] (if the model has one),
  then per layer: attention norm (all 1.0), Wq, Wk, Wv, Wo, MLP norm (all
  1.0), Wgate, Wup, Wdown; then the final norm (all 1.0). Every matrix entry
  is N(0, 0.02) drawn in binary32 and kept as its upper 16 bits (bf16 by
  truncation toward zero).
* stream 1, K/V pools: every entry N(0, 1), bf16 by truncation, K pool then
  V pool.
* stream 2, tokens: uniform in [0, V).
* stream 3, lengths: the workload's fixed length, or uniform in [lo, hi]
  per request.
* stream 4, page table: a random permutation of the pool's pages handed out
  request by request, or the identity for contiguous workloads.
* stream 5, hidden input of the one-layer block: N(0, 1) binary32.
"""
from .configs import WORKLOADS, Workload, workload  # noqa: F401
from .gen import Model, State, make_model, make_state, sha256_of  # noqa: F401
