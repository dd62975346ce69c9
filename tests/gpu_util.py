"""Helpers shared by the GPU tests: the comparison bar against the oracle.
Device upload and the step runner live in the package (devio) and are
re-exported here for the tests."""
from __future__ import annotations

import numpy as np

from persistent_megakernel_decode_cu_amd.devio import (DevState, make_decoder, run_step, u16_to_dev,  # noqa: F401
                                                       upload_model)

LOGIT_TOL = 5e-2       # max |logit difference| allowed against the oracle
TOP2_GAP = 1e-2        # greedy tokens must match where the oracle's top-2 gap exceeds this


def top2_gap(logits_row: np.ndarray) -> float:
    f = logits_row.astype(np.float32)
    i = int(np.argmax(f))
    rest = np.delete(f, i)
    return float(f[i] - rest.max())


def check_logits(gpu_logits, ora_logits, gpu_tokens, ora_tokens, tol=LOGIT_TOL):
    """Returns (max |diff|, number of token mismatches that are allowed)."""
    diff = float(np.max(np.abs(gpu_logits.astype(np.float64) - ora_logits)))
    assert np.all(np.isfinite(gpu_logits)), "non-finite GPU logits"
    assert diff <= tol, f"max |logit diff| {diff} > {tol}"
    allowed = 0
    for b in range(len(ora_tokens)):
        if gpu_tokens[b] != ora_tokens[b]:
            gap = top2_gap(ora_logits[b])
            assert gap <= TOP2_GAP, f"token mismatch at request {b} with top-2 gap {gap}"
            allowed += 1
    return diff, allowed


def bf16_ulp_diff(a_u16: np.ndarray, b_u16: np.ndarray) -> int:
    """Largest distance in bf16 steps between two arrays of bf16 patterns
    (ordered as sign-magnitude integers)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7fff), x)
    return int(np.max(np.abs(key(a_u16) - key(b_u16)))) if a_u16.size else 0
