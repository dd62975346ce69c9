"""The five decode workloads: model shape, batch, K/V lengths, steps.

All stand in for the Llama-3.2-1B batch-1 case that the page "Inference
MegaKernel" (shaojiemike.top) quotes in its sections "why conventional
inference still has bubbles" and "hand-written whole-model MegaKernel /
effects and applicability", with random weights of that shape.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    cid: int                 # seed id of the workload
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int               # 0 when the model has no embedding / head
    has_embed: bool
    batch: int
    kv_len: int = 0          # fixed prefilled length (all requests)
    kv_len_range: tuple = field(default=())   # (lo, hi) inclusive, per request
    steps: int = 1           # decode steps the workload runs
    paged_random: bool = False
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    page_tokens: int = 16

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def weight_bytes(self) -> int:
        """bf16 bytes of every weight tensor the step streams once."""
        H, F, L = self.hidden, self.ffn, self.n_layers
        per_layer = 2 * (self.qkv_rows * H + H * self.n_q_heads * self.head_dim + 3 * H * F) + 4 * H
        total = L * per_layer
        if self.has_embed:
            total += 2 * self.vocab * H + 2 * H   # LM head (tied embedding) + final norm
        return total


WORKLOADS = {
    # tiny correctness model
    "tiny-2l": Workload(1, "tiny-2l", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2,
                        head_dim=64, ffn=1024, vocab=4096, has_embed=True, batch=1,
                        kv_len=64, steps=1),
    # one layer of the 1B shape, no embedding or head, hidden vector in/out
    "1b-layer-kv512": Workload(2, "1b-layer-kv512", n_layers=1, hidden=2048, n_q_heads=32,
                               n_kv_heads=8, head_dim=64, ffn=8192, vocab=0, has_embed=False,
                               batch=1, kv_len=512, steps=1),
    # the headline case: 16-layer 1B shape at batch 1, 128 greedy steps
    "1b-kv1024": Workload(3, "1b-kv1024", n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8,
                          head_dim=64, ffn=8192, vocab=128256, has_embed=True, batch=1,
                          kv_len=1024, steps=128),
    "1b-kv8192": Workload(4, "1b-kv8192", n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8,
                          head_dim=64, ffn=8192, vocab=128256, has_embed=True, batch=1,
                          kv_len=8192, steps=128),
    "1b-b8-paged": Workload(5, "1b-b8-paged", n_layers=16, hidden=2048, n_q_heads=32,
                            n_kv_heads=8, head_dim=64, ffn=8192, vocab=128256, has_embed=True,
                            batch=8, kv_len_range=(128, 4096), steps=1, paged_random=True),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
