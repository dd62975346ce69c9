"""The attention split, stated directly (test helper, CPU only).

Each kv head has T attention tiles; at every step they are shared out over
the batch's requests from their current lengths (mk_attn_split in mk.h).
Request b, whose newest position is p_b, covers nb_b = ceil((p_b + 1) / 16)
K/V blocks.

* balanced: s is the smallest tile size (in blocks) for which
  sum_b ceil(nb_b / s) <= T, found here by trying s = 1, 2, ...; request b
  gets ceil(nb_b / s) tiles, and the spare tiles go to the request with the
  most blocks (the lowest index among equals);
* per_request: T / B tiles each.

Tiles are numbered request by request; tile j of request b's n_b covers
blocks [j nb_b / n_b, (j + 1) nb_b / n_b) (floors), and the last of them
holds the request's newest position.
"""
from __future__ import annotations


def n_blocks(p: int, capacity: int) -> int:
    p = min(max(p, 0), capacity - 1)
    return (p + 16) // 16


def tile_counts(nb: list, T: int, balanced: bool = True) -> list:
    B = len(nb)
    assert 1 <= B <= T
    if not balanced:
        assert T % B == 0
        return [T // B] * B
    s = 1
    while sum(-(-x // s) for x in nb) > T:
        s += 1
    n = [-(-x // s) for x in nb]
    big = max(range(B), key=lambda b: (nb[b], -b))
    n[big] += T - sum(n)
    return n


def split(kv_lens, T: int, balanced: bool = True, capacity: int = 1 << 20):
    """Returns (tiles, first): tiles[t] = (request, lo, hi, last);
    first[b] = the request's first tile (first[B] = T)."""
    nb = [n_blocks(int(p), capacity) for p in kv_lens]
    n = tile_counts(nb, T, balanced)
    tiles, first = [], [0]
    for b, (x, k) in enumerate(zip(nb, n)):
        for j in range(k):
            tiles.append((b, j * x // k, (j + 1) * x // k, j == k - 1))
        first.append(first[-1] + k)
    return tiles, first
