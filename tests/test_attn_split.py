"""The attention split's rule (tests/attn_split_ref.py) against what it
must achieve, on the CPU: every request's blocks covered once and in order,
the newest position in the request's last tile, every request at least one
tile, all T tiles used, and - the point of the balanced mode - the largest
tile no larger than under any other way of handing T tiles to the requests
(found by brute force on small cases). The device's own computation of the
split is compared with this rule in tests/test_gpu_split.py."""
import itertools
import random

import pytest

from tests import attn_split_ref as ref


def _check_cover(kv_lens, T, balanced):
    tiles, first = ref.split(kv_lens, T, balanced)
    assert len(tiles) == T and first[-1] == T and len(first) == len(kv_lens) + 1
    for b, p in enumerate(kv_lens):
        mine = tiles[first[b]:first[b + 1]]
        assert len(mine) >= 1 and all(t[0] == b for t in mine)
        nb = (p + 16) // 16
        at = 0
        for (_, lo, hi, _) in mine:
            assert lo == at and hi >= lo
            at = hi
        assert at == nb
        # exactly the last tile is marked, and it holds block nb - 1 (position p)
        assert [t[3] for t in mine] == [False] * (len(mine) - 1) + [True]
        assert mine[-1][1] <= p // 16 < mine[-1][2]
    return tiles


def _max_tile(tiles):
    return max(hi - lo for (_, lo, hi, _) in tiles)


@pytest.mark.parametrize("balanced", [True, False])
def test_cover_random(balanced):
    rng = random.Random(5)
    for _ in range(400):
        B = rng.randint(1, 8)
        C = rng.randint(1, 16)
        kv = [rng.choice([0, 1, 15, 16, 17, rng.randint(0, 300), rng.randint(0, 70000)]) for _ in range(B)]
        _check_cover(kv, B * C, balanced)


def test_balanced_is_optimal_by_brute_force():
    """No allocation of T tiles (each request at least one, blocks cut as
    evenly as the rule cuts them) has a smaller largest tile."""
    rng = random.Random(11)
    for _ in range(150):
        B = rng.randint(1, 4)
        T = rng.randint(B, 9)
        kv = [rng.randint(0, 200) for _ in range(B)]
        nb = [(p + 16) // 16 for p in kv]
        best = min(max(-(-x // k) for x, k in zip(nb, alloc))
                   for alloc in itertools.product(range(1, T + 1), repeat=B) if sum(alloc) == T)
        assert _max_tile(_check_cover(kv, T, True)) == best, (kv, T)


def test_single_request_is_the_even_cut():
    # one request: tile t of T takes blocks [t nb / T, (t + 1) nb / T)
    for p in (0, 7, 16, 1000, 4095):
        nb = (p + 16) // 16
        for T in (1, 3, 16):
            tiles, _ = ref.split([p], T)
            assert [(lo, hi) for (_, lo, hi, _) in tiles] == [(t * nb // T, (t + 1) * nb // T) for t in range(T)]


def test_skewed_batch_example():
    # eight requests of 288..3982 positions, 32 tiles: the balanced split
    # keeps every tile within 37 blocks (the per-request split of 4 tiles
    # each gives the longest request's tiles 63 blocks)
    kv = [3982, 2953, 1262, 306, 3951, 2664, 288, 1678]
    bal = _check_cover(kv, 32, True)
    per = _check_cover(kv, 32, False)
    assert _max_tile(bal) == 37
    assert _max_tile(per) == 63
    assert ref.tile_counts([(p + 16) // 16 for p in kv], 32) == [7, 5, 3, 1, 7, 5, 1, 3]


def test_spare_tiles_go_to_the_longest_request():
    # all requests of one block: s = 1, one tile each, and the 5 spare tiles
    # to request 0 (the lowest index among the longest)
    assert ref.tile_counts([1, 1, 1], 8) == [6, 1, 1]
    assert ref.tile_counts([1, 5, 5], 8) == [1, 4, 3]


def test_lengths_are_clamped_to_the_capacity():
    assert ref.n_blocks(-3, 64) == 1
    assert ref.n_blocks(10 ** 6, 64) == 4
