"""The attention split as the device computes it (mk_debug_attn_split runs
the same device function the interpreter and the unfused kernels use)
against the rule stated in tests/attn_split_ref.py, through the C ABI, on
random and edge-case batches of lengths."""
import random

import numpy as np
import pytest
import torch

from persistent_megakernel_decode_cu_amd import _mk
from tests import attn_split_ref as ref

pytestmark = pytest.mark.gpu

CAP = 65535 * 16


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _device_split(cases, T, mode, cap=CAP):
    B = len(cases[0])
    kv = torch.tensor(np.asarray(cases, dtype=np.int32), device="cuda")
    out = torch.full((len(cases), 4 * T + B + 1), -7, dtype=torch.int32, device="cuda")
    _mk.mk_debug_attn_split(kv.data_ptr(), len(cases), B, T, mode, cap, out.data_ptr())
    return out.cpu().numpy()


def _expect(kv, T, balanced, cap=CAP):
    tiles, first = ref.split(kv, T, balanced, cap)
    return np.array([w for t in tiles for w in (t[0], t[1], t[2], int(t[3]))] + first, dtype=np.int32)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("B,C", [(1, 16), (2, 16), (3, 8), (4, 8), (5, 3), (8, 4), (8, 8), (8, 16), (7, 1)])
def test_random_batches(mode, B, C):
    rng = random.Random(B * 100 + C * 7 + mode)
    T = B * C
    cases = []
    for _ in range(300):
        kind = rng.random()
        if kind < 0.3:
            kv = [rng.randint(0, 4096) for _ in range(B)]
        elif kind < 0.6:  # one long request among short ones
            kv = [rng.randint(0, 40) for _ in range(B)]
            kv[rng.randrange(B)] = rng.randint(1000, 200000)
        elif kind < 0.8:
            kv = [rng.choice([0, 15, 16, 31, 32]) for _ in range(B)]
        else:
            kv = [rng.randint(0, CAP + 100) for _ in range(B)]  # beyond the capacity: clamped
        cases.append(kv)
    got = _device_split(cases, T, mode)
    for i, kv in enumerate(cases):
        want = _expect(kv, T, mode == 0)
        assert np.array_equal(got[i], want), (kv, T, mode)


def test_edge_batches():
    cases = {
        (8, 32): [[3982, 2953, 1262, 306, 3951, 2664, 288, 1678], [0] * 8, [CAP - 1] * 8,
                  [CAP - 1] + [0] * 7, [0] * 7 + [CAP - 1], [-5] * 8],
        (8, 8): [[100, 200, 300, 400, 500, 600, 700, 800], [0] * 8],
        (1, 1): [[0], [5000], [CAP - 1]],
        (2, 128 // 2 * 2): [[0, CAP - 1], [CAP - 1, CAP - 1]],
    }
    for (B, T), cs in cases.items():
        got = _device_split(cs, T, 0)
        for i, kv in enumerate(cs):
            assert np.array_equal(got[i], _expect(kv, T, True)), (kv, T)


def test_rejects_bad_arguments():
    kv = torch.zeros(8, dtype=torch.int32, device="cuda")
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for B, T, mode in ((0, 8, 0), (9, 72, 0), (8, 4, 0), (8, 129, 0), (3, 8, 1), (2, 8, 2)):
        with pytest.raises(_mk.MkError):
            _mk.mk_debug_attn_split(kv.data_ptr(), 1, B, T, mode, CAP, out.data_ptr())
