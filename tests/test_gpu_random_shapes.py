"""Seeded random shapes through the whole hot path, against the fp64 oracle:
stream counts, cache capacities (not multiples of 128), query positions
(block edges and position 0 included by chance) and top_k drawn per seed, so
that combinations the hand-picked cases do not name are exercised too.  The
tolerances are those of the other GPU parity tests.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_dsa import _dsa_parity
from test_gpu_msa import _decode_parity, _prefill_parity

pytestmark = pytest.mark.gpu


def _positions(rng, cap, n):
    pos = rng.integers(0, cap, size=n)
    # bias a third of the queries onto block edges
    edge = rng.random(n) < 0.33
    pos[edge] = np.clip((pos[edge] // 128) * 128 + rng.choice([-1, 0, 127], size=edge.sum()), 0, cap - 1)
    return tuple(int(p) for p in pos)


@pytest.mark.parametrize("seed", [101, 102, 103, 104, 105])
def test_random_msa_decode(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 9))
    cap = int(rng.integers(200, 9000))
    n_q = int(rng.integers(1, 20))
    top_k = int(rng.choice([1, 3, 16, 33, 64]))
    stream = tuple(int(s) for s in rng.integers(0, S, size=n_q))
    pos = _positions(rng, cap, n_q)
    # distinct (stream, position) pairs: the append writes each query's row
    pairs = {}
    for s, p in zip(stream, pos):
        pairs[(s, p)] = True
    stream, pos = zip(*pairs.keys())
    wl = W.Workload(f"rand{seed}", "msa_decode", S, cap, tuple(stream), tuple(pos), seed=seed, top_k=top_k)
    _decode_parity(wl)


@pytest.mark.parametrize("seed", [201, 202, 203])
def test_random_msa_prefill(seed):
    rng = np.random.default_rng(seed)
    cap = int(rng.integers(300, 6000))
    n_q = int(rng.integers(1, min(cap, 700)))
    pos0 = int(rng.integers(0, cap - n_q + 1))
    wl = W.prefill_workload(f"randpf{seed}", cap, pos0, n_q, seed=seed)
    _prefill_parity(wl)


@pytest.mark.parametrize("seed", [301, 302, 303])
def test_random_dsa_decode(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 5))
    cap = int(rng.integers(100, 12000))
    n_q = int(rng.integers(1, 9))
    top_k = int(rng.choice([1, 100, 2048, 4096]))
    stream = tuple(int(s) for s in rng.integers(0, S, size=n_q))
    pos = _positions(rng, cap, n_q)
    wl = W.Workload(f"randdsa{seed}", "dsa_decode", S, cap, stream, pos, seed=seed, top_k=top_k)
    _dsa_parity(wl)
