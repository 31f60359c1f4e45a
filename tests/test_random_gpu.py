"""Seeded random steps through the HIP path (the C ABI), compared with the CPU oracle.

Each case draws, from its own seed, a shape, a routing and a receive capacity: one to 32
ranks, empty ranks, rows of 2 to 2,560 bytes (every vector width), top-k up to 8 with
distinct experts, with experts repeated inside a token, or with one id in ten outside
[0, E), and receive capacities from the worst case down to a single row.  Every case is
one dispatch -> expert stand-in -> combine on both data paths and both receive layouts,
compared with the oracle element by element: tables, positions, receive rows and expert
rows bit-exact, the combine within the tolerance of tests/gpu_util.py.

Definition under test: abhik.ai "Collective Communication for 100k+ GPUs", section
"Inference: small messages, unknown sizes", Figure 13, and the combine of
qiguanping.github.io "NCCLX", section 7, figure 13.
"""
import numpy as np
import pytest

import oracle
from moe_alltoallv_resident_amd import workloads as W
from tests.test_parity_gpu import LAYOUT_IDS, LAYOUTS, PATH_IDS, PATHS, _full_oracle_check

pytestmark = pytest.mark.gpu

CASES = 120


def drawn_step(i):
    """Case i: (workload, x, ids, gates), everything from seed i."""
    rng = np.random.default_rng([4242, i])
    R = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16, 32]))
    epr = int(rng.integers(1, 9))
    E = R * epr
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([0, 1, 2, 5, 17, 64, 129, 300]))
    dtype = int(rng.choice([W.F32, W.BF16]))
    H = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 99, 100, 129, 640]))
    mode = int(rng.choice([W.EXPERT_IDENTITY, W.EXPERT_SCALE]))
    worst = R * T * min(k, epr)
    shift = int(rng.integers(0, 4))                     # 0: worst case; else a quarter, a sixteenth, ...
    cap = max(1, worst >> (2 * shift)) if worst and shift else 0
    w = W.Workload(f"drawn{i}", R, T, H, dtype, epr, k, "uniform", "softmax", mode, seed=10_000 + i,
                   recv_capacity_rows=cap)
    x, ids, gates = W.make_inputs(w)
    kind = ("distinct", "repeats", "out-of-range")[i % 3]
    if kind != "distinct" and ids.size:
        ids = rng.integers(0, E, size=ids.shape).astype(np.int32)       # experts repeat in a token
        if kind == "out-of-range":
            hit = rng.random(ids.shape) < 0.1
            ids[hit] = rng.choice(np.array([-1, E, E + 5, -(1 << 20)], np.int32), size=int(hit.sum()))
    return w, x, ids, gates


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("i", range(CASES))
def test_drawn_steps_match_oracle(i, path, layout):
    w, x, ids, gates = drawn_step(i)
    ref = _full_oracle_check(w, x, ids, gates, path, layout)
    bad = bool(((ids < 0) | (ids >= w.num_experts)).any())
    assert bool(ref["status"] & oracle.ST_EXPERT_RANGE) == bad
