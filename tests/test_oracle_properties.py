"""Property-based pins of the CPU oracle (no GPU): shapes and id patterns drawn at random
beyond the two-rank brute force -- one to six ranks, empty ranks, top-k up to four,
repeated ids within a token, ids outside [0, E) and receive capacities below the rows
sent -- each checked against the nested-loop formulation in ``oracle.naive`` (rows
appended to lists in the order the definition fixes: no counts, offsets or cursors).

Definition: abhik.ai "Collective Communication for 100k+ GPUs", section "Inference: small
messages, unknown sizes", Figure 13 (tokens sorted by expert into a send buffer, an
all-to-allv to the rank holding each expert, received counts returned).
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import naive


def _tags(R, T):
    """int32 rows [s, t, s*T + t]: every received row names its token."""
    x = np.zeros((R, T, 3), np.int32)
    x[:, :, 0] = np.arange(R)[:, None]
    x[:, :, 1] = np.arange(T)[None, :]
    x[:, :, 2] = np.arange(R)[:, None] * T + np.arange(T)[None, :]
    return x


@st.composite
def routings(draw):
    R = draw(st.integers(1, 6))
    T = draw(st.integers(0, 6))
    epr = draw(st.integers(1, 4))
    E = R * epr
    k = draw(st.integers(1, min(4, E)))
    # ids mostly in range, sometimes one step outside it on either side
    ids = np.array(draw(st.lists(st.integers(-1, E), min_size=R * T * k, max_size=R * T * k)),
                   np.int32).reshape(R, T, k)
    worst = R * T * min(k, epr)
    cap = draw(st.integers(0, worst)) if worst else 0
    layout = draw(st.sampled_from([oracle.SOURCE_MAJOR, oracle.EXPERT_MAJOR]))
    return R, T, k, epr, ids, cap, layout


@settings(max_examples=400, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(routings())
def test_oracle_dispatch_matches_nested_loops(case):
    R, T, k, epr, ids, cap, layout = case
    E = R * epr
    d = oracle.dispatch(oracle.as_rows(_tags(R, T)), ids, epr, cap, layout=layout)
    send = d["send"].view(np.int32).reshape(R, T * k, 3)
    recv = d["recv"].view(np.int32).reshape(R, cap, 3)
    sl = naive.send_lists(ids, R, T, k, epr)
    rl = (naive.recv_lists_expert_major if layout == oracle.EXPERT_MAJOR else naive.recv_lists)(
        ids, R, T, k, epr)
    # send order and positions; dropped (out-of-range) slots have no place
    for s in range(R):
        placed = set()
        for p, (t, j) in enumerate(sl[s]):
            assert d["pos"][s, t, j] == p
            assert send[s, p, 0] == s and send[s, p, 1] == t
            placed.add((t, j))
        for t in range(T):
            for j in range(k):
                if (t, j) not in placed:
                    assert d["pos"][s, t, j] == -1
        # the split table counts rows per (sender, expert)
        for e in range(E):
            assert d["cnt"][s, e] == sum(1 for (t, j) in sl[s] if ids[s, t, j] == e)
    # receive counts stay true past the capacity; only the first `cap` rows are written
    for dst in range(R):
        assert d["recv_off"][dst, R] == len(rl[dst])
        for s in range(R):
            assert d["recv_counts"][dst, s] == sum(1 for r in rl[dst] if r[0] == s)
        for q, (s, t, j, e) in enumerate(rl[dst][:cap]):
            assert recv[dst, q, 0] == s and recv[dst, q, 1] == t and recv[dst, q, 2] == s * T + t
    bad = bool(((ids < 0) | (ids >= E)).any())
    over = any(len(rl[dst]) > cap for dst in range(R))
    expect = (oracle.ST_EXPERT_RANGE if bad else 0) | (oracle.ST_RECV_OVERFLOW if over else 0)
    assert d["status"] == expect
