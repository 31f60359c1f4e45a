"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test fixes part of the oracle with a library routine, a closed form, an invariant
that the definition implies, exact rational arithmetic, brute-force search, or the
independent nested-loop formulation in ``oracle.naive``.  The definition being pinned:
abhik.ai "Collective Communication for 100k+ GPUs", section "Inference: small messages,
unknown sizes" (Figure 13) -- tokens sorted by expert into a send buffer, an all-to-allv
to the rank holding each expert, received counts returned; the combine merges each
token's k expert outputs (qiguanping.github.io "NCCLX", section 7, figure 13).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import naive
from moe_alltoallv_resident_amd import workloads as W


# ----------------------------------------------------------------------------- helpers

def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    ok = np.isfinite(f)
    return bits[ok].astype(np.uint16), f[ok].astype(np.float64)


_BF16_BITS, _BF16_VALS = _all_finite_bf16()
_ORDER = np.argsort(_BF16_VALS, kind="stable")


def _nearest_bf16_bruteforce(v: float) -> int:
    """Nearest finite bf16 to v by search over every finite bf16 value; ties go to the
    pattern whose last stored fraction bit is 0.  -0.0 and +0.0 compare equal; the sign
    of v decides."""
    vals = _BF16_VALS[_ORDER]
    bits = _BF16_BITS[_ORDER]
    i = np.searchsorted(vals, v)
    cands = [c for c in (i - 2, i - 1, i, i + 1) if 0 <= c < len(vals)]
    best = min(abs(vals[c] - v) for c in cands)
    near = [c for c in cands if abs(vals[c] - v) == best]
    signed_zero = 0x8000 if np.signbit(v) else 0
    near_bits = sorted({signed_zero if vals[c] == 0.0 else int(bits[c]) for c in near})
    if len(near_bits) == 1:
        return near_bits[0]
    even = [b for b in near_bits if (b & 1) == 0]
    assert len(even) == 1
    return even[0]


def _tags(R, T, width):
    """Row payload that names its token: int32 row [s, t, s*T+t, ...] padded to width."""
    x = np.zeros((R, T, width), np.int32)
    s = np.arange(R)[:, None]
    t = np.arange(T)[None, :]
    x[:, :, 0] = s
    x[:, :, 1] = t
    if width > 2:
        x[:, :, 2] = s * T + t
    for c in range(3, width):
        x[:, :, c] = (s * 7919 + t * 104729 + c) & 0x7FFFFFFF
    return x


def _random_ids(rng, R, T, k, E, distinct=True):
    if distinct:
        return np.argsort(rng.random((R * T, E)), axis=1)[:, :k].reshape(R, T, k).astype(np.int32)
    return rng.integers(0, E, size=(R, T, k)).astype(np.int32)


# ----------------------------------------------------------------------- number format

def test_bf16_to_double_is_exact_for_every_pattern():
    for b in list(range(0, 1 << 16, 251)) + [0x0000, 0x8000, 0x0001, 0x7F7F, 0xFF7F, 0x3F80]:
        f = np.array([b << 16], np.uint32).view(np.float32)[0]
        if np.isfinite(f):
            assert oracle.bf16_to_double(b) == float(f)


def test_double_to_bf16_matches_bruteforce_nearest():
    rng = np.random.default_rng(123)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-40, 40, 3000)))
    # exact ties between two neighbouring bf16 values, both parities, both signs
    for b in rng.integers(0x0080, 0x7F00, 400):
        lo = float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(int(b) + 1) << 16], np.uint32).view(np.float32)[0])
        vals += [(lo + hi) / 2, -(lo + hi) / 2, lo + (hi - lo) * 0.4999, lo + (hi - lo) * 0.5001]
    # subnormal range and a value just below the largest finite bf16
    vals += [1e-39, -3e-40, 2.0 ** -133, 2.0 ** -134, 3.38e38, 0.0, -0.0]
    for v in vals:
        assert oracle.double_to_bf16(v) == _nearest_bf16_bruteforce(v), v


def test_double_to_bf16_matches_torch_for_float32_values():
    # torch's float32 -> bfloat16 cast rounds to nearest even; on values that are
    # already float32 there is no double rounding, so the two must agree exactly.
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------ counts and offset tables

@pytest.mark.parametrize("R,T,k,epr,seed", [(1, 40, 1, 4, 0), (2, 33, 2, 3, 1), (4, 64, 2, 2, 2),
                                            (8, 17, 3, 4, 3), (16, 5, 8, 16, 4), (64, 3, 2, 1, 5),
                                            (3, 0, 2, 2, 6)])
def test_tables_match_bincount_and_cumsum(R, T, k, epr, seed):
    rng = np.random.default_rng(seed)
    E = R * epr
    ids = _random_ids(rng, R, T, min(k, E), E)
    k = ids.shape[2]
    d = oracle.dispatch(oracle.as_rows(_tags(R, T, 3)), ids, epr, cap=R * T * k)
    assert d["status"] == 0
    for s in range(R):
        c = np.bincount(ids[s].ravel(), minlength=E)
        assert np.array_equal(d["cnt"][s], c)
        per_dst = c.reshape(R, epr).sum(axis=1)
        assert np.array_equal(d["send_off"][s], np.concatenate([[0], np.cumsum(per_dst)]))
    # received counts are the transposed per-destination sends
    per_dst_all = d["cnt"].reshape(R, R, epr).sum(axis=2)          # [src][dst]
    assert np.array_equal(d["recv_counts"], per_dst_all.T)
    assert np.array_equal(d["recv_off"], np.concatenate(
        [np.zeros((R, 1), np.int64), np.cumsum(d["recv_counts"], axis=1)], axis=1))
    # conservation: everything sent is received
    assert d["recv_counts"].sum() == R * T * k == d["recv_off"][:, R].sum()


def test_send_order_at_one_rank_is_a_stable_argsort():
    rng = np.random.default_rng(11)
    T, k, E = 300, 3, 7
    ids = _random_ids(rng, 1, T, k, E, distinct=False)
    x = _tags(1, T, 3)
    d = oracle.dispatch(oracle.as_rows(x), ids, E, cap=T * k)
    order = np.argsort(ids.ravel(), kind="stable")                 # assignment index per place
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(d["pos"].ravel(), inv)
    send = d["send"].view(np.int32).reshape(T * k, 3)
    assert np.array_equal(send[:, 1], order // k)
    # one rank talks to itself: the receive buffer is the send buffer
    assert np.array_equal(d["recv"], d["send"])


# ----------------------------------------------------------------------- tagged rows

@pytest.mark.parametrize("R,T,k,epr,seed", [(2, 50, 2, 2, 0), (4, 64, 2, 2, 1), (8, 40, 1, 16, 2),
                                            (16, 12, 8, 16, 3), (64, 8, 2, 1, 4), (5, 9, 5, 1, 5)])
def test_tagged_rows_each_token_arrives_k_times_in_its_segment(R, T, k, epr, seed):
    rng = np.random.default_rng(seed)
    E = R * epr
    ids = _random_ids(rng, R, T, k, E)
    cap = R * T * min(k, epr)
    d = oracle.dispatch(oracle.as_rows(_tags(R, T, 4)), ids, epr, cap)
    recv = d["recv"].view(np.int32).reshape(R, cap, 4)
    seen = np.zeros((R, T), np.int64)
    for dst in range(R):
        for src in range(R):
            lo, hi = d["recv_off"][dst, src], d["recv_off"][dst, src + 1]
            rows = recv[dst, lo:hi]
            assert np.all(rows[:, 0] == src)
            # with one slot per token, rows inside a source segment are sorted by expert
            if k == 1:
                assert np.all(np.diff(ids[src, rows[:, 1], 0]) >= 0)
            for s_, t_ in rows[:, :2]:
                seen[s_, t_] += 1
                assert dst in (ids[s_, t_] // epr)
    expect = np.zeros((R, T), np.int64)
    for s_ in range(R):
        for t_ in range(T):
            expect[s_, t_] = k
    assert np.array_equal(seen, expect)
    # every payload word survives (rows are copied, not rebuilt)
    full = _tags(R, T, 4)
    for dst in range(R):
        n = d["recv_off"][dst, R]
        rows = recv[dst, :n]
        assert np.array_equal(rows, full[rows[:, 0], rows[:, 1]])


# -------------------------------------------------- brute force against nested loops

def _check_against_naive(ids, R, T, k, epr):
    E = R * epr
    x = _tags(R, T, 3)
    cap = R * T * k
    d = oracle.dispatch(oracle.as_rows(x), ids, epr, cap)
    sl = naive.send_lists(ids, R, T, k, epr)
    rl = naive.recv_lists(ids, R, T, k, epr)
    send = d["send"].view(np.int32).reshape(R, T * k, 3)
    recv = d["recv"].view(np.int32).reshape(R, cap, 3)
    for s in range(R):
        for p, (t, j) in enumerate(sl[s]):
            assert d["pos"][s, t, j] == p
            assert send[s, p, 1] == t
        placed = {(t, j) for (t, j) in sl[s]}
        for t in range(T):
            for j in range(k):
                if (t, j) not in placed:
                    assert d["pos"][s, t, j] == -1
    for dst in range(R):
        assert d["recv_off"][dst, R] == len(rl[dst])
        for q, (s, t, j, e) in enumerate(rl[dst]):
            assert recv[dst, q, 0] == s and recv[dst, q, 1] == t
        for s in range(R):
            assert d["recv_counts"][dst, s] == sum(1 for r in rl[dst] if r[0] == s)
    bad = bool(((ids < 0) | (ids >= E)).any())
    assert d["status"] == (oracle.ST_EXPERT_RANGE if bad else 0)


@pytest.mark.parametrize("T,E,k", [(2, 2, 1), (2, 2, 2), (2, 4, 1), (2, 4, 2), (4, 2, 1), (4, 4, 1)])
def test_bruteforce_every_id_pattern_two_ranks(T, E, k):
    """Every assignment of expert ids (repeats included) for two ranks."""
    R, epr = 2, E // 2
    n = R * T * k
    for combo in itertools.product(range(E), repeat=n):
        ids = np.array(combo, np.int32).reshape(R, T, k)
        _check_against_naive(ids, R, T, k, epr)


def test_bruteforce_with_out_of_range_ids():
    R, T, k, epr = 2, 2, 1, 1
    for combo in itertools.product([-1, 0, 1, 2], repeat=R * T * k):
        ids = np.array(combo, np.int32).reshape(R, T, k)
        _check_against_naive(ids, R, T, k, epr)


# --------------------------------------------------------------- hand-worked example

def test_hand_worked_example():
    """Two ranks, two experts per rank (experts 0,1 on rank 0; 2,3 on rank 1), three
    tokens, top-2.  Worked out by hand from the definition (sort by expert, stable in
    token then slot; the all-to-allv concatenates source segments in source order).

    rank 0 ids: t0 (3,0)  t1 (1,2)  t2 (0,3)     rows 10, 11, 12
    rank 1 ids: t0 (2,1)  t1 (0,2)  t2 (3,1)     rows 20, 21, 22
    rank 0 send, by expert: e0: t0,t2  e1: t1  e2: t1  e3: t0,t2 -> 10 12 11 | 11 10 12
    rank 1 send, by expert: e0: t1  e1: t0,t2  e2: t0,t1  e3: t2 -> 21 20 22 | 20 21 22
    rank 0 receives 10 12 11 (from 0) then 21 20 22 (from 1)
    rank 1 receives 11 10 12 (from 0) then 20 21 22 (from 1)
    """
    x = np.array([[[10], [11], [12]], [[20], [21], [22]]], np.float32)
    ids = np.array([[[3, 0], [1, 2], [0, 3]], [[2, 1], [0, 2], [3, 1]]], np.int32)
    d = oracle.dispatch(oracle.as_rows(x), ids, 2, cap=6)
    send = d["send"].view(np.float32).reshape(2, 6)
    recv = d["recv"].view(np.float32).reshape(2, 6)
    assert send.tolist() == [[10, 12, 11, 11, 10, 12], [21, 20, 22, 20, 21, 22]]
    assert recv.tolist() == [[10, 12, 11, 21, 20, 22], [11, 10, 12, 20, 21, 22]]
    assert d["cnt"].tolist() == [[2, 1, 1, 2], [1, 2, 2, 1]]
    assert d["send_off"].tolist() == [[0, 3, 6], [0, 3, 6]]
    assert d["recv_counts"].tolist() == [[3, 3], [3, 3]]
    assert d["recv_off"].tolist() == [[0, 3, 6], [0, 3, 6]]
    assert d["pos"].tolist() == [[[4, 0], [2, 3], [1, 5]], [[3, 1], [0, 4], [5, 2]]]
    # combine with the identity expert: y = (g0 + g1) * x
    gates = np.array([[[0.25, 0.75], [0.5, 0.5], [1.0, 2.0]], [[0.125, 0.25], [1.0, 0.0], [3.0, 1.0]]],
                     np.float32)
    out = oracle.full_step(x, ids, gates, 2, oracle.F32, 0, cap=6)
    assert out["y"].reshape(2, 3).tolist() == [[10.0, 11.0, 36.0], [7.5, 21.0, 88.0]]


# ----------------------------------------------------------------- capacity overflow

def test_capacity_overflow_drops_rows_and_keeps_counts():
    rng = np.random.default_rng(21)
    R, T, k, epr = 4, 32, 2, 2
    ids = _random_ids(rng, R, T, k, R * epr)
    full = oracle.dispatch(oracle.as_rows(_tags(R, T, 3)), ids, epr, cap=R * T * k)
    cap = int(full["recv_off"][:, R].max()) - 5
    d = oracle.dispatch(oracle.as_rows(_tags(R, T, 3)), ids, epr, cap=cap)
    assert d["status"] == oracle.ST_RECV_OVERFLOW
    assert np.array_equal(d["recv_counts"], full["recv_counts"])
    assert np.array_equal(d["recv_off"], full["recv_off"])
    fr = full["recv"].view(np.int32).reshape(R, -1, 3)
    dr = d["recv"].view(np.int32).reshape(R, cap, 3)
    assert np.array_equal(dr, fr[:, :cap])
    # returned rows that were dropped come back as zeros
    ret = oracle.return_exchange(d["recv"], d["send_off"], d["recv_off"], T, k).view(np.int32).reshape(R, T * k, 3)
    sent = d["send"].view(np.int32).reshape(R, T * k, 3)
    for s in range(R):
        for dst in range(R):
            for i in range(d["recv_counts"][dst, s]):
                p = d["send_off"][s, dst] + i
                q = d["recv_off"][dst, s] + i
                if q < cap:
                    assert np.array_equal(ret[s, p], sent[s, p])
                else:
                    assert not ret[s, p].any()


# ---------------------------------------------------------------- return exchange

@pytest.mark.parametrize("R,T,k,epr", [(2, 7, 1, 1), (4, 64, 2, 2), (16, 9, 8, 16), (64, 4, 2, 1)])
def test_return_exchange_inverts_the_exchange(R, T, k, epr):
    rng = np.random.default_rng(R + T)
    ids = _random_ids(rng, R, T, k, R * epr)
    d = oracle.dispatch(oracle.as_rows(_tags(R, T, 3)), ids, epr, cap=R * T * min(k, epr))
    ret = oracle.return_exchange(d["recv"], d["send_off"], d["recv_off"], T, k)
    assert np.array_equal(ret, d["send"])


# ------------------------------------------------------------------ expert stand-in

def test_expert_scale_matches_torch_cast():
    # the product of a bf16 value (8 significant bits) and 1 + e/256 (at most 9) is exact
    # in float32, so torch's float32 multiply then round-to-nearest-even cast is the
    # exactly rounded result.
    w = W.workload("edge", tokens_per_rank=4, hidden=64)
    x, ids, gates = W.make_inputs(w)
    cap = w.capacity
    d = oracle.dispatch(oracle.as_rows(x), ids, w.experts_per_rank, cap)
    recv = d["recv"].view(np.uint16).reshape(w.num_ranks, cap, w.hidden)
    z = oracle.expert(recv, d["cnt"], d["recv_off"], w.experts_per_rank, oracle.BF16, 1)
    rl = naive.recv_lists(ids, w.num_ranks, w.tokens_per_rank, w.top_k, w.experts_per_rank)
    for dst in range(w.num_ranks):
        for q, (s, t, j, e) in enumerate(rl[dst]):
            v = torch.from_numpy(recv[dst, q].view(np.int16).copy()).view(torch.bfloat16).float()
            ref = (v * (1.0 + e / 256.0)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(z[dst, q], ref)


def test_expert_scale_f32_is_one_rounding():
    rng = np.random.default_rng(5)
    R, T, k, epr, H = 2, 5, 2, 2, 16
    x = rng.standard_normal((R, T, H)).astype(np.float32)
    ids = _random_ids(rng, R, T, k, R * epr)
    d = oracle.dispatch(oracle.as_rows(x), ids, epr, cap=R * T * k)
    recv = d["recv"].view(np.float32).reshape(R, -1, H)
    z = oracle.expert(recv, d["cnt"], d["recv_off"], epr, oracle.F32, 1)
    rl = naive.recv_lists(ids, R, T, k, epr)
    for dst in range(R):
        for q, (s, t, j, e) in enumerate(rl[dst]):
            # float32 multiply in numpy rounds the exact product once
            assert np.array_equal(z[dst, q], recv[dst, q] * np.float32(1.0 + e / 256.0))


# ------------------------------------------------------------------------- combine

@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_combine_unit_gates_reproduce_the_input(k, dtype):
    """Identity experts: gates 1 give k*x and gates 1/k give x, both exactly (k a power
    of two, so neither product nor sum rounds)."""
    rng = np.random.default_rng(k)
    R, T, epr, H = 4, 16, 4, 24
    w = W.Workload("t", R, T, H, dtype, epr, k, "uniform", "softmax", 0)
    x = W.make_x(w)
    ids = _random_ids(rng, R, T, k, R * epr)
    xf = x if dtype == oracle.F32 else (x.astype(np.uint32) << 16).view(np.float32)
    for g, factor in ((1.0, float(k)), (1.0 / k, 1.0)):
        gates = np.full((R, T, k), g, np.float32)
        y = oracle.full_step(x, ids, gates, epr, dtype, 0, cap=R * T * k)["y"]
        yf = y if dtype == oracle.F32 else (y.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(yf, xf * np.float32(factor))


def _round_fraction_to_f32(q: Fraction) -> float:
    # nearest float32 to an exact rational, ties to even, by searching neighbours
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        dist = abs(Fraction(float(c)) - q)
        key = (dist, int(np.array([c], np.float32).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return float(best[1])


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_combine_against_exact_rational_sum(dtype):
    w = W.workload("wide", num_ranks=2, tokens_per_rank=6, hidden=32, experts_per_rank=4, dtype=dtype)
    x, ids, gates = W.make_inputs(w)
    y = oracle.full_step(x, ids, gates, w.experts_per_rank, dtype, 1, cap=w.capacity)["y"]
    R, T, k, H = w.num_ranks, w.tokens_per_rank, w.top_k, w.hidden
    mism = 0
    for s in range(R):
        for t in range(T):
            for h in range(H):
                if dtype == oracle.F32:
                    v = Fraction(float(x[s, t, h]))
                else:
                    v = Fraction(oracle.bf16_to_double(int(x[s, t, h])))
                q = Fraction(0)
                for j in range(k):
                    e = int(ids[s, t, j])
                    scaled = v * (1 + Fraction(e, 256))
                    if dtype == oracle.F32:
                        f = Fraction(_round_fraction_to_f32(scaled))
                    else:
                        f = Fraction(_nearest_bf16_value(float(scaled)))   # float() exact: <= 17 bits
                    q += Fraction(float(gates[s, t, j])) * f
                if dtype == oracle.F32:
                    ref = _round_fraction_to_f32(q)
                    got = float(y[s, t, h])
                    if got != ref:
                        # a float64 sum can miss the exact rounding only by one float32 step
                        mism += 1
                        assert got in (float(np.nextafter(np.float32(ref), np.float32(-np.inf))),
                                       float(np.nextafter(np.float32(ref), np.float32(np.inf))))
                else:
                    if int(y[s, t, h]) != _nearest_bf16_bruteforce(float(q)):
                        mism += 1
    assert mism <= 1


def _nearest_bf16_value(v: float) -> float:
    b = _nearest_bf16_bruteforce(v)
    return float(np.array([b << 16], np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "wide", "edge"])
def test_staged_path_equals_layout_free_closed_form(name):
    """The staged path (sort, exchange, expert, return, combine) and the closed form that
    uses no layout at all agree bit for bit (same fp64 sums in the same slot order)."""
    small = dict(tiny={}, decode={}, prefill=dict(tokens_per_rank=256, hidden=512),
                 wide=dict(tokens_per_rank=32, hidden=256), edge={})[name]
    w = W.workload(name, **small)
    x, ids, gates = W.make_inputs(w)
    out = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, w.capacity)
    y2 = oracle.closed_form(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode)
    assert out["status"] == 0
    assert np.array_equal(out["y"], y2)


def test_closed_form_k1_is_gate_times_scaled_row():
    """k = 1: y = RNE(g * RNE(x * (1 + e/256))).  Checked with torch float64 products
    (both are exact: a bf16 value times 1 + e/256 needs at most 17 bits, a float32 gate
    times a bf16 value at most 32) and a brute-force nearest-bf16 search."""
    w = W.workload("decode", tokens_per_rank=8, hidden=40)
    x, ids, gates = W.make_inputs(w)
    y = oracle.closed_form(x, ids, gates, w.experts_per_rank, w.dtype, 1)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double()
    e = torch.from_numpy(ids[..., 0].astype(np.float64))
    z = (xt * (1.0 + e / 256.0)[..., None]).float().to(torch.bfloat16).double()   # exact product
    prod = (z * torch.from_numpy(gates[..., 0].astype(np.float64))[..., None]).numpy()
    ref = np.vectorize(_nearest_bf16_bruteforce)(prod).astype(np.uint16)
    assert np.array_equal(y, ref)


def test_dropped_slots_add_nothing():
    rng = np.random.default_rng(3)
    R, T, k, epr, H = 2, 6, 2, 2, 8
    x = rng.standard_normal((R, T, H)).astype(np.float32)
    ids = _random_ids(rng, R, T, k, R * epr)
    ids[0, 1, 0] = 99
    ids[1, 4, 1] = -3
    gates = rng.random((R, T, k)).astype(np.float32)
    out = oracle.full_step(x, ids, gates, epr, oracle.F32, 0, cap=R * T * k)
    assert out["status"] == oracle.ST_EXPERT_RANGE
    assert out["pos"][0, 1, 0] == -1 and out["pos"][1, 4, 1] == -1
    assert np.array_equal(out["y"][0, 1], (np.float64(gates[0, 1, 1]) * x[0, 1]).astype(np.float32))
    assert np.array_equal(out["y"][1, 4], (np.float64(gates[1, 4, 0]) * x[1, 4]).astype(np.float32))


# --------------------------------------------------------- expert-major receive layout

def _check_expert_major_against_naive(ids, R, T, k, epr):
    x = _tags(R, T, 3)
    cap = R * T * k
    d = oracle.dispatch(oracle.as_rows(x), ids, epr, cap, oracle.EXPERT_MAJOR)
    rl = naive.recv_lists_expert_major(ids, R, T, k, epr)
    recv = d["recv"].view(np.int32).reshape(R, cap, 3)
    for dst in range(R):
        assert d["recv_off"][dst, R] == len(rl[dst])
        for q, (s, t, j, e) in enumerate(rl[dst]):
            assert recv[dst, q, 0] == s and recv[dst, q, 1] == t
        # group starts: rows of d's local expert le begin at recv_eoff[d][le]
        for le in range(epr):
            first = next((q for q, r in enumerate(rl[dst]) if r[3] == dst * epr + le), None)
            if first is not None:
                assert d["recv_eoff"][dst, le] == first
        assert d["recv_eoff"][dst, epr] == len(rl[dst])


@pytest.mark.parametrize("T,E,k", [(2, 2, 1), (2, 2, 2), (2, 4, 1), (2, 4, 2), (4, 4, 1)])
def test_expert_major_bruteforce_every_id_pattern_two_ranks(T, E, k):
    R, epr = 2, E // 2
    for combo in itertools.product(range(E), repeat=R * T * k):
        ids = np.array(combo, np.int32).reshape(R, T, k)
        _check_expert_major_against_naive(ids, R, T, k, epr)


@pytest.mark.parametrize("R,T,k,epr,seed", [(2, 50, 2, 2, 0), (4, 64, 2, 4, 1), (16, 12, 8, 16, 3), (5, 9, 5, 3, 5)])
def test_expert_major_groups_and_tables(R, T, k, epr, seed):
    rng = np.random.default_rng(seed)
    E = R * epr
    ids = _random_ids(rng, R, T, k, E)
    cap = R * T * min(k, epr)
    sm = oracle.dispatch(oracle.as_rows(_tags(R, T, 4)), ids, epr, cap, oracle.SOURCE_MAJOR)
    em = oracle.dispatch(oracle.as_rows(_tags(R, T, 4)), ids, epr, cap, oracle.EXPERT_MAJOR)
    # the layout does not change counts, offsets of the send side, or positions
    for key in ("cnt", "send_off", "pos", "send", "recv_counts", "recv_off", "recv_eoff"):
        assert np.array_equal(sm[key], em[key]), key
    # group starts: exclusive prefix over local experts of the column sums of cnt
    col = em["cnt"].sum(axis=0).reshape(R, epr)
    assert np.array_equal(em["recv_eoff"], np.concatenate([np.zeros((R, 1), np.int64), np.cumsum(col, axis=1)], 1))
    rs = sm["recv"].view(np.int32).reshape(R, cap, 4)
    re_ = em["recv"].view(np.int32).reshape(R, cap, 4)
    for dst in range(R):
        n = em["recv_off"][dst, R]
        # the same rows, another order
        assert sorted(map(tuple, rs[dst, :n])) == sorted(map(tuple, re_[dst, :n]))
        for le in range(epr):
            lo, hi = em["recv_eoff"][dst, le], em["recv_eoff"][dst, le + 1]
            rows = re_[dst, lo:hi]
            e = dst * epr + le
            # every row of the group chose expert e; sources ascend, tokens ascend per source
            assert all(e in ids[s, t] for s, t in rows[:, :2])
            key = rows[:, 0].astype(np.int64) * T + rows[:, 1]
            assert np.all(np.diff(key) >= 0)


@pytest.mark.parametrize("R,T,k,epr", [(2, 7, 1, 1), (4, 64, 2, 2), (16, 9, 8, 16), (3, 20, 3, 4)])
def test_expert_major_return_inverts_the_exchange(R, T, k, epr):
    rng = np.random.default_rng(R * T)
    ids = _random_ids(rng, R, T, k, R * epr)
    cap = R * T * min(k, epr)
    d = oracle.dispatch(oracle.as_rows(_tags(R, T, 3)), ids, epr, cap, oracle.EXPERT_MAJOR)
    ret = oracle.return_exchange(d["recv"], d["send_off"], d["recv_off"], T, k, d["cnt"], epr, oracle.EXPERT_MAJOR)
    assert np.array_equal(ret, d["send"])


def test_expert_major_capacity_overflow_drops_the_last_rows():
    rng = np.random.default_rng(8)
    R, T, k, epr = 4, 40, 2, 3
    ids = _random_ids(rng, R, T, k, R * epr)
    full = oracle.dispatch(oracle.as_rows(_tags(R, T, 3)), ids, epr, R * T * k, oracle.EXPERT_MAJOR)
    cap = int(full["recv_off"][:, R].max()) - 4
    d = oracle.dispatch(oracle.as_rows(_tags(R, T, 3)), ids, epr, cap, oracle.EXPERT_MAJOR)
    assert d["status"] == oracle.ST_RECV_OVERFLOW
    assert np.array_equal(d["recv"].view(np.int32).reshape(R, cap, 3),
                          full["recv"].view(np.int32).reshape(R, -1, 3)[:, :cap])


@pytest.mark.parametrize("name", ["tiny", "decode", "wide", "edge"])
def test_expert_major_staged_path_equals_closed_form(name):
    small = dict(tiny={}, decode={}, wide=dict(tokens_per_rank=32, hidden=256), edge={})[name]
    w = W.workload(name, **small)
    x, ids, gates = W.make_inputs(w)
    out = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, w.capacity, oracle.EXPERT_MAJOR)
    y2 = oracle.closed_form(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode)
    assert out["status"] == 0
    assert np.array_equal(out["y"], y2)
