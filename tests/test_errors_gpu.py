"""Error paths of the C ABI.  Host-detectable problems return A2AV_ERR_INVALID and enqueue
nothing; problems only the GPU sees (expert ids out of range, a receive slice too small)
set status bits and never write out of bounds: guard rows around the receive buffer keep
their pattern.  All conditions are forced from the host; every kernel exits normally."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W
from tests.gpu_util import assert_combine_close, banner, host_bits, oracle_tables, to_device

pytestmark = pytest.mark.gpu


def _cfg(w, path=a2av.PATH_STAGED, layout=a2av.LAYOUT_SOURCE_MAJOR):
    return a2av.make_config(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k,
                            w.recv_capacity_rows, path, layout)


def test_host_side_rejections_enqueue_nothing():
    w = W.workload("tiny")
    x, ids, gates = W.make_inputs(w)
    xt, idt, gt = to_device(w, x, ids, gates)
    h = a2av.a2av_create(_cfg(w))
    L = a2av.lib()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    recv = torch.empty((w.num_ranks, w.capacity, w.hidden), dtype=torch.float32, device="cuda")
    y = torch.empty_like(xt)
    vp = ctypes.c_void_p
    P = lambda t: vp(t.data_ptr())  # noqa: E731
    null = vp(0)
    stream = vp(torch.cuda.current_stream().cuda_stream)
    # combine before any dispatch
    assert L.a2av_combine(h, P(recv), P(gt), P(y), P(st), stream) == a2av.ERR_INVALID
    # null required pointers
    assert L.a2av_dispatch(h, null, P(idt), P(recv), None, None, None, P(st), stream) == a2av.ERR_INVALID
    assert L.a2av_dispatch(h, P(xt), null, P(recv), None, None, None, P(st), stream) == a2av.ERR_INVALID
    assert L.a2av_dispatch(h, P(xt), P(idt), null, None, None, None, P(st), stream) == a2av.ERR_INVALID
    assert L.a2av_dispatch(h, P(xt), P(idt), P(recv), None, None, None, null, stream) == a2av.ERR_INVALID
    # misaligned row data (float32 rows need 4-byte alignment)
    assert L.a2av_dispatch(h, vp(xt.data_ptr() + 2), P(idt), P(recv), None, None, None, P(st),
                           stream) == a2av.ERR_INVALID
    # a status word the device atomics cannot update (not 4-byte aligned)
    st8 = torch.zeros(2, dtype=torch.int32, device="cuda")
    assert L.a2av_dispatch(h, P(xt), P(idt), P(recv), None, None, None, vp(st8.data_ptr() + 2),
                           stream) == a2av.ERR_INVALID
    # stage timing budgets outside 1 .. A2AV_TIMING_MAX_CALLS
    assert L.a2av_timing_begin(h, 0) == a2av.ERR_INVALID
    assert L.a2av_timing_begin(h, (1 << 20) + 1) == a2av.ERR_INVALID
    # bad expert stand-in mode
    a2av.a2av_dispatch(h, xt, idt, recv, None, None, None, st)
    assert L.a2av_expert_apply(h, P(recv), P(recv), 7, stream) == a2av.ERR_INVALID
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    # the expert-major group starts exist only for that layout
    with pytest.raises(a2av.A2AVError):
        a2av.a2av_copy_recv_expert_offsets(h, torch.empty((w.num_ranks, w.experts_per_rank + 1), dtype=torch.int32,
                                                          device="cuda"))
    a2av.a2av_destroy(h)
    # invalid configurations
    for field, value in (("top_k", 99), ("path", 5), ("recv_layout", 3)):
        bad = _cfg(w)
        setattr(bad, field, value)
        with pytest.raises(a2av.A2AVError):
            a2av.a2av_create(bad)


# 64 tokens per rank: one-launch dispatch (512 assignments), with 4 KB rows also with
# each row's count split over a block's wavefronts; 1100: planned (8800)
@pytest.mark.parametrize("tokens,hidden", [(64, 96), (64, 2048), (1100, 96)],
                         ids=["one-launch", "one-launch-split-count", "planned"])
@pytest.mark.parametrize("layout", [a2av.LAYOUT_SOURCE_MAJOR, a2av.LAYOUT_EXPERT_MAJOR], ids=["srcmaj", "expmaj"])
@pytest.mark.parametrize("path", [a2av.PATH_STAGED, a2av.PATH_DIRECT], ids=["staged", "direct"])
def test_receive_overflow_keeps_guard_rows_and_true_counts(path, layout, tokens, hidden):
    w = W.workload("wide", num_ranks=4, tokens_per_rank=tokens, hidden=hidden, experts_per_rank=2, top_k=2)
    x, ids, gates = W.make_inputs(w)
    full = oracle.dispatch(oracle.as_rows(x), ids, w.experts_per_rank, w.capacity)
    cap = int(full["recv_off"][:, w.num_ranks].max()) - 7
    w = W.workload("wide", num_ranks=4, tokens_per_rank=tokens, hidden=hidden, experts_per_rank=2, top_k=2,
                   recv_capacity_rows=cap)
    banner(f"overflow: cap {cap} rows per rank")
    xt, idt, gt = to_device(w, x, ids, gates)
    guard = 5
    R = w.num_ranks
    big = torch.full((R * cap + 2 * guard, w.hidden), -7.0, dtype=torch.bfloat16, device="cuda")
    recv = big[guard:guard + R * cap].view(R, cap, w.hidden)
    split = torch.empty((R, w.num_experts), dtype=torch.int32, device="cuda")
    rc = torch.empty((R, R), dtype=torch.int32, device="cuda")
    ro = torch.empty((R, R + 1), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    h = a2av.a2av_create(_cfg(w, path, layout))
    a2av.a2av_dispatch(h, xt, idt, recv, split, rc, ro, st)
    torch.cuda.synchronize()
    assert int(st.item()) == a2av.ST_RECV_OVERFLOW
    ref = oracle.dispatch(oracle.as_rows(x), ids, w.experts_per_rank, cap, layout)
    assert ref["status"] == oracle.ST_RECV_OVERFLOW
    assert np.array_equal(host_bits(rc), ref["recv_counts"])
    assert np.array_equal(host_bits(ro), ref["recv_off"])
    got = host_bits(recv)
    want = ref["recv"].view(np.uint16).reshape(R, cap, w.hidden)
    for d in range(R):
        n = min(int(ref["recv_off"][d, R]), cap)
        assert np.array_equal(got[d, :n], want[d, :n])
        assert np.all(got[d, n:] == np.uint16(0xC0E0)), "rows past the received count were written"
    g = host_bits(big)
    assert np.all(g[:guard] == np.uint16(0xC0E0)) and np.all(g[-guard:] == np.uint16(0xC0E0))
    # combine: dropped rows add nothing, as in the oracle
    y = torch.empty_like(xt)
    a2av.a2av_expert_apply(h, recv, recv, a2av.EXPERT_SCALE)
    a2av.a2av_combine(h, recv, gt, y, st)
    torch.cuda.synchronize()
    oref = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, cap, layout)
    assert_combine_close(host_bits(y), oref["y"], w.dtype, "overflow combine")
    a2av.a2av_destroy(h)


# Streaming sizes (over 256 MiB per exchange): the top-1 gather pack, the receive-order
# forward exchange and the non-temporal copies, with the hottest receiver 7 rows over.
STREAMING_OVERFLOW = [
    ("prefill", dict(tokens_per_rank=4096)),                                             # 335 MB
    ("wide", dict(num_ranks=8, tokens_per_rank=2048, hidden=2048, experts_per_rank=32, top_k=8)),   # 537 MB
]


_STREAMING_Y: dict = {}


@pytest.mark.parametrize("path", [a2av.PATH_STAGED, a2av.PATH_DIRECT], ids=["staged", "direct"])
@pytest.mark.parametrize("layout", [a2av.LAYOUT_SOURCE_MAJOR, a2av.LAYOUT_EXPERT_MAJOR], ids=["srcmaj", "expmaj"])
@pytest.mark.parametrize("name,over", STREAMING_OVERFLOW, ids=["top1", "top8"])
def test_receive_overflow_at_streaming_sizes(name, over, path, layout):
    w0 = W.workload(name, **over)
    x, ids, gates = W.make_inputs(w0)
    R = w0.num_ranks
    cap = int(oracle_tables(w0, ids)["recv_off"][:, R].max()) - 7
    w = W.workload(name, recv_capacity_rows=cap, **over)
    assert w.tokens * w.top_k * w.row_bytes >= 256 << 20
    banner(f"streaming overflow: {w.describe()} cap {cap} rows per rank")
    ref = oracle_tables(w, ids, layout)
    assert ref["status"] == oracle.ST_RECV_OVERFLOW
    xt, idt, gt = to_device(w, x, ids, gates)
    guard = 3
    big = torch.full((R * cap + 2 * guard, w.hidden), -7.0, dtype=torch.bfloat16, device="cuda")
    recv = big[guard:guard + R * cap].view(R, cap, w.hidden)
    split = torch.empty((R, w.num_experts), dtype=torch.int32, device="cuda")
    rc = torch.empty((R, R), dtype=torch.int32, device="cuda")
    ro = torch.empty((R, R + 1), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    h = a2av.a2av_create(_cfg(w, path, layout))
    a2av.a2av_dispatch(h, xt, idt, recv, split, rc, ro, st)
    torch.cuda.synchronize()
    assert int(st.item()) == a2av.ST_RECV_OVERFLOW
    assert np.array_equal(host_bits(split), ref["cnt"])
    assert np.array_equal(host_bits(rc), ref["recv_counts"])
    assert np.array_equal(host_bits(ro), ref["recv_off"])
    xf = xt.reshape(w.tokens, w.hidden)
    pattern = big[0, 0].view(torch.int16)
    for d in range(R):
        n = min(int(ref["recv_off"][d, R]), cap)
        tags = torch.from_numpy(ref["recv_tags"][d, :n].astype(np.int64)).cuda()
        assert torch.equal(recv[d, :n], xf.index_select(0, tags)), f"receive rows of rank {d}"
        assert bool((recv[d, n:].view(torch.int16) == pattern).all()), f"rows past the count of rank {d}"
    assert bool((big[:guard].view(torch.int16) == pattern).all())
    assert bool((big[-guard:].view(torch.int16) == pattern).all())
    banner("  receive rows bit-exact, nothing written past the capacity")
    y = torch.empty_like(xt)
    a2av.a2av_expert_apply(h, recv, recv, a2av.EXPERT_SCALE)
    a2av.a2av_combine(h, recv, gt, y, st)
    torch.cuda.synchronize()
    assert int(st.item()) == a2av.ST_RECV_OVERFLOW
    a2av.a2av_destroy(h)
    yb = host_bits(y)
    del big, recv, xt, idt, gt, y, xf
    torch.cuda.empty_cache()
    key = (name, layout)
    if key not in _STREAMING_Y:             # the oracle's step does not depend on the path
        _STREAMING_Y.clear()
        _STREAMING_Y[key] = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, cap,
                                             layout)["y"]
    assert_combine_close(yb, _STREAMING_Y[key], w.dtype, "streaming overflow combine")


@pytest.mark.parametrize("R,T,H", [(6, 40, 64), (1024, 3, 16)], ids=["6-ranks", "1024-ranks"])
def test_bare_alltoallv_matches_oracle_exchange(R, T, H):
    """a2av_alltoallv on pre-sorted send buffers and device counts equals the oracle's
    exchange of the same rows (ids chosen so that the sort is the identity); counts that
    are negative or exceed a sender's rows are flagged and that sender sends nothing."""
    rng = np.random.default_rng(4)
    dest = np.sort(rng.integers(0, R, size=(R, T)), axis=1).astype(np.int32)   # sorted per sender
    dest[2] = 0                                                                 # one sender, one peer
    dest[4, :] = np.sort(rng.integers(3, 5, size=T))                             # zero-length segments
    w = W.Workload("bare", R, T, H, W.BF16, 1, 1, "uniform", "softmax", 0)
    x = W.make_x(w)
    ref = oracle.dispatch(oracle.as_rows(x), dest[..., None], 1, w.capacity)
    send_counts = np.stack([np.bincount(dest[s], minlength=R) for s in range(R)]).astype(np.int32)
    xt, _, _ = to_device(w, x, dest[..., None], np.ones((R, T, 1), np.float32))
    h = a2av.a2av_create(_cfg(w))
    recv = torch.empty((R, w.capacity, H), dtype=torch.bfloat16, device="cuda")
    rc = torch.empty((R, R), dtype=torch.int32, device="cuda")
    ro = torch.empty((R, R + 1), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    sc = torch.from_numpy(send_counts).cuda()
    a2av.a2av_alltoallv(h, xt, sc, recv, rc, ro, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(host_bits(rc), ref["recv_counts"])
    assert np.array_equal(host_bits(ro), ref["recv_off"])
    got = host_bits(recv)
    want = ref["recv"].view(np.uint16).reshape(R, w.capacity, H)
    for d in range(R):
        n = int(ref["recv_off"][d, R])
        assert np.array_equal(got[d, :n], want[d, :n])
    # combine is refused after the bare collective
    y = torch.empty_like(xt)
    with pytest.raises(a2av.A2AVError):
        a2av.a2av_combine(h, recv, torch.ones((R, T, 1), device="cuda"), y, st)
    # bad counts: a negative count and a sender over its rows are flagged and sent as 0
    # (sender 5's counts would overflow a 32-bit sum)
    bad = send_counts.copy()
    bad[1, 0] = -1
    bad[3, 2] += T
    bad[5, 0] = np.iinfo(np.int32).max
    bad[5, 1] = np.iinfo(np.int32).max
    st.zero_()
    a2av.a2av_alltoallv(h, xt, torch.from_numpy(bad).cuda(), recv, rc, ro, st)
    torch.cuda.synchronize()
    assert int(st.item()) == a2av.ST_EXPERT_RANGE
    rch = host_bits(rc)
    assert np.all(rch[:, 1] == 0) and np.all(rch[:, 3] == 0) and np.all(rch[:, 5] == 0)
    kept = [s for s in range(R) if s not in (1, 3, 5)]
    assert np.array_equal(rch[:, kept], ref["recv_counts"][:, kept])
    a2av.a2av_destroy(h)


@pytest.mark.parametrize("path", [a2av.PATH_STAGED, a2av.PATH_DIRECT], ids=["staged", "direct"])
def test_zero_tokens(path):
    w = W.workload("decode", tokens_per_rank=0)
    h = a2av.a2av_create(_cfg(w, path))
    R = w.num_ranks
    split = torch.full((R, w.num_experts), 5, dtype=torch.int32, device="cuda")
    rc = torch.full((R, R), 5, dtype=torch.int32, device="cuda")
    ro = torch.full((R, R + 1), 5, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    empty = torch.empty(0, device="cuda")
    a2av.a2av_dispatch(h, empty, empty, empty, split, rc, ro, st)
    torch.cuda.synchronize()
    assert not split.any() and not rc.any() and not ro.any() and int(st.item()) == 0
    a2av.a2av_destroy(h)


@pytest.mark.parametrize("rows,row_bytes", [(0, 16), (1, 16), (37, 10240), (1000, 4096), (65, 1040)])
def test_reference_copy(rows, row_bytes):
    src = torch.randint(-2 ** 15, 2 ** 15, (rows, row_bytes // 2), dtype=torch.int16, device="cuda")
    dst = torch.zeros_like(src)
    a2av.a2av_copy_reference(src, dst, rows, row_bytes)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    L = a2av.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if rows:
        assert L.a2av_copy_reference(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr() + 8), rows,
                                     row_bytes, stream) == a2av.ERR_INVALID
    assert L.a2av_copy_reference(None, None, 1, 24, stream) == a2av.ERR_INVALID


@pytest.mark.parametrize("nbytes", [16, 16 * 1000, 3 << 20, 16 * 2_000_003])
def test_stream_reference(nbytes):
    """The measurement streams do what they claim: the write stream writes every vector's
    pattern, the read stream's words XOR to the XOR of every word it read."""
    n = nbytes // 16
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    a2av.a2av_stream_reference(None, dst, nbytes, a2av.STREAM_WRITE)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(n, 4)
    i = np.arange(n, dtype=np.uint64)
    assert np.array_equal(got[:, 0], (i & 0xFFFFFFFF).astype(np.uint32))
    assert np.array_equal(got[:, 1], (i >> np.uint64(32)).astype(np.uint32))
    assert np.all(got[:, 2] == 0x5A5A5A5A)
    assert np.array_equal(got[:, 3], (~(i & 0xFFFFFFFF)).astype(np.uint32) & np.uint32(0xFFFFFFFF))
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    out = torch.full((a2av.STREAM_READ_OUT_BYTES // 4,), 7, dtype=torch.int32, device="cuda")
    a2av.a2av_stream_reference(src, out, nbytes, a2av.STREAM_READ)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    used = out.cpu().numpy().view(np.uint32)
    # the kernel writes one word per thread of its grid (at most the whole output); words it
    # did not write keep the fill value 7, which the XOR below must leave out
    grid_words = min(4 * torch.cuda.get_device_properties(0).multi_processor_count * 256, used.size)
    assert np.bitwise_xor.reduce(used[:grid_words]) == want
    assert np.all(used[grid_words:] == 7)


def test_bare_alltoallv_reads_counts_by_reference():
    """The counts are device data read when the collective executes: counts written by
    GPU work enqueued just before the call (no host synchronisation in between) are the
    ones used, eagerly and in a replayed graph whose captured producer changes them."""
    R, T, H = 4, 32, 64
    w = W.Workload("byref", R, T, H, W.BF16, 1, 1, "uniform", "softmax", 0)
    x = W.make_x(w)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    h = a2av.a2av_create(_cfg(w))
    recv = torch.empty((R, w.capacity, H), dtype=torch.bfloat16, device="cuda")
    rc = torch.empty((R, R), dtype=torch.int32, device="cuda")
    ro = torch.empty((R, R + 1), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(2)
    tables = []
    for _ in range(6):
        dest = np.sort(rng.integers(0, R, size=(R, T)), axis=1)
        tables.append(np.stack([np.bincount(dest[s], minlength=R) for s in range(R)]).astype(np.int32))
    table_dev = torch.from_numpy(np.stack(tables)).cuda()
    counts = torch.zeros((R, R), dtype=torch.int32, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")

    def produce_and_exchange():
        # a device-side producer picks this step's counts; nothing goes through the host
        counts.copy_(table_dev.index_select(0, step).reshape(R, R))
        step.add_(1)
        a2av.a2av_alltoallv(h, xt, counts, recv, rc, ro, st)

    def expect(i):
        return oracle.dispatch(oracle.as_rows(x), _dest_ids(tables[i], T), 1, w.capacity)

    produce_and_exchange()                               # eager, step 0
    torch.cuda.synchronize()
    ref = expect(0)
    assert np.array_equal(host_bits(rc), ref["recv_counts"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        produce_and_exchange()                           # step 1 (warm-up on the side stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        produce_and_exchange()
    for i in range(2, 6):
        step.fill_(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = expect(i)
        assert np.array_equal(host_bits(rc), ref["recv_counts"]), f"replay for step {i}"
        assert np.array_equal(host_bits(ro), ref["recv_off"])
        got = host_bits(recv)
        want = ref["recv"].view(np.uint16).reshape(R, w.capacity, H)
        for d in range(R):
            n = int(ref["recv_off"][d, R])
            assert np.array_equal(got[d, :n], want[d, :n])
    assert int(st.item()) == 0
    del g
    a2av.a2av_destroy(h)


def _dest_ids(counts, T):
    """Expert ids (one expert per rank, k = 1) whose expert-sorted order is the identity
    and whose per-destination counts are `counts` [src][dst]."""
    R = counts.shape[0]
    ids = np.zeros((R, T, 1), np.int32)
    for s in range(R):
        ids[s, :, 0] = np.repeat(np.arange(R), counts[s])
    return ids


@pytest.mark.parametrize("name,over,path,expected", [
    # planned form: plan, pack, exchange / return, combine (staged); plan, pack / combine (direct)
    ("decode", dict(tokens_per_rank=600), a2av.PATH_STAGED, [1, 1, 1, 1, 1]),
    ("decode", dict(tokens_per_rank=600), a2av.PATH_DIRECT, [1, 1, 0, 0, 1]),
    # one-launch form: its single launch counts as pack
    ("decode", {}, a2av.PATH_STAGED, [0, 1, 1, 1, 1]),
    ("decode", {}, a2av.PATH_DIRECT, [0, 1, 0, 0, 1]),
], ids=["planned-staged", "planned-direct", "one-launch-staged", "one-launch-direct"])
def test_stage_timing_counts_each_launch_once(name, over, path, expected):
    """Stage timing records one event pair per library launch while its budget lasts:
    per step the launches named in include/a2av.h, times non-negative, nothing recorded
    once the budget is spent."""
    w = W.workload(name, **over)
    x, ids, gates = W.make_inputs(w)
    xt, idt, gt = to_device(w, x, ids, gates)
    s = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k, path=path)
    y = torch.empty_like(xt)
    steps = 3
    a2av.a2av_timing_begin(s.handle, steps)
    for _ in range(steps + 2):          # two steps past the budget
        s.dispatch(xt, idt)
        s.combine(s.recv, gt, y)
    ms, launches = a2av.a2av_timing_end(s.handle)
    assert int(s.status.item()) == 0
    per_step = sum(expected)
    budget = steps * a2av.STAGES
    # the budget holds steps * 5 launches; a step makes per_step of them
    want = [0] * a2av.STAGES
    done = 0
    for _ in range(steps + 2):
        for i, c in enumerate(expected):
            if c and done < budget:
                want[i] += 1
                done += 1
    assert launches == want, (launches, want)
    assert all(m >= 0.0 for m in ms) and all((m > 0.0) == (n > 0) for m, n in zip(ms, launches))
    # a second window starts from zero
    a2av.a2av_timing_begin(s.handle, 1)
    s.dispatch(xt, idt)
    ms2, launches2 = a2av.a2av_timing_end(s.handle)
    assert launches2 == [1 if (c and i < 3) else 0 for i, c in enumerate(expected)]
    s.close()
