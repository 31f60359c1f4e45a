"""The allocation-free bare collective (a2av_alltoallv_noalloc) against the handle-based
one (a2av_alltoallv), through the C ABI: identical receive rows, counts, offsets and
status on consecutive calls that share the library's one scratch array, the second
call smaller than the first, and at a streaming size; the largest rank count it
accepts; shapes past its limit rejected on the host."""
import numpy as np
import pytest
import torch

import oracle
from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W
from tests.gpu_util import banner, host_bits

pytestmark = pytest.mark.gpu


def _inputs(R, T, H, seed, cap=0):
    """Sorted per-sender destinations, their counts, and bf16 token rows (receive capacity
    cap rows per rank, 0: the worst case)."""
    rng = np.random.default_rng(seed)
    dest = np.sort(rng.integers(0, R, size=(R, T)), axis=1).astype(np.int32)
    if R > 2:
        dest[1] = 0                                   # one sender, one peer
        dest[2, :] = np.sort(rng.integers(0, 2, size=T))   # zero-length segments to the rest
    counts = np.stack([np.bincount(dest[s], minlength=R) for s in range(R)]).astype(np.int32)
    w = W.Workload("noalloc", R, T, H, W.BF16, 1, 1, "uniform", "softmax", 0, seed=seed, recv_capacity_rows=cap)
    return w, dest, counts, W.make_x(w)


def _buffers(R, cap, H, fill):
    recv = torch.full((R, cap, H), fill, dtype=torch.bfloat16, device="cuda")
    rc = torch.full((R, R), -7, dtype=torch.int32, device="cuda")
    ro = torch.full((R, R + 1), -7, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    return recv, rc, ro, st


def _both(w, counts, x, bad_counts=None):
    """Runs the handle-based and the no-alloc collective on the same inputs; returns the
    host copies of (recv, recv_counts, recv_offsets, status) of each."""
    R, T, H, cap = w.num_ranks, w.tokens_per_rank, w.hidden, w.capacity
    cfg = a2av.make_config(R, T, H, W.BF16, 1, 1, w.recv_capacity_rows)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    sc = torch.from_numpy(counts if bad_counts is None else bad_counts).cuda()
    outs = []
    h = a2av.a2av_create(cfg)
    b = _buffers(R, cap, H, 3.0)
    a2av.a2av_alltoallv(h, xt, sc, *b)
    torch.cuda.synchronize()
    outs.append([host_bits(t) for t in b])
    a2av.a2av_destroy(h)
    b = _buffers(R, cap, H, 3.0)
    a2av.a2av_alltoallv_noalloc(cfg, xt, sc, *b)
    torch.cuda.synchronize()
    outs.append([host_bits(t) for t in b])
    return outs


@pytest.mark.parametrize("shapes", [((8, 96, 640), (5, 40, 128)), ((256, 3, 64), (2, 7, 8))],
                         ids=["8-then-5-ranks", "256-then-2-ranks"])
def test_noalloc_matches_handle_collective_on_consecutive_calls(shapes):
    for i, (R, T, H) in enumerate(shapes):
        banner(f"no-alloc call {i}: R={R} T={T} H={H}")
        w, dest, counts, x = _inputs(R, T, H, seed=11 + i)
        ref_handle, got = _both(w, counts, x)
        for a, b, name in zip(ref_handle, got, ("recv", "recv_counts", "recv_offsets", "status")):
            assert np.array_equal(a, b), f"call {i}: {name} differs from a2av_alltoallv"
        assert int(got[3][0]) == 0
        # and both equal the oracle's exchange of the same rows
        ref = oracle.dispatch(oracle.as_rows(x), dest[..., None], 1, w.capacity)
        assert np.array_equal(got[1], ref["recv_counts"])
        assert np.array_equal(got[2], ref["recv_off"])
        want = ref["recv"].view(np.uint16).reshape(R, w.capacity, H)
        for d in range(R):
            n = int(ref["recv_off"][d, R])
            assert np.array_equal(got[0][d, :n], want[d, :n]), f"call {i}: receive rows of rank {d}"


def test_noalloc_matches_handle_collective_at_streaming_size():
    """335 MB of send rows (4 ranks x 8192 rows of 10 KiB): the collective's non-temporal,
    two-blocks-per-CU copy form, from the scratch tables as from the handle's."""
    R, T, H = 4, 8192, 5120
    banner(f"no-alloc streaming call: R={R} T={T} H={H}")
    w, dest, counts, x = _inputs(R, T, H, seed=21, cap=3 * T)
    ref_handle, got = _both(w, counts, x)
    for a, b, name in zip(ref_handle, got, ("recv", "recv_counts", "recv_offsets", "status")):
        assert np.array_equal(a, b), f"{name} differs from a2av_alltoallv"
    assert int(got[3][0]) == 0
    ref = oracle.dispatch(oracle.as_rows(x), dest[..., None], 1, w.capacity)
    assert np.array_equal(got[1], ref["recv_counts"])
    assert np.array_equal(got[2], ref["recv_off"])
    want = ref["recv"].view(np.uint16).reshape(R, w.capacity, H)
    for d in range(R):
        n = int(ref["recv_off"][d, R])
        assert np.array_equal(got[0][d, :n], want[d, :n]), f"receive rows of rank {d}"


def test_noalloc_flags_bad_counts_like_the_handle_collective():
    w, dest, counts, x = _inputs(6, 40, 64, seed=5)
    bad = counts.copy()
    bad[1, 0] = -1                                     # negative
    bad[3, 2] += w.tokens_per_rank                     # more rows than the sender holds
    ref_handle, got = _both(w, counts, x, bad_counts=bad)
    for a, b, name in zip(ref_handle, got, ("recv", "recv_counts", "recv_offsets", "status")):
        assert np.array_equal(a, b), f"{name} differs from a2av_alltoallv"
    assert int(got[3][0]) == a2av.ST_EXPERT_RANGE


def test_noalloc_rejects_shapes_past_its_scratch_on_the_host():
    R = a2av.NOALLOC_MAX_RANKS + 1
    cfg = a2av.make_config(R, 2, 8, W.BF16, 1, 1)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    counts = torch.zeros((R, R), dtype=torch.int32, device="cuda")
    x = torch.zeros((R, 2, 8), dtype=torch.bfloat16, device="cuda")
    recv = torch.zeros((R, 2 * R, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(a2av.A2AVError) as e:
        a2av.a2av_alltoallv_noalloc(cfg, x, counts, recv, None, None, st)
    assert e.value.code == a2av.ERR_SCRATCH
    with pytest.raises(a2av.A2AVError) as e:
        a2av.a2av_alltoallv_noalloc(cfg, x, None, recv, None, None, st)
    assert e.value.code == a2av.ERR_INVALID
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_noalloc_replays_in_a_captured_graph_with_changing_counts():
    """The point of the allocation-free form: captured in a graph (after its first call on
    the device, which looks up its scratch address), it replays with counts a captured
    device-side producer changes every replay, each replay equal to the handle-based
    collective run eagerly on the same counts."""
    R, T, H = 6, 48, 64
    w = W.Workload("noalloc-graph", R, T, H, W.BF16, 1, 1, "uniform", "softmax", 0, seed=3)
    x = W.make_x(w)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    cfg = a2av.make_config(R, T, H, W.BF16, 1, 1)
    rng = np.random.default_rng(8)
    tables = []
    for _ in range(6):
        dest = np.sort(rng.integers(0, R, size=(R, T)), axis=1)
        tables.append(np.stack([np.bincount(dest[s], minlength=R) for s in range(R)]).astype(np.int32))
    table_dev = torch.from_numpy(np.stack(tables)).cuda()
    counts = torch.zeros((R, R), dtype=torch.int32, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    recv, rc, ro, st = _buffers(R, w.capacity, H, 0.0)

    def produce_and_exchange():
        counts.copy_(table_dev.index_select(0, step).reshape(R, R))
        a2av.a2av_alltoallv_noalloc(cfg, xt, counts, recv, rc, ro, st)

    produce_and_exchange()                               # eager first call on this device
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        produce_and_exchange()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        produce_and_exchange()
    h = a2av.a2av_create(cfg)
    for i in (3, 1, 5, 0, 4):
        banner(f"no-alloc graph replay with counts table {i}")
        step.fill_(i)
        recv.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host_bits(t) for t in (recv, rc, ro)]
        b = _buffers(R, w.capacity, H, 0.0)
        a2av.a2av_alltoallv(h, xt, torch.from_numpy(tables[i]).cuda(), *b)
        torch.cuda.synchronize()
        want = [host_bits(t) for t in b[:3]]
        for a_, b_, name in zip(got, want, ("recv", "recv_counts", "recv_offsets")):
            assert np.array_equal(a_, b_), f"replay {i}: {name} differs from a2av_alltoallv"
    assert int(st.item()) == 0
    del g
    a2av.a2av_destroy(h)
