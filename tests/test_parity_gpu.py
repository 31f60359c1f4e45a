"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small and ragged cases: every output element by element against the oracle's staged path
(tables, positions, receive rows and expert rows bit-exact; the combine within the
tolerance in tests/gpu_util.py).  The five workloads at their full sizes, in the launch
configuration bench.py times: every table, every position and every receive row
bit-exact (the oracle routes 4-byte tags, row content not entering the routing, and each
GPU receive row must equal the input row its tag names), and the combine of every token
against the oracle's closed form (evaluated over disjoint token ranges by host threads,
each running the single-threaded C oracle on its range), plus a float32 torch
evaluation of the same definition on every token as an extra check.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W
from tests.gpu_util import (Run, assert_combine_close, assert_tables_equal, banner, host_bits,
                            oracle_tables, to_device)

pytestmark = pytest.mark.gpu


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


PATHS = [a2av.PATH_STAGED, a2av.PATH_DIRECT]
PATH_IDS = ["staged", "direct"]
LAYOUTS = [a2av.LAYOUT_SOURCE_MAJOR, a2av.LAYOUT_EXPERT_MAJOR]
LAYOUT_IDS = ["srcmaj", "expmaj"]


def _full_oracle_check(w: W.Workload, x, ids, gates, path=a2av.PATH_STAGED, layout=a2av.LAYOUT_SOURCE_MAJOR):
    banner(f"full check {w.describe()} cap={w.capacity} path={PATH_IDS[path]} layout={LAYOUT_IDS[layout]}")
    ref = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, w.capacity, layout)
    run = Run(w, x, ids, gates, path=path, layout=layout).all()
    R = w.num_ranks
    assert_tables_equal(run, ref, R)
    assert run.status == ref["status"], (run.status, ref["status"])
    for d in range(R):
        n = run.valid[d]
        assert np.array_equal(run.recv[d], ref["recv"][d, :n]), f"recv rows of rank {d}"
        assert np.array_equal(run.z[d], ref["z"][d, :n]), f"expert rows of rank {d}"
    exact = assert_combine_close(run.y, ref["y"], w.dtype, w.describe())
    banner(f"  combine bit-identical fraction {exact:.6f}")
    session = run.session
    del run
    session.close()
    _free()
    return ref


# -------------------------------------------------------------- small / ragged cases

SMALL = [
    ("tiny", {}),
    ("decode", {}),
    ("edge", {}),
    ("prefill", dict(tokens_per_rank=300, hidden=512)),
    ("wide", dict(tokens_per_rank=40, hidden=256)),
    # one rank talking to itself, row not a multiple of 64 vectors
    ("wide", dict(num_ranks=1, tokens_per_rank=37, hidden=1000, experts_per_rank=8, top_k=3)),
    # rows of 198 bytes: 2-byte vectors
    ("wide", dict(num_ranks=5, tokens_per_rank=13, hidden=99, experts_per_rank=3, top_k=3)),
    # rows of 200 bytes: 8-byte vectors
    ("wide", dict(num_ranks=3, tokens_per_rank=29, hidden=100, experts_per_rank=4, top_k=2)),
    # float32 rows of 132 bytes: 4-byte vectors, scaled experts
    ("tiny", dict(num_ranks=6, tokens_per_rank=21, hidden=33, experts_per_rank=2, top_k=4,
                  expert_mode=W.EXPERT_SCALE)),
    # every expert chosen by every token (k = E)
    ("tiny", dict(num_ranks=2, tokens_per_rank=9, hidden=64, experts_per_rank=2, top_k=4)),
    # no tokens at all
    ("decode", dict(tokens_per_rank=0)),
    # many ranks, one expert each
    ("edge", dict(num_ranks=64, tokens_per_rank=3, hidden=64)),
    # largest expert count held in LDS (4096 experts, two wavefronts per planning block)
    ("wide", dict(num_ranks=8, tokens_per_rank=64, hidden=64, experts_per_rank=512, top_k=4)),
    # largest top-k
    ("wide", dict(num_ranks=4, tokens_per_rank=5, hidden=64, experts_per_rank=32, top_k=64)),
    # largest rank count
    ("edge", dict(num_ranks=1024, tokens_per_rank=2, hidden=16, routing="uniform")),
    # long runs per wavefront: 8192 assignments per rank spread over 16 wavefronts
    ("decode", dict(num_ranks=2, tokens_per_rank=8192, hidden=8)),
    # one-launch dispatch: slots placed in groups of 4, 2 and 1 (k = 7); with 4 KB rows
    # cut into 4 pieces, each row's count split over the block's four wavefronts
    ("wide", dict(num_ranks=16, tokens_per_rank=8, hidden=64, experts_per_rank=4, top_k=7)),
    ("wide", dict(num_ranks=4, tokens_per_rank=16, hidden=2048, experts_per_rank=4, top_k=7)),
    # one-launch dispatch at its limits, and just past each of them: 4096 assignments
    # with rows of 8 KiB or more (planning blocks ranking 512 ids each in batches), 1024
    # per rank, 2048 with shorter rows on the zero-copy path (4096 on the staged path)
    ("decode", dict(num_ranks=8, tokens_per_rank=512, hidden=4096)),
    ("decode", dict(num_ranks=8, tokens_per_rank=513, hidden=4096)),
    ("decode", dict(num_ranks=4, tokens_per_rank=1024, hidden=4096)),
    ("decode", dict(num_ranks=2, tokens_per_rank=1025, hidden=4096)),
    ("wide", dict(num_ranks=8, tokens_per_rank=256, hidden=4096, experts_per_rank=4, top_k=2)),
    ("wide", dict(num_ranks=8, tokens_per_rank=257, hidden=4096, experts_per_rank=4, top_k=2)),
    ("decode", dict(num_ranks=8, tokens_per_rank=512, hidden=256)),
    ("wide", dict(num_ranks=8, tokens_per_rank=128, hidden=64, experts_per_rank=4, top_k=2)),
    ("wide", dict(num_ranks=8, tokens_per_rank=129, hidden=64, experts_per_rank=4, top_k=2)),
    ("wide", dict(num_ranks=8, tokens_per_rank=256, hidden=64, experts_per_rank=4, top_k=2)),
    ("wide", dict(num_ranks=8, tokens_per_rank=257, hidden=64, experts_per_rank=4, top_k=2)),
    # a small receive capacity (rows dropped, flagged, counts kept)
    ("wide", dict(num_ranks=4, tokens_per_rank=30, hidden=64, experts_per_rank=2, top_k=2,
                  recv_capacity_rows=20)),
    # the same at top-1: the one-launch dispatch, then the planned gather-form pack
    ("decode", dict(num_ranks=4, tokens_per_rank=30, hidden=64, recv_capacity_rows=20)),
    ("decode", dict(num_ranks=4, tokens_per_rank=1100, hidden=64, recv_capacity_rows=800)),
    # more assignments per wavefront than its registers hold: planning in several batches
    ("wide", dict(num_ranks=2, tokens_per_rank=9000, hidden=16, experts_per_rank=8, top_k=2)),
    ("wide", dict(num_ranks=8, tokens_per_rank=2000, hidden=16, experts_per_rank=512, top_k=4)),
    # ranks planned in 16 chunks of one wavefront each (4096 experts), each wavefront's run
    # longer than one batch; and a ragged last chunk
    ("wide", dict(num_ranks=2, tokens_per_rank=12000, hidden=8, experts_per_rank=2048, top_k=2)),
    ("decode", dict(num_ranks=3, tokens_per_rank=5001, hidden=8)),
]


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_small_and_ragged_cases_match_oracle(name, over, path, layout):
    w = W.workload(name, **over)
    x, ids, gates = W.make_inputs(w)
    ref = _full_oracle_check(w, x, ids, gates, path, layout)
    if over.get("recv_capacity_rows"):
        assert ref["status"] & oracle.ST_RECV_OVERFLOW


def _random_case(i):
    rng = np.random.default_rng(1000 + i)
    R = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 31, 64]))
    epr = int(rng.choice([1, 2, 3, 7, 16]))
    E = R * epr
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([0, 1, 7, 33, 100, 257]))
    dtype = int(rng.choice([W.F32, W.BF16]))
    H = int(rng.choice([1, 3, 8, 64, 99, 100, 640, 1000]))
    routing = "zipf" if (k == 1 and rng.random() < 0.5) else "uniform"
    return W.Workload(f"random{i}", R, T, H, dtype, epr, k, routing, str(rng.choice(["softmax", "sigmoid"])),
                      int(rng.integers(0, 2)), zipf_s=1.2, seed=i)


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("i", range(12))
def test_seeded_random_shapes_match_oracle(i, path, layout):
    w = _random_case(i)
    x, ids, gates = W.make_inputs(w)
    _full_oracle_check(w, x, ids, gates, path, layout)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_repeated_ids_within_a_token_are_sent_k_times(path):
    w = W.workload("tiny", num_ranks=3, tokens_per_rank=50, hidden=32, experts_per_rank=2, top_k=3)
    x, _, gates = W.make_inputs(w)
    ids = np.random.default_rng(9).integers(0, w.num_experts, size=(3, 50, 3)).astype(np.int32)
    _full_oracle_check(w, x, ids, gates, path)


# Small steps (at most 1024 assignments per rank, and at most 2048 in all, 4096 on the
# staged path or at top-1) dispatch in one launch that places rows by counting over the
# ids; larger ones plan first.  Cases that probe error handling run on both sides of that
# line.


@pytest.mark.parametrize("tokens", [128, 600], ids=["one-launch", "planned"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_every_token_routed_to_the_same_two_experts(path, layout, tokens):
    # the most skewed step: one rank receives everything, every other split is empty,
    # and all assignments hit the same two (expert, sender) counters
    w = W.workload("tiny", num_ranks=4, tokens_per_rank=tokens, hidden=512, dtype=W.BF16, experts_per_rank=2,
                   top_k=2, expert_mode=W.EXPERT_SCALE)
    x, _, gates = W.make_inputs(w)
    ids = np.empty((4, tokens, 2), dtype=np.int32)
    ids[..., 0], ids[..., 1] = 5, 4
    ref = _full_oracle_check(w, x, ids, gates, path, layout)
    assert int(ref["recv_off"][2, 4]) == 4 * tokens * 2


@pytest.mark.parametrize("tokens,hidden", [(24, 128), (16, 2048), (1100, 128), (3000, 64)],
                         ids=["one-launch", "one-launch-split-count", "planned", "planned-in-chunks"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_out_of_range_ids_are_dropped_and_flagged(path, tokens, hidden):
    w = W.workload("wide", num_ranks=4, tokens_per_rank=tokens, hidden=hidden, experts_per_rank=4, top_k=2)
    x, ids, gates = W.make_inputs(w)
    ids = ids.copy()
    ids[0, 3, 1] = w.num_experts
    ids[2, 0, 0] = -1
    ids[3, tokens - 1, 1] = 1 << 30
    # ids whose low 16 bits (or the value shifted left by 16) equal a valid expert's, and
    # the int32 extremes: they must be dropped like any other, never taken for that expert
    ids[1, 2, 0] = (1 << 16) + 3
    ids[1, 5, 1] = -(1 << 16)
    ids[0, 7, 0] = np.iinfo(np.int32).min
    ids[2, 4, 1] = np.iinfo(np.int32).max
    if tokens > 1000:
        ids[1, tokens // 2, 0] = -5          # in a middle chunk of a rank planned in chunks
    ref = _full_oracle_check(w, x, ids, gates, path)
    assert ref["status"] == oracle.ST_EXPERT_RANGE


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_decode_steps_with_fresh_routing(path):
    w = W.workload("decode")
    x = W.make_x(w)
    session = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k,
                           path=path)
    for step in range(3):
        ids, gates = W.make_ids(w, step), W.make_gates(w, step)
        run = Run(w, x, ids, gates, session=session).all()
        ref = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, w.capacity)
        assert_tables_equal(run, ref, w.num_ranks)
        assert_combine_close(run.y, ref["y"], w.dtype, f"decode step {step}")
    session.close()
    _free()


# ------------------------------------------------------------ full-size workloads

def _torch_definition_f32(w: W.Workload, x_dev, ids_dev, gates_dev, chunk=4096):
    """y = sum_j g_j * round(x * (1 + e_j/256)) evaluated by torch in float32 (a property
    check at full size: same definition, float32 accumulation in slot order)."""
    N, k = w.tokens, w.top_k
    xf = x_dev.reshape(N, w.hidden)
    idsf = ids_dev.reshape(N, k)
    gf = gates_dev.reshape(N, k)
    out = torch.empty_like(xf)
    for a in range(0, N, chunk):
        b = min(N, a + chunk)
        acc = torch.zeros((b - a, w.hidden), dtype=torch.float32, device=xf.device)
        for j in range(k):
            e = idsf[a:b, j].to(torch.float32)
            z = xf[a:b].float()
            if w.expert_mode == W.EXPERT_SCALE:
                z = (z * (1.0 + e / 256.0)[:, None]).to(xf.dtype).float()
            acc = torch.addcmul(acc, gf[a:b, j:j + 1], z)
        out[a:b] = acc.to(xf.dtype)
    return out.reshape(x_dev.shape)


def _host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_closed_form_all(w: W.Workload, x, ids, gates, chunk=1024):
    """The oracle's closed form for every token, [R*T][H]: disjoint token ranges, each
    computed by one call of the single-threaded C oracle, run side by side on host
    threads (the foreign calls release the interpreter lock)."""
    N = w.tokens
    y = np.empty((N, w.hidden), dtype=x.dtype)

    def job(a):
        b = min(N, a + chunk)
        y[a:b] = oracle.closed_form(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, a, b).reshape(
            b - a, w.hidden)

    with ThreadPoolExecutor(_host_threads()) as pool:
        list(pool.map(job, range(0, N, chunk)))
    return y


def assert_combine_close_chunked(y_gpu, y_ref, dtype, what, chunk=4096):
    """assert_combine_close over token chunks (bounded host memory at full size): the
    element-wise bound on every element and the norm-wise bound on every chunk, which
    implies it over all tokens.  Returns the bit-identical fraction."""
    y_gpu = y_gpu.reshape(y_ref.shape)
    exact = 0.0
    for a in range(0, y_ref.shape[0], chunk):
        exact += assert_combine_close(y_gpu[a:a + chunk], y_ref[a:a + chunk], dtype, f"{what} tokens {a}+") \
            * y_ref[a:a + chunk].size
    return exact / max(1, y_ref.size)


@pytest.mark.parametrize("name", ["decode", "prefill", "wide", "edge", "tiny"])
def test_full_size_workload(name):
    _check_at_size(W.workload(name))


def test_streaming_sizes_with_two_byte_vectors():
    # rows of 4094 bytes (2-byte vectors, 32 per lane) at sizes where every row kernel
    # streams (655 MB per exchange): the non-temporal copies, the receive-order exchange
    # and the top-k pack through the caches, with the narrowest vector type
    w = W.workload("wide", num_ranks=4, tokens_per_rank=20000, hidden=2047, experts_per_rank=4, top_k=2)
    assert w.assignments * w.row_bytes >= 256 << 20 and w.row_bytes % 4 == 2
    _check_at_size(w)


@pytest.mark.parametrize("name,over", [
    # top-1: the gather-form pack and the single-slot combine on rows of four-float vectors
    ("prefill", dict(tokens_per_rank=4096, hidden=2560, dtype=W.F32)),
    # top-2: the top-k pack through the caches and the paired-slot combine
    ("wide", dict(num_ranks=8, tokens_per_rank=2048, hidden=2048, dtype=W.F32, experts_per_rank=16, top_k=2)),
], ids=["top1", "top2"])
def test_streaming_sizes_in_float32(name, over):
    # float32 rows at sizes where every row kernel streams (the workloads that reach those
    # sizes are bf16)
    w = W.workload(name, **over)
    assert w.assignments * w.row_bytes >= 256 << 20
    _check_at_size(w)


def _check_at_size(w: W.Workload):
    name = w.name
    banner(f"full size {w.describe()} cap={w.capacity}")
    x, ids, gates = W.make_inputs(w)
    refs = {lay: oracle_tables(w, ids, lay) for lay in LAYOUTS}
    banner(f"  oracle closed form on all {w.tokens} tokens ({_host_threads()} host threads)")
    yref = oracle_closed_form_all(w, x, ids, gates)
    dev = to_device(w, x, ids, gates)
    yt = None
    for path, pname, layout in [(p, n, lay) for p, n in zip(PATHS, PATH_IDS) for lay in LAYOUTS]:
        banner(f"  path {pname} layout {LAYOUT_IDS[layout]}")
        ref = refs[layout]
        run = Run(w, x, ids, gates, path=path, layout=layout, device_inputs=dev).dispatch(keep_recv=False)
        assert_tables_equal(run, ref, w.num_ranks)
        assert run.session.status.item() == 0

        # every receive row equals the input row its oracle tag names
        s = run.session
        xf = run.x_dev.reshape(w.tokens, w.hidden)
        for d in range(w.num_ranks):
            n = run.valid[d]
            if n == 0:
                continue
            tags = torch.from_numpy(ref["recv_tags"][d, :n].astype(np.int64)).cuda()
            assert torch.equal(s.recv[d, :n], xf.index_select(0, tags)), f"receive rows of rank {d}"
        banner("    receive rows bit-exact")
        run.expert(keep_z=False).combine()
        assert run.status == 0

        # combine of every token against the oracle's closed form
        exact = assert_combine_close_chunked(run.y.reshape(w.tokens, w.hidden), yref, w.dtype, f"{name} {pname}")
        banner(f"    combine matches the oracle on {w.tokens} / {w.tokens} tokens "
               f"(bit-identical fraction {exact:.6f})")

        # every token: the same definition in float32 torch arithmetic
        if yt is None:
            yt = host_bits(_torch_definition_f32(w, run.x_dev, run.ids_dev, run.gates_dev))
        assert_combine_close(run.y, yt, w.dtype, f"{name} {pname} torch float32 definition")
        s.close()
        del run, s
        _free()
