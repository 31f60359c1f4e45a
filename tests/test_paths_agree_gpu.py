"""The four path/layout pairs against one another, and a step against its own repeat.

The staged and zero-copy paths are two schedules of one computation, and no atomic
operation decides a place or the order of a sum: every table and position is the same
on all four (path, layout) pairs, the receive rows are the same for the two paths of one
layout, and the combine output is bit-identical for the two paths of one layout (each
token's k products are summed in slot order, whichever path carried the rows; a slot
dropped past the capacity adds a zero row on the staged path and nothing on the
zero-copy path, which leaves the float32 sum unchanged either way).  When every row
fits, the combine is bit-identical across the layouts too; past the capacity it is
not, since each layout drops the rows at the end of its own order (source-major: the
last senders' rows, expert-major: the last local experts' rows).  A repeated step on
the same handle reproduces the first bit for bit.  These compare the HIP path with
itself, on both sides of the one-launch limit; the comparisons with the oracle are in
test_parity_gpu.py.
"""
import numpy as np
import pytest
import torch

from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W
from tests.gpu_util import Run, banner, to_device

pytestmark = pytest.mark.gpu

PAIRS = [(a2av.PATH_STAGED, a2av.LAYOUT_SOURCE_MAJOR), (a2av.PATH_DIRECT, a2av.LAYOUT_SOURCE_MAJOR),
         (a2av.PATH_STAGED, a2av.LAYOUT_EXPERT_MAJOR), (a2av.PATH_DIRECT, a2av.LAYOUT_EXPERT_MAJOR)]

CASES = [
    ("decode", {}),                                                  # one launch, top-1
    ("decode", dict(tokens_per_rank=600)),                           # planned, top-1
    ("edge", {}),                                                    # one launch, 64 ranks, top-2
    ("wide", dict(tokens_per_rank=16)),                              # one launch, top-8
    ("wide", dict(tokens_per_rank=200, hidden=512)),                 # planned, top-8
    ("prefill", dict(tokens_per_rank=300, hidden=512)),              # planned, Zipf(1.2)
    ("tiny", {}),                                                    # float32 rows
    # receive capacity below the hottest rank's rows, and invalid ids
    ("wide", dict(num_ranks=4, tokens_per_rank=30, hidden=64, experts_per_rank=2, top_k=2,
                  recv_capacity_rows=20)),
    ("wide", dict(num_ranks=4, tokens_per_rank=1100, hidden=64, experts_per_rank=4, top_k=2,
                  recv_capacity_rows=1500)),
]

TABLES = ("split", "send_off", "recv_counts", "recv_off", "pos")


def _step(run: Run) -> dict:
    run.all()
    out = {name: getattr(run, name) for name in TABLES}
    out["recv"], out["z"], out["y"], out["status"] = run.recv, run.z, run.y, run.status
    if run.recv_eoff is not None:
        out["recv_eoff"] = run.recv_eoff
    return out


def _same(a: dict, b: dict, keys, what: str):
    for key in keys:
        if key in ("recv", "z"):
            assert len(a[key]) == len(b[key]), f"{what}: {key} ranks"
            for d, (ra, rb) in enumerate(zip(a[key], b[key])):
                assert np.array_equal(ra, rb), f"{what}: {key} rows of rank {d}"
        elif key == "status":
            assert a[key] == b[key], f"{what}: status {a[key]} against {b[key]}"
        else:
            assert np.array_equal(a[key], b[key]), f"{what}: {key}"


@pytest.mark.parametrize("name,over", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_paths_and_layouts_agree_and_repeat_bitwise(name, over):
    w = W.workload(name, **over)
    x, ids, gates = W.make_inputs(w)
    if over.get("recv_capacity_rows"):
        ids = ids.copy()
        ids[0, 1, 0] = -3                  # dropped and flagged
        ids[w.num_ranks - 1, w.tokens_per_rank - 1, w.top_k - 1] = w.num_experts
    device_inputs = to_device(w, x, ids, gates)
    results = {}
    for path, layout in PAIRS:
        banner(f"paths agree: {w.describe()} cap={w.capacity} path={path} layout={layout}")
        first = Run(w, x, ids, gates, path=path, layout=layout, device_inputs=device_inputs)
        a = _step(first)
        b = _step(Run(w, x, ids, gates, session=first.session, device_inputs=device_inputs))
        _same(a, b, TABLES + ("recv", "z", "y", "status"), f"repeat of path {path} layout {layout}")
        first.session.close()
        results[(path, layout)] = a
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    base = results[PAIRS[0]]
    overflow = bool(over.get("recv_capacity_rows"))
    flagged = a2av.ST_EXPERT_RANGE | a2av.ST_RECV_OVERFLOW
    assert base["status"] == (flagged if overflow else 0), base["status"]
    for pair in PAIRS[1:]:
        keys = TABLES + ("status",) + (() if overflow else ("y",))
        _same(base, results[pair], keys, f"pair {pair} against {PAIRS[0]}")
    for layout in (a2av.LAYOUT_SOURCE_MAJOR, a2av.LAYOUT_EXPERT_MAJOR):
        staged, direct = results[(a2av.PATH_STAGED, layout)], results[(a2av.PATH_DIRECT, layout)]
        keys = ("recv", "z", "y") + (("recv_eoff",) if layout == a2av.LAYOUT_EXPERT_MAJOR else ())
        _same(staged, direct, keys, f"layout {layout}, staged against zero-copy")
    if overflow:
        ys = results[(a2av.PATH_STAGED, a2av.LAYOUT_SOURCE_MAJOR)]["y"]
        ye = results[(a2av.PATH_STAGED, a2av.LAYOUT_EXPERT_MAJOR)]["y"]
        assert not np.array_equal(ys, ye), "the layouts should drop different rows past the capacity"
