"""The debug build on the GPU.

liba2av_debug.so is the library's source compiled with A2AV_DEBUG=1: every row index and
every table value a kernel of the path turns into an address is checked on the device
before the access, and a failed check sets status bit ST_BOUNDS and skips the access
instead of touching memory.  Here it runs the cases that reach every kernel form: the
one-launch dispatch (planning, table and row blocks, rows whose count a block's four
wavefronts split), the planned pack in scatter form (top-k) and gather form (top-1 at
streaming sizes), the forward exchange in send order and in receive order, the return,
the combine on both paths and both layouts, receive-capacity overflow with guard rows,
out-of-range ids, and the bare collective.  Each case is checked against the oracle as
the release tests check it, status included, so a check that fired where nothing was out
of range fails its case.  The debug library is swapped in for each test and the release
library put back after it; sessions never outlive the swap.
"""
import os

import pytest
import torch

from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import build as lib_build
from moe_alltoallv_resident_amd import workloads as W
from tests import test_errors_gpu as errors
from tests import test_parity_gpu as parity

pytestmark = pytest.mark.gpu

PATHS = [a2av.PATH_STAGED, a2av.PATH_DIRECT]
PATH_IDS = ["staged", "direct"]
LAYOUTS = [a2av.LAYOUT_SOURCE_MAJOR, a2av.LAYOUT_EXPERT_MAJOR]
LAYOUT_IDS = ["srcmaj", "expmaj"]


@pytest.fixture
def debug_library():
    if not os.path.exists(lib_build.DEBUG_LIB):
        raise RuntimeError(f"{lib_build.DEBUG_LIB} is missing: build it with __graft_entry__.build()")
    saved_lib, saved_path = a2av._lib, a2av.LIB_PATH
    torch.cuda.synchronize()
    a2av._lib, a2av.LIB_PATH = None, lib_build.DEBUG_LIB
    try:
        lib = a2av.lib()
        assert os.path.basename(lib._name) == "liba2av_debug.so"
        yield lib
    finally:
        torch.cuda.synchronize()
        a2av._lib, a2av.LIB_PATH = saved_lib, saved_path


CASES = [
    ("decode", {}),                                                   # one launch, top-1
    ("edge", {}),                                                     # one launch, 64 ranks
    # one launch with 4 KiB rows cut into four pieces that split their count
    ("wide", dict(num_ranks=4, tokens_per_rank=16, hidden=2048, experts_per_rank=4, top_k=7)),
    ("decode", dict(tokens_per_rank=600, hidden=256)),                # planned, top-1 scatter pack
    ("wide", dict(tokens_per_rank=200, hidden=512)),                  # planned, top-8
    ("decode", dict(num_ranks=3, tokens_per_rank=5001, hidden=8)),    # planned in chunks
    # receive capacity overflow and out-of-range ids, one launch and planned
    ("wide", dict(num_ranks=4, tokens_per_rank=30, hidden=64, experts_per_rank=2, top_k=2,
                  recv_capacity_rows=20)),
    ("decode", dict(num_ranks=4, tokens_per_rank=1100, hidden=64, recv_capacity_rows=800)),
    ("tiny", {}),                                                     # float32 rows
]


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("name,over", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_debug_build_matches_oracle(debug_library, name, over, path, layout):
    w = W.workload(name, **over)
    x, ids, gates = W.make_inputs(w)
    if over.get("recv_capacity_rows"):
        ids = ids.copy()
        ids[0, 1, 0] = -3
        ids[w.num_ranks - 1, w.tokens_per_rank - 1, w.top_k - 1] = w.num_experts
    parity._full_oracle_check(w, x, ids, gates, path, layout)


@pytest.mark.parametrize("tokens,hidden", [(64, 2048), (1100, 96)], ids=["one-launch", "planned"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_debug_build_overflow_keeps_guard_rows(debug_library, path, layout, tokens, hidden):
    errors.test_receive_overflow_keeps_guard_rows_and_true_counts(path, layout, tokens, hidden)


# the gather-form pack, the receive-order exchange and the non-temporal copies (top-1),
# the top-k pack through the caches and the paired-slot combine (top-8), with the hottest
# receiver over its capacity
@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("name,over", errors.STREAMING_OVERFLOW, ids=["top1", "top8"])
def test_debug_build_at_streaming_sizes(debug_library, name, over, path, layout):
    errors.test_receive_overflow_at_streaming_sizes(name, over, path, layout)


def test_debug_build_bare_collective(debug_library):
    errors.test_bare_alltoallv_matches_oracle_exchange(6, 40, 64)
