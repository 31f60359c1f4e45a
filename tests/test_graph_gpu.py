"""A decode step captured once in a hipGraph (through torch.cuda.graph) and replayed with
routing that changes on the device every step: router stand-in -> dispatch -> expert
stand-in -> combine.  Capture itself fails if any captured call synchronises or copies to
the host, so a successful capture shows the step has no host synchronisation; every
replay is checked against the oracle for its own routing, with eager GPU work and host
synchronisations between replays.

The pages' reason for this test: under a captured graph a host-side all-to-allv has to
pad every count to the worst case, while counts resident on the GPU let each replay send
exactly what the router chose (abhik.ai "Collective Communication for 100k+ GPUs",
section "Inference: small messages, unknown sizes"; qiguanping.github.io "NCCLX",
section 7, figure 14).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W
from tests.gpu_util import assert_combine_close, banner, host_bits, to_device

pytestmark = pytest.mark.gpu


def _tables(w, steps):
    ids = np.stack([W.make_ids(w, i) for i in range(steps)])
    gates = np.stack([W.make_gates(w, i) for i in range(steps)])
    return ids, gates


@pytest.mark.parametrize("path,layout", [(a2av.PATH_STAGED, 0), (a2av.PATH_DIRECT, 0), (a2av.PATH_DIRECT, 1)],
                         ids=["staged", "direct", "direct-expmaj"])
# decode and edge dispatch in one launch; the 640-token decode plans first
@pytest.mark.parametrize("name,over,steps,full_every", [("decode", {}, 100, 10), ("edge", {}, 24, 1),
                                                        ("decode", dict(tokens_per_rank=640), 24, 8)],
                         ids=["decode", "edge", "decode-planned"])
def test_graph_replay_with_device_side_routing(name, over, steps, full_every, path, layout):
    w = W.workload(name, **over)
    banner(f"graph replay {w.describe()} steps={steps} path={path} layout={layout}")
    x = W.make_x(w)
    ids_tab, gates_tab = _tables(w, steps)
    xt, _, _ = to_device(w, x, ids_tab[0], gates_tab[0])
    n = w.tokens * w.top_k
    ids_table = torch.from_numpy(ids_tab.reshape(steps, n)).cuda()
    gates_table = torch.from_numpy(gates_tab.reshape(steps, n)).cuda()
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids = torch.empty((w.num_ranks, w.tokens_per_rank, w.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((w.num_ranks, w.tokens_per_rank, w.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty_like(xt)
    s = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k, path=path,
                     recv_layout=layout)

    def step():
        a2av.a2av_route_step(ids_table, gates_table, steps, n, counter, ids, gates)
        s.dispatch(xt, ids)
        s.expert(s.recv, s.recv, w.expert_mode)
        s.combine(s.recv, gates, y)

    # warm up eagerly on a side stream (as graph capture wants), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    counter.zero_()
    s.status.zero_()

    seen_counts = set()
    for i in range(steps):
        g.replay()
        # unrelated eager work and a host synchronisation between replays
        _ = (xt[:1].float() * 2).sum().item()
        torch.cuda.synchronize()
        assert int(counter.item()) == i + 1
        rc = host_bits(s.recv_counts)
        seen_counts.add(rc.tobytes())
        ref = oracle.dispatch(oracle.as_rows(np.arange(w.tokens, dtype=np.int32).reshape(
            w.num_ranks, w.tokens_per_rank, 1)), ids_tab[i], w.experts_per_rank, w.capacity)
        assert np.array_equal(rc, ref["recv_counts"]), f"replay {i}: receive counts"
        assert np.array_equal(host_bits(s.recv_offsets), ref["recv_off"]), f"replay {i}: receive offsets"
        assert np.array_equal(host_bits(s.split), ref["cnt"]), f"replay {i}: split table"
        span = w.tokens if i % full_every == 0 else 64
        a = 0 if span == w.tokens else (i * 997) % (w.tokens - span)
        yref = oracle.closed_form(x, ids_tab[i], gates_tab[i], w.experts_per_rank, w.dtype, w.expert_mode,
                                  a, a + span)
        yg = host_bits(y).reshape(w.tokens, w.hidden)[a:a + span]
        assert_combine_close(yg, yref.reshape(span, w.hidden), w.dtype, f"replay {i}")
    assert int(s.status.item()) == 0
    assert len(seen_counts) > steps // 2, "routing did not change across replays"
    banner(f"  {steps} replays match the oracle; {len(seen_counts)} distinct count tables")
    s.close()
    del g
    torch.cuda.empty_cache()
