"""Handles on separate streams, and one handle moved between streams.

A handle owns its workspace, and its kernels touch only that workspace and the caller's
buffers, so the steps of different handles enqueued on different streams may run at
the same time; each must give exactly its result on its own (receive rows bit-exact
against the oracle, the combine within the oracle tolerance, status clear).  One handle
may also be driven from two streams when the caller orders them (an event between the
dispatch on one and the combine on the other, and back).  Every stream keeps the
default priority.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W
from tests.gpu_util import assert_combine_close, banner, host_bits, to_device

pytestmark = pytest.mark.gpu

SHAPES = [
    ("decode", {}, a2av.PATH_DIRECT, a2av.LAYOUT_SOURCE_MAJOR),                      # one launch
    ("edge", {}, a2av.PATH_STAGED, a2av.LAYOUT_SOURCE_MAJOR),                        # one launch, 64 ranks
    ("wide", dict(tokens_per_rank=16), a2av.PATH_DIRECT, a2av.LAYOUT_EXPERT_MAJOR),  # one launch, top-8
    ("decode", dict(tokens_per_rank=600, hidden=512), a2av.PATH_STAGED,
     a2av.LAYOUT_EXPERT_MAJOR),                                                      # planned
    ("prefill", dict(tokens_per_rank=1024, hidden=1024), a2av.PATH_DIRECT,
     a2av.LAYOUT_SOURCE_MAJOR),                                                      # planned, Zipf(1.2)
]


def _check_against_oracle(w, s, y, ref, what):
    R = w.num_ranks
    assert int(s.status.item()) == ref["status"] == 0, what
    ro = host_bits(s.recv_offsets)
    assert np.array_equal(ro, ref["recv_off"]), f"{what}: receive offsets"
    got = host_bits(s.recv)
    for d in range(R):
        n = min(int(ref["recv_off"][d, R]), w.capacity)
        assert np.array_equal(got[d, :n], ref["z"][d, :n]), f"{what}: expert rows of rank {d}"
    assert_combine_close(host_bits(y), ref["y"], w.dtype, what)


def test_handles_on_separate_streams_run_together():
    jobs = []
    for name, over, path, layout in SHAPES:
        w = W.workload(name, **over)
        x, ids, gates = W.make_inputs(w)
        xt, idt, gt = to_device(w, x, ids, gates)
        s = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k,
                         w.recv_capacity_rows, path=path, recv_layout=layout)
        ref = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, w.capacity, layout)
        jobs.append(dict(w=w, s=s, xt=xt, idt=idt, gt=gt, y=torch.empty_like(xt), ref=ref,
                         stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    banner(f"{len(jobs)} handles on {len(jobs)} streams, 5 steps each, enqueued round-robin")
    for _ in range(5):
        for j in jobs:      # every stream gets its next step before any stream waits
            s, st = j["s"], j["stream"]
            with torch.cuda.stream(st):
                s.dispatch(j["xt"], j["idt"], stream=st)
                s.expert(s.recv, s.recv, j["w"].expert_mode, stream=st)
                s.combine(s.recv, j["gt"], j["y"], stream=st)
    torch.cuda.synchronize()
    for j in jobs:
        _check_against_oracle(j["w"], j["s"], j["y"], j["ref"], j["w"].describe())
        j["s"].close()


@pytest.mark.parametrize("path", [a2av.PATH_STAGED, a2av.PATH_DIRECT], ids=["staged", "direct"])
def test_one_handle_across_two_streams_in_caller_order(path):
    # decode steps with fresh routing: dispatch and the expert on one stream, the combine
    # on the other after an event, the next dispatch after an event back
    w = W.workload("decode")
    x = W.make_x(w)
    s = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k,
                     path=path)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    xt = to_device(w, x, W.make_ids(w, 0), W.make_gates(w, 0))[0]
    steps = 4
    inputs, ys, zs = [], [], []
    for i in range(steps):
        ids, gates = W.make_ids(w, i), W.make_gates(w, i)
        _, idt, gt = to_device(w, x, ids, gates)
        inputs.append((ids, gates, idt, gt))
        ys.append(torch.empty_like(xt))
    torch.cuda.synchronize()
    back = None
    for i, (_, _, idt, gt) in enumerate(inputs):
        if back is not None:
            a.wait_event(back)
        with torch.cuda.stream(a):
            s.dispatch(xt, idt, stream=a)
            s.expert(s.recv, s.recv, w.expert_mode, stream=a)
            z = s.recv.clone()              # this step's expert rows, before the next dispatch
            zs.append(z)
            there = torch.cuda.Event()
            there.record(a)
        b.wait_event(there)
        with torch.cuda.stream(b):
            s.combine(s.recv, gt, ys[i], stream=b)
            back = torch.cuda.Event()
            back.record(b)
    torch.cuda.synchronize()
    assert int(s.status.item()) == 0
    for i, (ids, gates, _, _) in enumerate(inputs):
        ref = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, w.capacity)
        got = host_bits(zs[i])
        for d in range(w.num_ranks):
            n = min(int(ref["recv_off"][d, w.num_ranks]), w.capacity)
            assert np.array_equal(got[d, :n], ref["z"][d, :n]), f"step {i}: expert rows of rank {d}"
        assert_combine_close(host_bits(ys[i]), ref["y"], w.dtype, f"step {i}")
    s.close()
