"""Shared pieces of the GPU tests: moving seeded inputs to the device, running the HIP path
through the C ABI, and comparing with the CPU oracle.

Comparison rules (the bar the tests hold the HIP path to):
  - counts, offsets, positions, receive rows and expert-stand-in rows: bit-exact;
  - combine: every element within max(1e-3 * |ref|, one unit in the last place of the
    output dtype at |ref|) of the oracle's fp64 result rounded once, and the norm-wise
    relative error within 1e-3.  Why one unit in the last place: the GPU sums k products
    in float32 with one rounding per FMA; with positive gates and experts that scale by
    positive factors every term of a token's sum has the same sign, so the float32 sum is
    within k * 2^-24 (relative) of the exact sum; rounding that value and the exact value
    to the dtype gives the same result or two neighbours.  A bare 1e-3 relative test
    would be tighter than one bf16 step (2^-8 .. 2^-7 relative) and fail on any
    neighbour.
"""
import numpy as np
import torch

import oracle
from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W


def banner(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def to_device(w: W.Workload, x, ids, gates):
    if w.dtype == W.BF16:
        xt = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x))
    return xt.cuda(), torch.from_numpy(np.ascontiguousarray(ids)).cuda(), torch.from_numpy(
        np.ascontiguousarray(gates)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy raw values (uint16 for bf16, float32, int32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == W.BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ulp(ref: np.ndarray, dtype: int) -> np.ndarray:
    sp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    return sp * (65536.0 if dtype == W.BF16 else 1.0)


def assert_combine_close(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: int, what: str = "") -> float:
    """Returns the fraction of bit-identical elements."""
    if y_ref.size == 0:
        assert y_gpu.size == 0
        return 1.0
    g = as_f64(y_gpu, dtype)
    r = as_f64(y_ref, dtype)
    diff = np.abs(g - r)
    allowed = np.maximum(1e-3 * np.abs(r), ulp(r, dtype))
    bad = diff > allowed
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, e.g. at {idx.tolist()}: "
                             f"gpu {g[tuple(idx[0])]} ref {r[tuple(idx[0])]}")
    nr = np.linalg.norm(r)
    assert np.linalg.norm(g - r) <= 1e-3 * max(nr, 1e-30), f"{what}: norm-wise error too large"
    return float(np.mean(y_gpu == y_ref))


class Run:
    """One dispatch -> expert stand-in -> combine pass of the HIP path, step by step,
    with the tables and rows copied to the host for comparison."""

    def __init__(self, w: W.Workload, x, ids, gates, session=None, path=a2av.PATH_STAGED,
                 layout=a2av.LAYOUT_SOURCE_MAJOR, device_inputs=None):
        self.w = w
        self.x_dev, self.ids_dev, self.gates_dev = device_inputs or to_device(w, x, ids, gates)
        self.session = session or a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype,
                                               w.experts_per_rank, w.top_k, w.recv_capacity_rows, path=path,
                                               recv_layout=layout)
        self.layout = self.session.recv_layout
        self.recv = self.z = None

    def dispatch(self, keep_recv=True):
        s, R = self.session, self.w.num_ranks
        s.status.zero_()
        s.dispatch(self.x_dev, self.ids_dev)
        self.split = host_bits(s.split)
        self.recv_counts = host_bits(s.recv_counts)
        self.recv_off = host_bits(s.recv_offsets)
        self.pos = host_bits(s.positions())
        self.send_off = host_bits(s.send_offsets())
        self.recv_eoff = host_bits(s.recv_expert_offsets()) if self.layout == a2av.LAYOUT_EXPERT_MAJOR else None
        self.valid = [int(min(self.recv_off[d, R], s.cap)) for d in range(R)]
        if keep_recv:
            self.recv = [host_bits(s.recv[d, :self.valid[d]]) for d in range(R)]
        return self

    def expert(self, keep_z=True):
        s, R = self.session, self.w.num_ranks
        if self.w.expert_mode == W.EXPERT_SCALE:
            s.expert(s.recv, s.recv, a2av.EXPERT_SCALE)          # in place
        if keep_z:
            self.z = [host_bits(s.recv[d, :self.valid[d]]) for d in range(R)]
        return self

    def combine(self):
        s = self.session
        self.y_dev = torch.empty_like(self.x_dev)
        s.combine(s.recv, self.gates_dev, self.y_dev)
        self.y = host_bits(self.y_dev)
        torch.cuda.synchronize()
        self.status = int(s.status.item())
        return self

    def all(self, keep=True):
        return self.dispatch(keep).expert(keep).combine()


def oracle_tables(w: W.Workload, ids, layout=oracle.SOURCE_MAJOR):
    """The oracle's dispatch with 4-byte tag rows (global token index): the full routing
    at any size, cheap because no hidden-size rows are moved."""
    R, T = w.num_ranks, w.tokens_per_rank
    tags = np.arange(R * T, dtype=np.int32).reshape(R, T, 1)
    d = oracle.dispatch(oracle.as_rows(tags), ids, w.experts_per_rank, w.capacity, layout)
    d["recv_tags"] = d["recv"].view(np.int32).reshape(R, w.capacity)
    return d


def assert_tables_equal(run: Run, ref: dict, R: int):
    assert np.array_equal(run.split, ref["cnt"]), "split table"
    assert np.array_equal(run.send_off, ref["send_off"]), "send offsets"
    assert np.array_equal(run.recv_counts, ref["recv_counts"]), "receive counts"
    assert np.array_equal(run.recv_off, ref["recv_off"]), "receive offsets"
    assert np.array_equal(run.pos, ref["pos"]), "positions"
    if run.recv_eoff is not None:
        assert np.array_equal(run.recv_eoff, ref["recv_eoff"]), "expert group starts"
