"""Seeded synthetic inputs for MoE dispatch/combine: token rows, routing and gates.

This module holds the input recipe only (random numbers and their shapes); it performs
none of the dispatch/combine arithmetic, and both the HIP path's tests and the CPU oracle
draw their inputs from it.

The workloads stand in for the pages' decode measurement (Llama 4 Maverick routing on
H100 hosts, abhik.ai "Collective Communication for 100k+ GPUs", section "Inference:
small messages, unknown sizes", Table 3), whose model, router and traces are not
available: token rows are N(0, 1), routing follows each workload's stated law, gates are
drawn as stated.  Seeds: numpy ``default_rng([seed, 1])`` for x, ``[seed, 2]`` for the
expert ids, ``[seed, 3]`` for the gates, ``default_rng(seed)`` for the permutation that
maps Zipf popularity ranks to expert ids; decode step i uses ``[seed, 2, i]`` and
``[seed, 3, i]``.
"""
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}

# expert stand-in: 0 = identity, 1 = per-expert scalar scale 1 + e/256
EXPERT_IDENTITY = 0
EXPERT_SCALE = 1


@dataclass(frozen=True)
class Workload:
    name: str
    num_ranks: int          # R virtual ranks
    tokens_per_rank: int    # T
    hidden: int             # H
    dtype: int              # F32 or BF16
    experts_per_rank: int   # epr; E = R * epr, expert e lives on rank e // epr
    top_k: int              # k
    routing: str            # "uniform" | "zipf" | "edge"
    gates: str              # "softmax" (over the k selected logits) | "sigmoid"
    expert_mode: int        # EXPERT_IDENTITY | EXPERT_SCALE
    zipf_s: float = 0.0
    steps: int = 1          # routing steps (decode: fresh routing per step)
    seed: int = 0
    recv_capacity_rows: int = 0   # per rank; 0 = worst case R*T*min(k, epr)
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def num_experts(self) -> int:
        return self.num_ranks * self.experts_per_rank

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    @property
    def row_bytes(self) -> int:
        return self.hidden * self.elem_bytes

    @property
    def tokens(self) -> int:
        return self.num_ranks * self.tokens_per_rank

    @property
    def assignments(self) -> int:
        return self.tokens * self.top_k

    @property
    def capacity(self) -> int:
        if self.recv_capacity_rows:
            return self.recv_capacity_rows
        return self.num_ranks * self.tokens_per_rank * min(self.top_k, self.experts_per_rank)

    def describe(self) -> str:
        return (f"{self.name}: R{self.num_ranks} T{self.tokens_per_rank} H{self.hidden} "
                f"{DTYPE_NAMES[self.dtype]} E{self.num_experts} top{self.top_k} {self.routing}"
                + (f"(s={self.zipf_s})" if self.routing == "zipf" else ""))


WORKLOADS = {
    "tiny": Workload("tiny", 4, 64, 128, F32, 2, 2, "uniform", "softmax", EXPERT_IDENTITY),
    "decode": Workload("decode", 8, 128, 5120, BF16, 16, 1, "zipf", "sigmoid", EXPERT_SCALE,
                       zipf_s=1.1, steps=100),
    "prefill": Workload("prefill", 8, 8192, 5120, BF16, 16, 1, "zipf", "sigmoid", EXPERT_SCALE,
                        zipf_s=1.2),
    # receive capacity twice the mean rows per rank (2 * 2048 * 8 = 32,768 rows, 470 MB per
    # rank) rather than the worst case (262,144 rows, 3.76 GB per rank, 60 GB in all)
    "wide": Workload("wide", 16, 2048, 7168, BF16, 16, 8, "uniform", "softmax", EXPERT_SCALE,
                     recv_capacity_rows=32768),
    "edge": Workload("edge", 64, 16, 2048, BF16, 1, 2, "edge", "softmax", EXPERT_SCALE),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced.  A named workload's receive
    capacity belongs to its own shape: when the shape changes (ranks, tokens, experts or
    top-k) and no capacity is given, the worst case is taken."""
    shape = {"num_ranks", "tokens_per_rank", "experts_per_rank", "top_k"}
    if shape & set(overrides) and "recv_capacity_rows" not in overrides:
        overrides = dict(overrides, recv_capacity_rows=0)
    return replace(WORKLOADS[name], **overrides)


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) with torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_x(w: Workload) -> np.ndarray:
    """Token rows [R][T][H]: float32 for F32, uint16 bf16 bit patterns for BF16."""
    rng = np.random.default_rng([w.seed, 1])
    x = rng.standard_normal((w.num_ranks, w.tokens_per_rank, w.hidden), dtype=np.float32)
    return x if w.dtype == F32 else _bf16_bits(x)


def zipf_expert_order(w: Workload) -> np.ndarray:
    """Popularity rank i -> expert id, a seeded permutation of the experts."""
    return np.random.default_rng(w.seed).permutation(w.num_experts).astype(np.int64)


def _uniform_topk(rng, n, E, k):
    # a uniformly random ordering of the experts per token; its first k are a uniform
    # k-subset without replacement, in random order
    return np.argsort(rng.random((n, E)), axis=1, kind="stable")[:, :k]


def _zipf_topk(rng, n, E, k, s, order):
    p = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    p /= p.sum()
    if k == 1:
        ranks = rng.choice(E, size=(n, 1), p=p)
    else:
        # without replacement, proportional to p: top-k of log p + Gumbel noise
        g = rng.gumbel(size=(n, E))
        ranks = np.argsort(-(np.log(p)[None, :] + g), axis=1, kind="stable")[:, :k]
    return order[ranks]


def _edge_topk(rng, w):
    """Latency/edge routing: 25 % of the ranks receive nothing, one rank receives 40 % of
    all assignments, the rest uniform without replacement over the remaining experts.
    Built for experts_per_rank == 1 (one expert per rank) and k == 2."""
    R, T, k, epr = w.num_ranks, w.tokens_per_rank, w.top_k, w.experts_per_rank
    E, N = w.num_experts, w.tokens
    A = N * k
    perm = rng.permutation(R)
    n_zero = R // 4
    hot_rank = int(perm[n_zero])
    live_ranks = perm[n_zero + 1:]
    live_experts = np.concatenate([np.arange(r * epr, (r + 1) * epr) for r in live_ranks])
    hot_expert = hot_rank * epr + int(rng.integers(epr))
    n_hot = int(round(0.4 * A))
    if n_hot > N:
        raise ValueError("edge routing: the hot rank would need more than one slot per token")
    ids = np.empty((N, k), np.int64)
    hot_tokens = np.zeros(N, bool)
    hot_tokens[rng.choice(N, size=n_hot, replace=False)] = True
    for n in range(N):
        if hot_tokens[n]:
            others = live_experts[_uniform_topk(rng, 1, len(live_experts), k - 1)[0]]
            slot = int(rng.integers(k))
            row = list(others)
            row.insert(slot, hot_expert)
            ids[n] = row
        else:
            ids[n] = live_experts[_uniform_topk(rng, 1, len(live_experts), k)[0]]
    w.extra.update(zero_ranks=sorted(int(r) for r in perm[:n_zero]), hot_rank=hot_rank)
    return ids


def make_ids(w: Workload, step: Optional[int] = None) -> np.ndarray:
    """Expert ids [R][T][k] int32."""
    seq = [w.seed, 2] if step is None else [w.seed, 2, step]
    rng = np.random.default_rng(seq)
    N, E, k = w.tokens, w.num_experts, w.top_k
    if w.routing == "uniform":
        ids = _uniform_topk(rng, N, E, k)
    elif w.routing == "zipf":
        ids = _zipf_topk(rng, N, E, k, w.zipf_s, zipf_expert_order(w))
    elif w.routing == "edge":
        ids = _edge_topk(rng, w)
    else:
        raise ValueError(w.routing)
    return ids.astype(np.int32).reshape(w.num_ranks, w.tokens_per_rank, k)


def make_gates(w: Workload, step: Optional[int] = None) -> np.ndarray:
    """Gates [R][T][k] float32, computed in float64 and stored once as float32."""
    seq = [w.seed, 3] if step is None else [w.seed, 3, step]
    rng = np.random.default_rng(seq)
    logits = rng.standard_normal((w.tokens, w.top_k))
    if w.gates == "sigmoid":
        g = 1.0 / (1.0 + np.exp(-logits))
    elif w.gates == "softmax":
        m = logits.max(axis=1, keepdims=True)
        ex = np.exp(logits - m)
        g = ex / ex.sum(axis=1, keepdims=True)
    else:
        raise ValueError(w.gates)
    return g.astype(np.float32).reshape(w.num_ranks, w.tokens_per_rank, w.top_k)


def make_inputs(w: Workload, step: Optional[int] = None):
    return make_x(w), make_ids(w, step), make_gates(w, step)

