"""Writes tests/golden/tiny_oracle.json from the CPU oracle alone.

The fixture locks the oracle's output on the tiny workload (4 ranks, 64 tokens per rank,
hidden 128 float32, 8 experts, top-2, identity experts, seed 0): the full metadata tables
and SHA-256 digests of the receive rows, the positions and the combined output.  A
change to the oracle that moves any of them fails tests/test_golden.py; regenerate only
with a reason taken from the pages (abhik.ai "Collective Communication for 100k+ GPUs",
section "Inference: small messages, unknown sizes").

Run: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from moe_alltoallv_resident_amd import workloads as W  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_fixture() -> dict:
    w = W.workload("tiny")
    x, ids, gates = W.make_inputs(w)
    out = oracle.full_step(x, ids, gates, w.experts_per_rank, w.dtype, w.expert_mode, w.capacity)
    recv_valid = [out["recv"][d, : out["recv_off"][d, w.num_ranks]] for d in range(w.num_ranks)]
    return {
        "workload": w.describe(),
        "source": "oracle.full_step (CPU oracle only)",
        "inputs_sha256": {"x": digest(x), "ids": digest(ids), "gates": digest(gates)},
        "cnt": out["cnt"].tolist(),
        "send_off": out["send_off"].tolist(),
        "recv_counts": out["recv_counts"].tolist(),
        "recv_off": out["recv_off"].tolist(),
        "status": out["status"],
        "sha256": {
            "recv_valid_rows": digest(np.concatenate(recv_valid)),
            "pos": digest(out["pos"]),
            "y": digest(out["y"]),
        },
    }


if __name__ == "__main__":
    path = os.path.join(HERE, "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(tiny_fixture(), f, indent=1)
        f.write("\n")
    print("wrote", path)
