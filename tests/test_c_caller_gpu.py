"""The library used from plain C (tests/c_caller/c_caller.c): no Python binding and no
torch between the caller and the C ABI.  The program builds its inputs from integer
formulas, runs dispatch -> expert stand-in (identity) -> combine on the direct and the
staged path, and writes back what it read; this test rebuilds the same inputs with
numpy and checks every table and receive row bit-exact and y to the combine tolerance
against the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_combine_close, banner

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_caller", "c_caller")
R, T, H, EPR, K = 4, 64, 128, 2, 2
E = R * EPR
CAP = R * T * K


def _inputs():
    s = np.arange(R)[:, None, None]
    t = np.arange(T)[None, :, None]
    h = np.arange(H)[None, None, :]
    x = ((s * 256 + t).astype(np.float32) + (h / 128.0).astype(np.float32)).astype(np.float32)
    j = np.arange(K)[None, None, :]
    ids = ((s * 3 + t * 5 + j * 3) % E).astype(np.int32)
    gates = np.broadcast_to(np.where(j == 0, 0.75, 0.25), (R, T, K)).astype(np.float32)
    return np.ascontiguousarray(x), np.ascontiguousarray(ids), np.ascontiguousarray(gates)


def test_plain_c_caller_matches_oracle(tmp_path):
    assert os.path.exists(EXE), f"{EXE} is missing: build it with __graft_entry__.build()"
    out = tmp_path / "c_caller.bin"
    banner("plain C caller: R4 T64 H128 f32 E8 top2, direct then staged")
    r = subprocess.run([EXE, str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    x, ids, gates = _inputs()
    ref = oracle.full_step(x, ids, gates, EPR, oracle.F32, 0, CAP)
    raw = out.read_bytes()
    per_path = 4 + 4 * R * R + 4 * R * (R + 1) + 4 * R * CAP * H + 4 * R * T * H
    assert len(raw) == 2 * per_path
    for i, name in enumerate(("direct", "staged")):
        b = raw[i * per_path:(i + 1) * per_path]
        o = 0

        def take(n, dt):
            nonlocal o
            a = np.frombuffer(b, dtype=dt, count=n, offset=o)
            o += n * np.dtype(dt).itemsize
            return a

        status = int(take(1, np.uint32)[0])
        counts = take(R * R, np.int32).reshape(R, R)
        offs = take(R * (R + 1), np.int32).reshape(R, R + 1)
        recv = take(R * CAP * H, np.uint32).reshape(R, CAP, H)
        y = take(R * T * H, np.uint32).reshape(R, T, H)
        assert status == 0, name
        assert np.array_equal(counts, ref["recv_counts"]), f"{name}: receive counts"
        assert np.array_equal(offs, ref["recv_off"]), f"{name}: receive offsets"
        want = ref["recv"].view(np.uint32)
        for d in range(R):
            n = int(ref["recv_off"][d, R])
            assert np.array_equal(recv[d, :n], want[d, :n]), f"{name}: receive rows of rank {d}"
        assert_combine_close(y, ref["y"].view(np.uint32), oracle.F32, f"{name}: combine")
