"""Brute force through the HIP path: every expert-id pattern (repeats included) for two
ranks at the small shapes the oracle itself is brute-forced on, plus patterns with
out-of-range ids and with a receive capacity below the worst case, on both data paths
and both receive layouts, compared with the CPU oracle pattern by pattern.

Definition under test: abhik.ai "Collective Communication for 100k+ GPUs", section
"Inference: small messages, unknown sizes", Figure 13 (tokens sorted by expert into a
send buffer, an all-to-allv to the rank holding each expert, received counts returned),
and the combine of qiguanping.github.io "NCCLX", section 7, figure 13.

Every pattern is one dispatch + combine on one handle per (shape, path, layout); each
call writes its tables, positions, receive rows, combine output and status word into
its own slice of preallocated device arrays, and everything comes back to the host in
one copy per array.  Token rows are small integers in float32 and gates are 1/2 and
1/4, so every combine sum is exact and the combine is compared bit for bit as well.
These shapes all run the one-launch dispatch, whose placement count (a branch-free
ballot over the ids keyed on expert and index) is what the enumeration exercises:
every tie and every repeat of an expert within and across tokens.
"""
import ctypes
import itertools

import numpy as np
import pytest
import torch

import oracle
from moe_alltoallv_resident_amd import a2av
from moe_alltoallv_resident_amd import workloads as W
from tests.gpu_util import banner

pytestmark = pytest.mark.gpu

R = 2
H = 4   # float32 elements per row: 16-byte rows

# grouped by layout: the oracle's result depends on the layout only, and is kept for one
# (shape, layout) at a time
PATHS = [(a2av.PATH_STAGED, a2av.LAYOUT_SOURCE_MAJOR), (a2av.PATH_DIRECT, a2av.LAYOUT_SOURCE_MAJOR),
         (a2av.PATH_STAGED, a2av.LAYOUT_EXPERT_MAJOR), (a2av.PATH_DIRECT, a2av.LAYOUT_EXPERT_MAJOR)]
PATH_IDS = ["staged-srcmaj", "direct-srcmaj", "staged-expmaj", "direct-expmaj"]

# (tokens per rank T, experts E, top-k, id values (None: every expert), receive capacity
# (0: the worst case R*T*min(k, E/R)))
CASES = [
    (2, 2, 1, None, 0),
    (2, 2, 2, None, 0),
    (2, 4, 1, None, 0),
    (2, 4, 2, None, 0),
    (4, 2, 1, None, 0),
    (4, 4, 1, None, 0),
    (2, 2, 1, (-1, 0, 1, 2), 0),        # out-of-range ids on either side of [0, E)
    (2, 4, 2, (-1, 0, 3, 4), 0),
    (2, 2, 2, None, 3),                 # capacity below the worst case: rows dropped, flagged
    (4, 2, 1, None, 2),
]
CASE_IDS = [f"T{T}-E{E}-k{k}" + ("-oor" if v else "") + (f"-cap{c}" if c else "")
            for T, E, k, v, c in CASES]


def _patterns(T, E, k, values):
    vals = np.arange(E, dtype=np.int32) if values is None else np.asarray(values, np.int32)
    combos = np.array(list(itertools.product(range(len(vals)), repeat=R * T * k)), dtype=np.int64)
    return vals[combos].reshape(-1, R, T, k)


def _rows(T):
    """Token rows: small integers in float32, distinct per token."""
    n = np.arange(1, R * T + 1, dtype=np.float32).reshape(R, T, 1)
    return np.concatenate([n, 2 * n, -n, 3 * n], axis=2).astype(np.float32)


def _gates(T, k):
    g = np.array([0.5, 0.25][:k], np.float32)
    return np.broadcast_to(g, (R, T, k)).copy()


def _oracle_all(pats, x, gates, epr, cap, layout):
    """The oracle's tables, positions, receive rows, status and combine, per pattern."""
    P, _, T, k = pats.shape
    E = R * epr
    out = dict(split=np.zeros((P, R, E), np.int32), recv_counts=np.zeros((P, R, R), np.int32),
               recv_off=np.zeros((P, R, R + 1), np.int32), pos=np.zeros((P, R, T, k), np.int32),
               recv_eoff=np.zeros((P, R, epr + 1), np.int32), recv=np.zeros((P, R, cap, H), np.float32),
               status=np.zeros(P, np.int32), y=np.zeros((P, R, T, H), np.float32))
    for p in range(P):
        d = oracle.full_step(x, pats[p], gates, epr, W.F32, W.EXPERT_IDENTITY, cap, layout)
        out["split"][p] = d["cnt"]
        out["recv_counts"][p] = d["recv_counts"]
        out["recv_off"][p] = d["recv_off"]
        out["pos"][p] = d["pos"]
        out["recv_eoff"][p] = d["recv_eoff"]
        out["recv"][p] = d["recv"]
        out["status"][p] = d["status"]
        out["y"][p] = d["y"]
    return out


def _gpu_all(pats, x, gates, epr, cap, path, layout):
    P, _, T, k = pats.shape
    E = R * epr
    cfg = a2av.make_config(R, T, H, W.F32, epr, k, cap, path, layout)
    h = a2av.a2av_create(cfg)
    dev = "cuda"
    xt = torch.from_numpy(x).to(dev)
    gt = torch.from_numpy(gates).to(dev)
    ids = torch.from_numpy(np.ascontiguousarray(pats)).to(dev)
    recv = torch.zeros((P, R, cap, H), dtype=torch.float32, device=dev)
    split = torch.full((P, R, E), -9, dtype=torch.int32, device=dev)
    rc = torch.full((P, R, R), -9, dtype=torch.int32, device=dev)
    ro = torch.full((P, R, R + 1), -9, dtype=torch.int32, device=dev)
    pos = torch.full((P, R, T, k), -9, dtype=torch.int32, device=dev)
    reo = torch.full((P, R, epr + 1), -9, dtype=torch.int32, device=dev)
    y = torch.full((P, R, T, H), -9.0, dtype=torch.float32, device=dev)
    st = torch.zeros(P, dtype=torch.int32, device=dev)
    L = a2av.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hp = h
    A = R * T * k
    strides = dict(ids=A * 4, recv=R * cap * H * 4, split=R * E * 4, rc=R * R * 4, ro=R * (R + 1) * 4,
                   pos=A * 4, reo=R * (epr + 1) * 4, y=R * T * H * 4, st=4)
    base = dict(ids=ids.data_ptr(), recv=recv.data_ptr(), split=split.data_ptr(), rc=rc.data_ptr(),
                ro=ro.data_ptr(), pos=pos.data_ptr(), reo=reo.data_ptr(), y=y.data_ptr(), st=st.data_ptr())
    expmaj = layout == a2av.LAYOUT_EXPERT_MAJOR
    xp, gp = xt.data_ptr(), gt.data_ptr()
    bad = 0
    for p in range(P):
        at = {n: base[n] + p * strides[n] for n in base}
        bad |= L.a2av_dispatch(hp, xp, at["ids"], at["recv"], at["split"], at["rc"], at["ro"], at["st"], stream)
        bad |= L.a2av_copy_positions(hp, at["pos"], stream)
        if expmaj:
            bad |= L.a2av_copy_recv_expert_offsets(hp, at["reo"], stream)
        bad |= L.a2av_combine(hp, at["recv"], gp, at["y"], at["st"], stream)
    torch.cuda.synchronize()
    a2av.a2av_destroy(h)
    assert bad == 0, "a library call returned an error"
    out = dict(split=split.cpu().numpy(), recv_counts=rc.cpu().numpy(), recv_off=ro.cpu().numpy(),
               pos=pos.cpu().numpy(), recv=recv.cpu().numpy(), status=st.cpu().numpy(), y=y.cpu().numpy())
    if expmaj:
        out["recv_eoff"] = reo.cpu().numpy()
    return out


_ORACLE_CACHE = {}


@pytest.mark.parametrize("path,layout", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("T,E,k,values,cap", CASES, ids=CASE_IDS)
def test_every_id_pattern_two_ranks_matches_oracle(T, E, k, values, cap, path, layout):
    epr = E // R
    cap = cap or R * T * min(k, epr)
    pats = _patterns(T, E, k, values)
    P = pats.shape[0]
    x, gates = _rows(T), _gates(T, k)
    key = (T, E, k, values, cap, layout)
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()   # keep one (shape, layout) at a time
        banner(f"brute force T={T} E={E} k={k} values={values} cap={cap}: oracle on {P} patterns")
        _ORACLE_CACHE[key] = _oracle_all(pats, x, gates, epr, cap, layout)
    ref = _ORACLE_CACHE[key]
    banner(f"  HIP path {PATH_IDS[PATHS.index((path, layout))]}: {P} dispatch+combine calls")
    got = _gpu_all(pats, x, gates, epr, cap, path, layout)
    names = ["split", "recv_counts", "recv_off", "pos", "status", "recv", "y"]
    if layout == a2av.LAYOUT_EXPERT_MAJOR:
        names.append("recv_eoff")
    for n in names:
        a, b = got[n], ref[n]
        if n in ("recv", "y"):
            a, b = a.view(np.uint32), b.view(np.uint32)   # bit for bit
        same = (a == b).reshape(P, -1).all(axis=1)
        if not same.all():
            p = int(np.argmin(same))
            raise AssertionError(f"{n} differs from the oracle on {int((~same).sum())} of {P} patterns, first "
                                 f"ids {pats[p].tolist()}: gpu {got[n][p].tolist()} oracle {ref[n][p].tolist()}")
    if values is not None:
        assert (ref["status"] & oracle.ST_EXPERT_RANGE).any()
    if cap < R * T * min(k, epr):
        assert (ref["status"] & oracle.ST_RECV_OVERFLOW).any()
