"""CPU oracle for MoE dispatch/combine over a GPU-resident-metadata all-to-allv.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and bench.py's cpu_baseline leg may use
this package; the product path never imports it, and it imports nothing from the product
path.  The arithmetic lives in ``a2av_oracle.c`` (plain single-threaded C, fp64); this
module only loads that library and marshals numpy arrays.  ``naive`` holds a second,
independent nested-loop formulation used to pin the C oracle on small inputs.

Sources: abhik.ai "Collective Communication for 100k+ GPUs", section "Inference: small
messages, unknown sizes" (Figure 13: router, sort by expert into a send buffer,
all-to-allv to the expert's GPU; counts read by reference on the GPU, received counts
returned); qiguanping.github.io "NCCLX", section 7 (figures 13-18: dispatch and
combine, metadata resident on the GPU and consumed by kernels).
"""
import ctypes
import os

import numpy as np

F32 = 0
BF16 = 1
ST_EXPERT_RANGE = 1
ST_RECV_OVERFLOW = 2
SOURCE_MAJOR = 0
EXPERT_MAJOR = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# A2AV_ORACLE_SANITIZED=1 selects the AddressSanitizer/UBSan build of the same source
# (oracle/build.py), for a process started with the sanitizer runtime preloaded.
_SANITIZED = os.environ.get("A2AV_ORACLE_SANITIZED") == "1"
_LIB_PATH = os.path.join(_HERE, "liba2av_oracle_san.so" if _SANITIZED else "liba2av_oracle.so")
_lib = None


def library_path() -> str:
    """The oracle library this process loads."""
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build(sanitize=_SANITIZED)
        lib = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_dispatch.argtypes = [i32, i32, i32, i32, i64, i64, i32] + [vp] * 11
        lib.oracle_expert.argtypes = [i32, i32, i64, i32, i64, i32, i32, vp, vp, vp, vp]
        lib.oracle_return.argtypes = [i32, i32, i32, i32, i64, i64, i32, vp, vp, vp, vp, vp]
        lib.oracle_combine.argtypes = [i32, i32, i32, i64, i32, vp, vp, vp, vp]
        lib.oracle_closed_form.argtypes = [i32, i32, i32, i32, i64, i32, i32, vp, vp, vp, vp, i64, i64]
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        for f in ("oracle_dispatch", "oracle_expert", "oracle_return", "oracle_combine", "oracle_closed_form"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def elem_bytes(dtype: int) -> int:
    return 2 if dtype == BF16 else 4


def as_rows(x: np.ndarray) -> np.ndarray:
    """View any [..., H] array (float32, uint16 for bf16 bits, int32 tags) as raw bytes rows."""
    x = np.ascontiguousarray(x)
    return x.view(np.uint8).reshape(x.shape[:-1] + (x.shape[-1] * x.itemsize,))


def alloc_dispatch(R: int, T: int, k: int, row_bytes: int, experts_per_rank: int, cap: int) -> dict:
    """Zeroed output arrays of ``dispatch`` (to pass as its ``out``)."""
    E = R * experts_per_rank
    return dict(
        cnt=np.zeros((R, E), np.int32),
        send_off=np.zeros((R, R + 1), np.int32),
        pos=np.zeros((R, T, k), np.int32),
        send=np.zeros((R, T * k, row_bytes), np.uint8),
        recv_counts=np.zeros((R, R), np.int32),
        recv_off=np.zeros((R, R + 1), np.int32),
        recv_eoff=np.zeros((R, experts_per_rank + 1), np.int32),
        recv=np.zeros((R, cap, row_bytes), np.uint8),
    )


def dispatch(x_rows: np.ndarray, ids: np.ndarray, experts_per_rank: int, cap: int, layout: int = SOURCE_MAJOR,
             out: dict = None):
    """Sort by expert into send buffers, then the all-to-allv.

    x_rows: [R][T][row_bytes] uint8 (see ``as_rows``); ids: [R][T][k] int32.
    Returns a dict with cnt [R][E], send_off [R][R+1], pos [R][T][k], send [R][T*k][row],
    recv_counts [R][R] ([dst][src]), recv_off [R][R+1], recv_eoff [R][epr+1],
    recv [R][cap][row] (source- or expert-major), status.  ``out`` (from
    ``alloc_dispatch``) supplies the output arrays instead of fresh zeroed ones: only the
    receive rows a dispatch places are written, so rows past them keep what they held.
    """
    x_rows = _c(x_rows, np.uint8)
    ids = _c(ids, np.int32)
    R, T, k = ids.shape
    assert x_rows.shape[:2] == (R, T)
    row = x_rows.shape[2]
    if out is None:
        out = alloc_dispatch(R, T, k, row, experts_per_rank, cap)
    else:
        assert out["recv"].shape == (R, cap, row) and out["send"].shape == (R, T * k, row)
    st = np.zeros(1, np.uint32)
    rc = _load().oracle_dispatch(R, T, k, experts_per_rank, row, cap, layout, _p(x_rows), _p(ids),
                                 _p(out["cnt"]), _p(out["send_off"]), _p(out["pos"]), _p(out["send"]),
                                 _p(out["recv_counts"]), _p(out["recv_off"]), _p(out["recv_eoff"]),
                                 _p(out["recv"]), _p(st))
    if rc != 0:
        raise ValueError("oracle_dispatch rejected its arguments")
    out["status"] = int(st[0])
    return out


def expert(recv: np.ndarray, cnt: np.ndarray, recv_off: np.ndarray, experts_per_rank: int,
           dtype: int, mode: int, layout: int = SOURCE_MAJOR) -> np.ndarray:
    """Expert stand-in on received rows: mode 0 identity, mode 1 scale by 1 + e/256.

    recv: [R][cap][H] float32 or uint16 (bf16 bits).  Returns z of the same shape.
    """
    recv = np.ascontiguousarray(recv)
    R, cap, H = recv.shape
    z = np.zeros_like(recv)
    rc = _load().oracle_expert(R, experts_per_rank, H, dtype, cap, mode, layout,
                               _p(_c(cnt, np.int32)), _p(_c(recv_off, np.int32)), _p(recv), _p(z))
    if rc != 0:
        raise ValueError("oracle_expert rejected its arguments")
    return z


def return_exchange(z_rows: np.ndarray, send_off: np.ndarray, recv_off: np.ndarray, T: int, k: int,
                    cnt: np.ndarray = None, experts_per_rank: int = 1, layout: int = SOURCE_MAJOR,
                    out: np.ndarray = None) -> np.ndarray:
    """Return all-to-all.  z_rows: [R][cap][row] uint8.  Returns ret [R][T*k][row] uint8
    (``out``, if given: a [R][T*k][row] uint8 array to write into).
    The expert-major layout needs the split table cnt [R][E]."""
    z_rows = _c(z_rows, np.uint8)
    R, cap, row = z_rows.shape
    if cnt is None:
        cnt = np.zeros((R, R * experts_per_rank), np.int32)
    if out is None:
        ret = np.zeros((R, T * k, row), np.uint8)
    else:
        assert out.shape == (R, T * k, row) and out.dtype == np.uint8 and out.flags.c_contiguous
        ret = out
    rc = _load().oracle_return(R, T, k, experts_per_rank, row, cap, layout, _p(_c(cnt, np.int32)),
                               _p(_c(send_off, np.int32)), _p(_c(recv_off, np.int32)), _p(z_rows), _p(ret))
    if rc != 0:
        raise ValueError("oracle_return rejected its arguments")
    return ret


def combine(ret: np.ndarray, pos: np.ndarray, gates: np.ndarray, dtype: int, out: np.ndarray = None) -> np.ndarray:
    """Gate-weighted combine.  ret: [R][T*k][H] float32/uint16; pos, gates: [R][T][k].
    ``out``, if given, is the [R][T][H] array to write into."""
    ret = np.ascontiguousarray(ret)
    pos = _c(pos, np.int32)
    gates = _c(gates, np.float32)
    R, T, k = pos.shape
    H = ret.shape[2]
    if out is None:
        y = np.zeros((R, T, H), ret.dtype)
    else:
        assert out.shape == (R, T, H) and out.dtype == ret.dtype and out.flags.c_contiguous
        y = out
    rc = _load().oracle_combine(R, T, k, H, dtype, _p(pos), _p(gates), _p(ret), _p(y))
    if rc != 0:
        raise ValueError("oracle_combine rejected its arguments")
    return y


def closed_form(x: np.ndarray, ids: np.ndarray, gates: np.ndarray, experts_per_rank: int, dtype: int,
                mode: int, tok_begin: int = 0, tok_end=None) -> np.ndarray:
    """Layout-free end result y[s][t] = RNE(sum_j g * f_e(x[s][t])).

    Computes the tokens [tok_begin, tok_end) of the flattened [R*T] range and returns
    them as an array of shape [tok_end - tok_begin][H] (the full [R][T][H] when the
    whole range is asked for)."""
    x = np.ascontiguousarray(x)
    ids = _c(ids, np.int32)
    gates = _c(gates, np.float32)
    R, T, k = ids.shape
    H = x.shape[2]
    N = R * T
    whole = tok_begin == 0 and (tok_end is None or tok_end == N)
    if tok_end is None:
        tok_end = N
    tok_begin, tok_end = max(0, tok_begin), min(N, tok_end)
    y = np.zeros((max(0, tok_end - tok_begin), H), x.dtype)
    rc = _load().oracle_closed_form(R, T, k, experts_per_rank, H, dtype, mode, _p(x), _p(ids), _p(gates),
                                    _p(y), tok_begin, tok_end)
    if rc != 0:
        raise ValueError("oracle_closed_form rejected its arguments")
    return y.reshape(R, T, H) if whole else y


def full_step(x: np.ndarray, ids: np.ndarray, gates: np.ndarray, experts_per_rank: int, dtype: int,
              mode: int, cap: int, layout: int = SOURCE_MAJOR):
    """dispatch -> expert stand-in -> return -> combine, the whole staged path on the CPU."""
    x = np.ascontiguousarray(x)
    d = dispatch(as_rows(x), ids, experts_per_rank, cap, layout)
    R, T, H = x.shape
    k = ids.shape[2]
    recv = d["recv"].view(x.dtype).reshape(R, cap, H)
    z = expert(recv, d["cnt"], d["recv_off"], experts_per_rank, dtype, mode, layout)
    ret = return_exchange(as_rows(z), d["send_off"], d["recv_off"], T, k, d["cnt"], experts_per_rank, layout)
    y = combine(ret.view(x.dtype).reshape(R, T * k, H), d["pos"], gates, dtype)
    d.update(recv=recv, z=z, ret=ret.view(x.dtype).reshape(R, T * k, H), y=y)
    return d


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(bits)


def double_to_bf16(v: float) -> int:
    return _load().oracle_double_to_bf16(v)
