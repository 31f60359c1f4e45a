"""Python binding of liba2av.so (include/a2av.h), argument marshalling only.

Every function has the name of the C entry point it calls and takes torch tensors (or
raw device addresses as ints) where the C call takes device pointers; the stream
defaults to torch's current stream.  No step of the path runs in Python: the library is
required, and a missing build raises at import of the first call.
"""
import ctypes
import os

import torch

F32 = 0
BF16 = 1
OK = 0
ERR_INVALID = -1
ERR_NOMEM = -2
ERR_HIP = -3
ERR_SCRATCH = -4
NOALLOC_MAX_RANKS = 256
NOALLOC_SCRATCH_BYTES = 1 << 20
ST_EXPERT_RANGE = 1
ST_RECV_OVERFLOW = 2
ST_BOUNDS = 4
EXPERT_IDENTITY = 0
EXPERT_SCALE = 1
PATH_STAGED = 0
PATH_DIRECT = 1
LAYOUT_SOURCE_MAJOR = 0
LAYOUT_EXPERT_MAJOR = 1
STAGES = 5
STREAM_READ = 0
STREAM_WRITE = 1
STREAM_READ_OUT_BYTES = 1 << 20
STAGE_NAMES = ("plan", "pack", "exchange", "return", "combine")

# A2AV_DEBUG=1 in the environment selects the debug build (device-side bounds checks,
# status bit ST_BOUNDS); same exports and results.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "liba2av_debug.so" if os.environ.get("A2AV_DEBUG") == "1" else "liba2av.so")
EXPORTS = ("a2av_create", "a2av_destroy", "a2av_workspace_bytes", "a2av_dispatch", "a2av_combine",
           "a2av_alltoallv", "a2av_alltoallv_noalloc", "a2av_copy_positions", "a2av_copy_recv_expert_offsets",
           "a2av_copy_send_offsets", "a2av_expert_apply", "a2av_route_step", "a2av_copy_reference",
           "a2av_stream_reference", "a2av_timing_begin", "a2av_timing_end", "a2av_error_string")

TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


class Config(ctypes.Structure):
    _fields_ = [("num_ranks", ctypes.c_int32), ("tokens_per_rank", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("experts_per_rank", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("recv_capacity_rows", ctypes.c_int64), ("path", ctypes.c_int32), ("recv_layout", ctypes.c_int32)]


class A2AVError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {code} ({error_string(code)})")
        self.code = code


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with moe_alltoallv_resident_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.a2av_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
        L.a2av_destroy.argtypes = [vp]
        L.a2av_workspace_bytes.argtypes = [ctypes.POINTER(Config)]
        L.a2av_workspace_bytes.restype = i64
        L.a2av_dispatch.argtypes = [vp] * 9
        L.a2av_combine.argtypes = [vp] * 6
        L.a2av_alltoallv.argtypes = [vp] * 8
        L.a2av_alltoallv_noalloc.argtypes = [ctypes.POINTER(Config)] + [vp] * 7
        L.a2av_copy_positions.argtypes = [vp, vp, vp]
        L.a2av_copy_send_offsets.argtypes = [vp, vp, vp]
        L.a2av_copy_recv_expert_offsets.argtypes = [vp, vp, vp]
        L.a2av_expert_apply.argtypes = [vp, vp, vp, i32, vp]
        L.a2av_route_step.argtypes = [vp, vp, i32, i64, vp, vp, vp, vp]
        L.a2av_copy_reference.argtypes = [vp, vp, i64, i64, vp]
        L.a2av_stream_reference.argtypes = [vp, vp, i64, i32, vp]
        L.a2av_timing_begin.argtypes = [vp, i32]
        L.a2av_timing_end.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
        L.a2av_error_string.argtypes = [ctypes.c_int]
        L.a2av_error_string.restype = ctypes.c_char_p
        for f in EXPORTS:
            if f not in ("a2av_workspace_bytes", "a2av_error_string"):
                getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def error_string(code: int) -> str:
    return lib().a2av_error_string(code).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("device tensors must be contiguous GPU tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(stream)


def _check(fn, rc):
    if rc != OK:
        raise A2AVError(fn, rc)


def make_config(num_ranks, tokens_per_rank, hidden, dtype, experts_per_rank, top_k, recv_capacity_rows=0,
                path=PATH_STAGED, recv_layout=LAYOUT_SOURCE_MAJOR) -> Config:
    return Config(num_ranks, tokens_per_rank, hidden, dtype, experts_per_rank, top_k, recv_capacity_rows, path,
                  recv_layout)


def a2av_workspace_bytes(cfg: Config) -> int:
    return lib().a2av_workspace_bytes(ctypes.byref(cfg))


def a2av_create(cfg: Config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check("a2av_create", lib().a2av_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def a2av_destroy(h) -> None:
    _check("a2av_destroy", lib().a2av_destroy(h))


def a2av_dispatch(h, x, topk_ids, recv, split, recv_counts, recv_offsets, status, stream=None) -> None:
    _check("a2av_dispatch", lib().a2av_dispatch(h, _ptr(x), _ptr(topk_ids), _ptr(recv), _ptr(split),
                                                _ptr(recv_counts), _ptr(recv_offsets), _ptr(status),
                                                _stream(stream)))


def a2av_combine(h, expert_out, gates, y, status, stream=None) -> None:
    _check("a2av_combine", lib().a2av_combine(h, _ptr(expert_out), _ptr(gates), _ptr(y), _ptr(status),
                                              _stream(stream)))


def a2av_alltoallv(h, send, send_counts, recv, recv_counts, recv_offsets, status, stream=None) -> None:
    _check("a2av_alltoallv", lib().a2av_alltoallv(h, _ptr(send), _ptr(send_counts), _ptr(recv),
                                                  _ptr(recv_counts), _ptr(recv_offsets), _ptr(status),
                                                  _stream(stream)))


def a2av_alltoallv_noalloc(cfg: Config, send, send_counts, recv, recv_counts, recv_offsets, status,
                           stream=None) -> None:
    _check("a2av_alltoallv_noalloc",
           lib().a2av_alltoallv_noalloc(ctypes.byref(cfg), _ptr(send), _ptr(send_counts), _ptr(recv),
                                        _ptr(recv_counts), _ptr(recv_offsets), _ptr(status), _stream(stream)))


def a2av_copy_positions(h, pos, stream=None) -> None:
    _check("a2av_copy_positions", lib().a2av_copy_positions(h, _ptr(pos), _stream(stream)))


def a2av_copy_recv_expert_offsets(h, recv_expert_offsets, stream=None) -> None:
    _check("a2av_copy_recv_expert_offsets",
           lib().a2av_copy_recv_expert_offsets(h, _ptr(recv_expert_offsets), _stream(stream)))


def a2av_copy_send_offsets(h, send_offsets, stream=None) -> None:
    _check("a2av_copy_send_offsets", lib().a2av_copy_send_offsets(h, _ptr(send_offsets), _stream(stream)))


def a2av_expert_apply(h, inp, out, mode, stream=None) -> None:
    _check("a2av_expert_apply", lib().a2av_expert_apply(h, _ptr(inp), _ptr(out), mode, _stream(stream)))


def a2av_route_step(ids_table, gates_table, steps, n, counter, ids, gates, stream=None) -> None:
    _check("a2av_route_step", lib().a2av_route_step(_ptr(ids_table), _ptr(gates_table), steps, n, _ptr(counter),
                                                    _ptr(ids), _ptr(gates), _stream(stream)))


def a2av_copy_reference(src, dst, rows, row_bytes, stream=None) -> None:
    _check("a2av_copy_reference", lib().a2av_copy_reference(_ptr(src), _ptr(dst), rows, row_bytes, _stream(stream)))


def _nbytes(t):
    return t.numel() * t.element_size() if isinstance(t, torch.Tensor) else None


def a2av_stream_reference(src, dst, nbytes, mode, stream=None) -> None:
    # the kernels write a fixed-size result (read) or nbytes (write): short tensors are
    # refused here rather than written past their end
    need_dst = STREAM_READ_OUT_BYTES if mode == STREAM_READ else nbytes
    if _nbytes(dst) is not None and _nbytes(dst) < need_dst:
        raise ValueError(f"a2av_stream_reference: dst holds {_nbytes(dst)} bytes, needs {need_dst}")
    if mode == STREAM_READ and _nbytes(src) is not None and _nbytes(src) < nbytes:
        raise ValueError(f"a2av_stream_reference: src holds {_nbytes(src)} bytes, reads {nbytes}")
    _check("a2av_stream_reference", lib().a2av_stream_reference(_ptr(src), _ptr(dst), nbytes, mode, _stream(stream)))


def a2av_timing_begin(h, max_calls) -> None:
    _check("a2av_timing_begin", lib().a2av_timing_begin(h, max_calls))


def a2av_timing_end(h):
    """Returns (ms_sum[5], launches[5]) per stage: plan, pack, exchange, return, combine."""
    ms = (ctypes.c_double * STAGES)()
    n = (ctypes.c_int32 * STAGES)()
    _check("a2av_timing_end", lib().a2av_timing_end(h, ms, n))
    return list(ms), list(n)


class Session:
    """A handle plus the caller-owned device buffers of one configuration.

    Allocates (once) recv [R][cap][H], split [R][E], recv_counts [R][R],
    recv_offsets [R][R+1] and status on the current GPU; dispatch/combine then only
    enqueue library calls, so they can be captured in a graph.
    """

    def __init__(self, num_ranks, tokens_per_rank, hidden, dtype, experts_per_rank, top_k,
                 recv_capacity_rows=0, path=PATH_STAGED, recv_layout=LAYOUT_SOURCE_MAJOR, device="cuda"):
        self.cfg = make_config(num_ranks, tokens_per_rank, hidden, dtype, experts_per_rank, top_k,
                               recv_capacity_rows, path, recv_layout)
        self.path = path
        self.recv_layout = recv_layout
        self.epr = experts_per_rank
        self.R, self.T, self.H, self.k = num_ranks, tokens_per_rank, hidden, top_k
        self.E = num_ranks * experts_per_rank
        self.cap = recv_capacity_rows or num_ranks * tokens_per_rank * min(top_k, experts_per_rank)
        self.dtype = dtype
        self.torch_dtype = TORCH_DTYPE[dtype]
        self.device = torch.device(device)
        with torch.cuda.device(self.device):
            self.handle = a2av_create(self.cfg)
        R = num_ranks
        self.recv = torch.empty((R, self.cap, hidden), dtype=self.torch_dtype, device=self.device)
        self.split = torch.empty((R, self.E), dtype=torch.int32, device=self.device)
        self.recv_counts = torch.empty((R, R), dtype=torch.int32, device=self.device)
        self.recv_offsets = torch.empty((R, R + 1), dtype=torch.int32, device=self.device)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)

    def _check_tensor(self, name, t, dtype, numel):
        # host-side checks only (no synchronisation): a wrong element type or a short
        # buffer would otherwise be read or written past its end by the kernels
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if t.numel() != numel:
            raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
        if t.device != self.device and not (t.is_cuda and self.device.index is None):
            raise ValueError(f"{name} is on {t.device}, the session on {self.device}")

    def dispatch(self, x, topk_ids, stream=None):
        R, T, H, k = self.R, self.T, self.H, self.k
        self._check_tensor("x", x, self.torch_dtype, R * T * H)
        self._check_tensor("topk_ids", topk_ids, torch.int32, R * T * k)
        a2av_dispatch(self.handle, x, topk_ids, self.recv, self.split, self.recv_counts, self.recv_offsets,
                      self.status, stream)
        return self.recv

    def expert(self, inp, out, mode, stream=None):
        n = self.R * self.cap * self.H
        self._check_tensor("expert input", inp, self.torch_dtype, n)
        self._check_tensor("expert output", out, self.torch_dtype, n)
        a2av_expert_apply(self.handle, inp, out, mode, stream)
        return out

    def combine(self, expert_out, gates, y, stream=None):
        R, T, H, k = self.R, self.T, self.H, self.k
        self._check_tensor("expert_out", expert_out, self.torch_dtype, R * self.cap * H)
        self._check_tensor("gates", gates, torch.float32, R * T * k)
        self._check_tensor("y", y, self.torch_dtype, R * T * H)
        a2av_combine(self.handle, expert_out, gates, y, self.status, stream)
        return y

    def positions(self):
        pos = torch.empty((self.R, self.T, self.k), dtype=torch.int32, device=self.device)
        a2av_copy_positions(self.handle, pos)
        return pos

    def recv_expert_offsets(self):
        out = torch.empty((self.R, self.epr + 1), dtype=torch.int32, device=self.device)
        a2av_copy_recv_expert_offsets(self.handle, out)
        return out

    def send_offsets(self):
        so = torch.empty((self.R, self.R + 1), dtype=torch.int32, device=self.device)
        a2av_copy_send_offsets(self.handle, so)
        return so

    def close(self):
        if self.handle is not None:
            torch.cuda.synchronize(self.device)
            a2av_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
