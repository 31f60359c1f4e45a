"""The C-ABI library loads and exports every entry point include/a2av.h declares; host-only
calls (no GPU work) behave as documented.  Runs without a GPU."""
import ctypes
import os
import re

import pytest

from moe_alltoallv_resident_amd import a2av

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "a2av.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(a2av_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for required in ("a2av_create", "a2av_dispatch", "a2av_combine", "a2av_destroy"):
        assert required in names
    assert set(names) == set(a2av.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = a2av.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_debug_library_exports_the_same_symbols():
    """liba2av_debug.so (A2AV_DEBUG=1: device-side bounds checks) is built beside the
    release library and exports every declared entry point too."""
    from moe_alltoallv_resident_amd import build as lib_build
    dbg = ctypes.CDLL(lib_build.DEBUG_LIB)
    for name in declared_functions():
        assert ctypes.cast(getattr(dbg, name), ctypes.c_void_p).value, name
    assert a2av.ST_BOUNDS == 4
    header = open(HEADER).read()
    assert re.search(r"#define A2AV_ST_BOUNDS\s+4u", header)


def test_environment_selects_the_debug_library():
    """A2AV_DEBUG=1 makes the binding load liba2av_debug.so (checked in a child process,
    where the variable is set before the binding is imported)."""
    import subprocess
    import sys
    code = ("from moe_alltoallv_resident_amd import a2av; import os; "
            "print(os.path.basename(a2av.LIB_PATH), os.path.basename(a2av.lib()._name))")
    for value, want in (("1", "liba2av_debug.so"), ("0", "liba2av.so")):
        env = dict(os.environ, A2AV_DEBUG=value)
        out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                             timeout=120, check=True).stdout.split()
        assert out == [want, want], (value, out)


def test_error_strings():
    assert a2av.error_string(a2av.OK) == "ok"
    assert "invalid" in a2av.error_string(a2av.ERR_INVALID)
    assert "unknown" in a2av.error_string(12345)


@pytest.mark.parametrize("bad", [
    dict(num_ranks=0), dict(num_ranks=2000), dict(tokens_per_rank=-1), dict(hidden=0), dict(dtype=7),
    dict(experts_per_rank=0), dict(experts_per_rank=513), dict(top_k=0), dict(top_k=65),
    dict(num_ranks=2, experts_per_rank=1, top_k=3), dict(recv_capacity_rows=-5), dict(path=2), dict(recv_layout=2),
])
def test_workspace_bytes_rejects_invalid_configs(bad):
    base = dict(num_ranks=8, tokens_per_rank=128, hidden=5120, dtype=a2av.BF16, experts_per_rank=16, top_k=1)
    base.update(bad)
    assert a2av.a2av_workspace_bytes(a2av.make_config(**base)) == -1


def test_workspace_bytes_counts_send_buffer_and_tables():
    R, T, H, epr, k = 8, 8192, 5120, 16, 1
    n = a2av.a2av_workspace_bytes(a2av.make_config(R, T, H, a2av.BF16, epr, k))
    send = R * T * k * H * 2
    assert send < n < send + 4 * 1024 * 1024
    # the direct path has no send buffer
    nd = a2av.a2av_workspace_bytes(a2av.make_config(R, T, H, a2av.BF16, epr, k, path=a2av.PATH_DIRECT))
    assert 0 < nd < 4 * 1024 * 1024


def test_noalloc_collective_rejects_on_the_host():
    """a2av_alltoallv_noalloc checks its shape before touching the GPU: an invalid
    configuration or a missing counts pointer is A2AV_ERR_INVALID, more ranks than its
    scratch array holds is A2AV_ERR_SCRATCH (pointers below are never dereferenced)."""
    L = a2av.lib()
    fake = ctypes.c_void_p(4096)
    ok = dict(num_ranks=8, tokens_per_rank=4, hidden=64, dtype=a2av.BF16, experts_per_rank=1, top_k=1)
    big = a2av.make_config(**dict(ok, num_ranks=a2av.NOALLOC_MAX_RANKS + 1))
    assert L.a2av_alltoallv_noalloc(ctypes.byref(big), fake, fake, fake, None, None, fake, None) == a2av.ERR_SCRATCH
    bad = a2av.make_config(**dict(ok, hidden=0))
    assert L.a2av_alltoallv_noalloc(ctypes.byref(bad), fake, fake, fake, None, None, fake, None) == a2av.ERR_INVALID
    good = a2av.make_config(**ok)
    assert L.a2av_alltoallv_noalloc(ctypes.byref(good), fake, None, fake, None, None, fake, None) == a2av.ERR_INVALID
    assert L.a2av_alltoallv_noalloc(None, fake, fake, fake, None, None, fake, None) == a2av.ERR_INVALID
    assert "scratch" in a2av.error_string(a2av.ERR_SCRATCH)


def test_stream_reference_rejects_on_the_host():
    L = a2av.lib()
    fake = ctypes.c_void_p(4096)
    assert L.a2av_stream_reference(fake, fake, 24, a2av.STREAM_READ, None) == a2av.ERR_INVALID     # not 16-byte units
    assert L.a2av_stream_reference(fake, fake, 32, 7, None) == a2av.ERR_INVALID                    # no such mode
    assert L.a2av_stream_reference(fake, None, 32, a2av.STREAM_WRITE, None) == a2av.ERR_INVALID    # no destination
    assert L.a2av_stream_reference(None, fake, 32, a2av.STREAM_READ, None) == a2av.ERR_INVALID     # no source
    assert L.a2av_stream_reference(fake, ctypes.c_void_p(4100), 32, a2av.STREAM_WRITE, None) == a2av.ERR_INVALID
