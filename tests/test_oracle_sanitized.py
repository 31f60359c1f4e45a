"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The oracle source is built a second time with both sanitizers, every finding fatal
(oracle/build.py), and the pin suite, the property-based pins and the golden test run
in a child process that has the sanitizer runtime preloaded and loads that build.  A
second child passes the
sanitized oracle a receive buffer one row short and must be stopped by the sanitizer,
which shows the checking layer is live.  Checking communication logic on CPUs before
it meets the hardware follows abhik.ai "Collective Communication for 100k+ GPUs",
section "Testing without the GPUs".
"""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_env():
    try:
        oracle_build.build(sanitize=True)
        runtime = oracle_build.sanitizer_runtime()
    except (OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("gcc has no AddressSanitizer runtime")
    env = dict(os.environ, LD_PRELOAD=runtime, A2AV_ORACLE_SANITIZED="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87",
               HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    return env


def test_sanitized_oracle_is_the_one_loaded(sanitized_env):
    code = ("import oracle; oracle._load(); p = oracle.library_path(); "
            "assert p.endswith('liba2av_oracle_san.so'), p; "
            "assert p in open('/proc/self/maps').read(); print('loaded', p)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized_env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]


def test_oracle_pins_pass_under_address_and_undefined_behaviour_sanitizers(sanitized_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_properties.py",
                        "tests/test_golden.py"],
                       cwd=ROOT, env=sanitized_env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "failed" not in r.stdout


def test_sanitizer_stops_an_out_of_bounds_write(sanitized_env):
    # the oracle writes a whole receive row past the end of a buffer one row too small
    code = """
import numpy as np
import oracle
R, T, k, epr, row = 2, 4, 1, 1, 64
ids = np.ones((R, T, k), np.int32)             # every row to the last rank: it receives R*T rows
x = np.zeros((R, T, row), np.uint8)
cap = R * T
out = oracle.alloc_dispatch(R, T, k, row, epr, cap)
recv = np.zeros(R * cap * row - row, np.uint8)  # the [R][cap][row] buffer, one row short
L = oracle._load()
st = np.zeros(1, np.uint32)
P = oracle._p
L.oracle_dispatch(R, T, k, epr, row, cap, 0, P(x), P(ids), P(out["cnt"]), P(out["send_off"]), P(out["pos"]),
                  P(out["send"]), P(out["recv_counts"]), P(out["recv_off"]), P(out["recv_eoff"]), P(recv), P(st))
print("not stopped")
"""
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized_env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 86, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
    assert "AddressSanitizer" in r.stderr and "not stopped" not in r.stdout
