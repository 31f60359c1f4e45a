"""Host-side logic of bench.py (no GPU): the algorithmic byte counts every bandwidth
figure divides by, the one-GPU guard, and the profile summaries read from rocprofv3
databases."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

import bench
from moe_alltoallv_resident_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (2N + 6A) rows staged and 2(N + A) rows direct, N = R*T tokens, A = N*k assignments,
# worked out by hand from each workload's shape
BYTES = {
    # name: (N, A, row bytes)
    "tiny": (256, 512, 512),
    "decode": (1024, 1024, 10240),
    "prefill": (65536, 65536, 10240),
    "wide": (32768, 262144, 14336),
    "edge": (1024, 2048, 4096),
}


@pytest.mark.parametrize("name", sorted(BYTES))
def test_step_bytes_are_the_real_rows_moved(name):
    N, A, row = BYTES[name]
    w = W.workload(name)
    assert (w.tokens, w.assignments, w.row_bytes) == (N, A, row)
    assert bench.step_bytes(w, False) == (2 * N + 6 * A) * row
    assert bench.step_bytes(w, True) == 2 * (N + A) * row


def test_step_bytes_at_the_prefill_and_wide_shapes():
    # the figures quoted next to the measurements: 5.369 GB / 2.684 GB at prefill,
    # 23.488 GB / 8.456 GB at the wide shape
    assert bench.step_bytes(W.workload("prefill"), False) == 5_368_709_120
    assert bench.step_bytes(W.workload("prefill"), True) == 2_684_354_560
    assert bench.step_bytes(W.workload("wide"), False) == 23_488_102_400
    assert bench.step_bytes(W.workload("wide"), True) == 8_455_716_864


def test_stage_bytes_sum_to_the_step_rows():
    for name in BYTES:
        w = W.workload(name)
        N, A, row = BYTES[name]
        staged = bench.stage_bytes(w, False)
        rows = staged["pack"] + staged["exchange"] + staged["return"] + staged["combine"]
        assert rows - A * (4 + 8) == bench.step_bytes(w, False)
        direct = bench.stage_bytes(w, True)
        assert direct["pack"] + direct["combine"] - A * (12 + 12) == bench.step_bytes(w, True)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _fake_db(path):
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, grid_x int, workgroup_x int, duration int)")
    c.executemany("insert into kernels values (?, ?, ?, ?)", [
        ("void a2av::(anonymous namespace)::pack_kernel<unsigned int __vector(4), 16, true, false>(int)",
         4194816, 256, 240000),
        ("void a2av::(anonymous namespace)::pack_kernel<unsigned int __vector(4), 16, true, false>(int)",
         4194816, 256, 260000),
        ("void a2av::(anonymous namespace)::plan_kernel<8>(int)", 8192, 1024, 12000),
    ])
    c.execute("create table counters_collection (kernel_name text, grid_size_x int, counter_name text, value real)")
    c.executemany("insert into counters_collection values (?, ?, ?, ?)", [
        ("void a2av::(anonymous namespace)::pack_kernel<unsigned int __vector(4), 16, true, false>(int)",
         4194816, "FETCH_SIZE", 100.0),
        ("void a2av::(anonymous namespace)::pack_kernel<unsigned int __vector(4), 16, true, false>(int)",
         4194816, "FETCH_SIZE", 300.0),
    ])
    c.execute("create table regions (category text, name text)")
    c.executemany("insert into regions values (?, ?)", [("HIP_RUNTIME_API", "hipGraphLaunch")] * 3 +
                  [("HIP_RUNTIME_API", "hipGetDevice")] * 2 + [("MARKER", "other")])
    c.commit()
    c.close()


def test_profile_summary_averages_durations_and_counters(tmp_path, capsys):
    db = str(tmp_path / "k_results.db")
    _fake_db(db)
    bench.profile_summary([db])
    out = capsys.readouterr().out
    pack = next(ln for ln in out.splitlines() if ln.startswith("| pack_kernel<u32x4, 16, true, false>"))
    cells = [c.strip() for c in pack.strip("|").split("|")]
    # kernel, grid, block, launches, avg, min, max (us), avg FETCH_SIZE
    assert cells[1:] == ["4194816", "256", "2", "250.00", "240.00", "260.00", "200.0"]
    assert any(ln.startswith("| plan_kernel<8> | 8192 | 1024 | 1 | 12.00") for ln in out.splitlines())


def test_api_summary_counts_hip_calls_only(tmp_path, capsys):
    db = str(tmp_path / "a_results.db")
    _fake_db(db)
    bench.api_summary([db])
    out = capsys.readouterr().out
    assert "| hipGraphLaunch | 3 |" in out and "| hipGetDevice | 2 |" in out
    assert "other" not in out


def test_stage_read_write_split_sums_to_stage_bytes():
    for name in BYTES:
        w = W.workload(name)
        for direct in (False, True):
            total, rw = bench.stage_bytes(w, direct), bench.stage_rw_bytes(w, direct)
            for st, (r, wr) in rw.items():
                assert r + wr == total[st], (name, direct, st)


def test_mix_ceiling():
    # pure streams reach their own rate; an even mix the harmonic mean; more writes, lower
    assert bench.mix_ceiling(10, 0, 7000.0, 5000.0) == 7000.0
    assert bench.mix_ceiling(0, 10, 7000.0, 5000.0) == 5000.0
    assert abs(bench.mix_ceiling(5, 5, 7000.0, 5000.0) - 2 / (1 / 7000.0 + 1 / 5000.0)) < 1e-9
    assert bench.mix_ceiling(1, 8, 7000.0, 5000.0) < bench.mix_ceiling(8, 1, 7000.0, 5000.0)


def _counter_db(path, counter, rows):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, grid_size_x int, counter_name text, value real)")
    c.executemany("insert into counters_collection values (?, ?, ?, ?)",
                  [(name, gx, counter, v) for name, gx, v in rows])
    c.commit()
    c.close()


_NS = "void a2av::(anonymous namespace)::"
_COPY = "__amd_rocclr_copyBuffer(int)"


def test_traffic_json_scales_by_the_copy_and_keeps_each_layout(tmp_path, capsys):
    w = W.workload("tiny")
    copy = w.assignments * w.row_bytes                    # bytes each way of the calibration copy
    out = str(tmp_path / "traffic.json")
    # the copy's FETCH_SIZE reads half its bytes (reads x2), WRITE_SIZE all of them (x1)
    src = [(_COPY, 64, copy / 2048.0), (_COPY, 32, 1.0),  # the largest copy is the calibration
           (_NS + "pack_gather_kernel<unsigned int __vector(4), 1, false, false, 4>(int)", 4096, 10.0),
           (_NS + "pack_gather_kernel<unsigned int __vector(4), 1, false, true, 4>(int)", 4096, 20.0),
           (_NS + "exchange_recv_order_kernel<unsigned int __vector(4), 1, false, 4>(int)", 2048, 30.0),
           (_NS + "exchange_kernel<unsigned int __vector(4), 1, false, true, false, 4>(int)", 2048, 40.0),
           (_NS + "combine_kernel<16, 0, 1, false, false, false, 4>(int)", 1024, 50.0),
           (_NS + "combine_kernel<16, 0, 1, false, true, false, 4>(int)", 1024, 60.0),
           (_NS + "plan_kernel<1>(int)", 4096, 70.0)]
    fetch, write = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _counter_db(fetch, "FETCH_SIZE", src)
    _counter_db(write, "WRITE_SIZE", [(n, g, v * 2 if n.startswith(_COPY) else v) for n, g, v in src])
    bench.traffic_json("tiny", fetch, write, "staged,direct", out_path=out)
    rec = json.load(open(out))
    per = rec["workloads"]["tiny"]["per_launch_bytes"]
    assert sorted(per) == ["direct", "staged"]
    assert sorted(per["staged"]) == ["combine", "exchange", "pack", "return"]
    assert sorted(per["direct"]) == ["combine", "pack"]
    assert per["staged"]["pack"]["read"] == 2 * 10 * 1024 and per["staged"]["pack"]["write"] == 10 * 1024
    assert per["direct"]["combine"]["read"] == 2 * 60 * 1024
    assert per["staged"]["return"]["write"] == 40 * 1024
    cal = rec["workloads"]["tiny"]["calibration"]
    assert cal["read_factor"] == 2.0 and cal["write_factor"] == 1.0
    # an expert-major pass lands beside the source-major figures, not over them
    _counter_db(str(tmp_path / "f2.db"), "FETCH_SIZE", src[:2] + [src[3], src[7]])
    _counter_db(str(tmp_path / "w2.db"), "WRITE_SIZE", [(n, g, v * 2 if n.startswith(_COPY) else v)
                                                        for n, g, v in src[:2] + [src[3], src[7]]])
    bench.traffic_json("tiny", str(tmp_path / "f2.db"), str(tmp_path / "w2.db"), "direct-expert-major",
                       out_path=out)
    rec = json.load(open(out))
    per = rec["workloads"]["tiny"]["per_launch_bytes"]
    assert sorted(per) == ["direct", "direct-expert-major", "staged"]
    assert per["direct-expert-major"]["pack"]["read"] == 2 * 20 * 1024
    assert per["direct"]["combine"]["read"] == 2 * 60 * 1024
    assert "calibration_expert_major" in rec["workloads"]["tiny"]
    # one layout per pass: both at once cannot be told apart
    with pytest.raises(RuntimeError):
        bench.traffic_json("tiny", fetch, write, "direct,direct-expert-major", out_path=out)
    capsys.readouterr()
