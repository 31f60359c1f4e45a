"""Dispatch+combine benchmark on one MI355X.

One step = router stand-in output already on the GPU -> dispatch (plan, pack, exchange)
-> expert stand-in (harness, not in the metric) -> combine (return exchange, combine),
over one batch of seeded synthetic input resident in HBM.  The default workload is the
prefill shape: 8 virtual ranks x 8192 tokens, hidden 5120 bf16, 128 experts (16 per
rank), top-1 with Zipf(1.2) expert popularity.

Printed: ONE JSON line.  `value` is the effective HBM bandwidth of dispatch+combine, the
algorithmic bytes of the staged path ((2N + 6A) rows of real tokens) divided by the
dispatch+combine time per step; `us_per_step` is that time: the median over 5 trials of
K back-to-back dispatch+combine pairs / K, with events only around each loop, so launch
gaps count and no event sits between kernels
(`us_per_step_min` is the fastest trial, `us_per_step_kernels` the sum of the library's
per-kernel event times, `stage_us` their breakdown); `ms_per_step` is the same
dispatch+combine time in milliseconds, and `ms_per_step_with_expert_stand_in` a whole
step with the harness expert between dispatch and combine.  `roofline` is for the
slowest kernel of the step, from its per-kernel event time; `cpu_baseline` is the CPU
oracle on the whole workload in a child process pinned to one core; `decode_graph` and
`edge_graph` are the decode and edge shapes captured in hipGraphs and replayed with
routing that changes on the device each step, with dispatch and combine measured
separately next to a reference copy of the same bytes; `graph_kernel_node_us` is what
one nearly empty dependent kernel adds to a replayed graph step (the launch gap); `wide`
is the top-8 shape (16 x 2048 tokens, hidden 7168, 256 experts) timed the same way as
the headline, 10 steps per path, at a receive capacity of twice the mean rows per rank
(32,768) and at the worst case (262,144 rows per rank, 60 GB), each path with its own
roofline entry.
"""
import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha256():
    """Hash of the kernels' source (kernels and the shared layout header)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("a2av_kernels.hip", "a2av_internal.h"):
        with open(os.path.join(ROOT, "moe_alltoallv_resident_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, path, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter passes
    (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a copy kernel of
    known size), or None when the kernels' source changed since the counters were taken
    or no counters exist for this workload and kernel."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f)
        sha = kernel_source_sha256()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    b = rec.get("workloads", {}).get(workload, {}).get("per_launch_bytes", {}).get(path, {}).get(kernel)
    return None if b is None else int(b["read"] + b["write"])


def step_bytes(w, direct):
    """Algorithmic HBM bytes of one dispatch+combine over real rows.  Staged: pack reads
    N rows and writes A, the exchange reads and writes A, the return reads and writes A,
    the combine reads A and writes N: (2N + 6A) rows.  Direct: pack reads N and writes A
    into the receivers' buffers, the combine reads A and writes N: 2(N + A) rows."""
    N, A, row = w.tokens, w.assignments, w.row_bytes
    return (2 * (N + A) if direct else 2 * N + 6 * A) * row


def stage_bytes(w, direct):
    """Algorithmic bytes per launch of each stage (real rows only).  Index bytes: planning
    reads the ids and writes every place (and, top-1, the inverse: which token sits at
    each send place); pack reads each assignment's place or its inverse (4 B) and, on the
    direct path, records its receive row (8 B); the combine reads each gate (4 B) and the
    place (4 B) or receive row (8 B)."""
    N, A, row = w.tokens, w.assignments, w.row_bytes
    return {
        "plan": A * 4 + 4 * (w.num_ranks * w.num_experts + w.num_ranks * (w.num_ranks + 1)) + A * 4
                + (A * 4 if w.top_k == 1 else 0),
        "pack": (N + A) * row + A * (12 if direct else 4),
        "exchange": 2 * A * row,
        "return": 2 * A * row,
        "combine": (A + N) * row + A * (12 if direct else 8),
    }


def stage_rw_bytes(w, direct):
    """(read, written) algorithmic bytes per launch of each row stage (stage_bytes split by
    direction)."""
    N, A, row = w.tokens, w.assignments, w.row_bytes
    return {
        "pack": (N * row + A * 4, A * row + (A * 8 if direct else 0)),
        "exchange": (A * row, A * row),
        "return": (A * row, A * row),
        "combine": (A * row + A * (12 if direct else 8), N * row),
    }


def mix_ceiling(read, written, read_gbps, write_gbps):
    """The fastest a kernel moving `read` + `written` bytes can go when reads alone stream
    at read_gbps and writes alone at write_gbps."""
    return (read + written) / (read / read_gbps + written / write_gbps)


def annotate_ceilings(m, w, direct, read_gbps, write_gbps):
    """Adds each row stage's mixed read/write ceiling and the fraction of it reached to a
    time_path result (and to its roofline entry)."""
    rw = stage_rw_bytes(w, direct)
    fr = {}
    for st, us in m["stage_us"].items():
        if st not in rw:
            continue
        achieved = (rw[st][0] + rw[st][1]) / (us * 1e-6) / 1e9
        fr[st] = round(achieved / mix_ceiling(rw[st][0], rw[st][1], read_gbps, write_gbps), 4)
    m["stage_frac_of_mix_ceiling"] = fr
    k = m["roofline"]["kernel"]
    if k in rw:
        m["roofline"]["mix_ceiling_GBps"] = round(mix_ceiling(rw[k][0], rw[k][1], read_gbps, write_gbps), 1)
        m["roofline"]["frac_of_mix_ceiling"] = fr[k]


def stream_ceilings(torch, a2av, nbytes, timed):
    """Read-only and write-only stream bandwidth over nbytes (GB/s)."""
    buf = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    out = torch.empty(a2av.STREAM_READ_OUT_BYTES // 4, dtype=torch.int32, device="cuda")
    r = nbytes / (timed(lambda: a2av.a2av_stream_reference(buf, out, nbytes, a2av.STREAM_READ)) * 1e-3) / 1e9
    wr = nbytes / (timed(lambda: a2av.a2av_stream_reference(None, buf, nbytes, a2av.STREAM_WRITE)) * 1e-3) / 1e9
    del buf, out
    return round(r, 1), round(wr, 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--recv-capacity", type=int, default=0, metavar="ROWS",
                    help="receive capacity per rank for the headline workload (0: the workload's own); "
                         "for counter passes at another capacity")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-graph", action="store_true")
    ap.add_argument("--no-wide", action="store_true",
                    help="skip the top-8 wide shape (16 x 2048 tokens, hidden 7168) timed after the headline")
    ap.add_argument("--cpu-baseline-child", metavar="WORKLOAD",
                    help=argparse.SUPPRESS)   # the pinned CPU oracle run (a child of this script)
    ap.add_argument("--cpu-core", type=int, default=0, help=argparse.SUPPRESS)
    ap.add_argument("--traffic-json", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="turn rocprofv3 FETCH_SIZE and WRITE_SIZE databases of a run with --workload W "
                         "--paths P (staged,direct or direct-expert-major; give the same --paths here) into "
                         "per-launch bytes and merge them into profiles/hbm_traffic.json under W (no GPU)")
    ap.add_argument("--paths", default="staged,direct,direct-expert-major",
                    help="paths to time (staged, direct, staged-expert-major, direct-expert-major); "
                         "the first one gives the headline value")
    ap.add_argument("--profile-summary", nargs="+", metavar="DB",
                    help="print per-kernel statistics of rocprofv3 database(s) and exit (no GPU)")
    ap.add_argument("--api-summary", nargs="+", metavar="DB",
                    help="print HIP API call counts of rocprofv3 database(s) and exit (no GPU)")
    ap.add_argument("--decode-graph-only", type=int, metavar="REPLAYS", default=0,
                    help="only capture the decode step and replay it REPLAYS times (for API tracing)")
    args = ap.parse_args()
    if args.cpu_baseline_child:
        cpu_baseline_child(args.cpu_baseline_child, args.cpu_core)
        return
    if args.traffic_json:
        traffic_json(args.workload, *args.traffic_json, paths=args.paths)
        return
    if args.profile_summary:
        profile_summary(args.profile_summary)
        return
    if args.api_summary:
        api_summary(args.api_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the R virtual ranks live in one GPU's HBM and no "
              f"collective crosses GPUs, so --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_alltoallv_resident_amd import a2av
    from moe_alltoallv_resident_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    paths = [p.strip() for p in args.paths.split(",") if p.strip()]
    if args.decode_graph_only:
        print(json.dumps(decode_graph(np, torch, a2av, W, paths[0], replays=args.decode_graph_only)), flush=True)
        return
    w = W.workload(args.workload, **({"recv_capacity_rows": args.recv_capacity} if args.recv_capacity else {}))
    log(f"workload {w.describe()}; generating inputs")
    x, ids, gates = W.make_inputs(w)
    if w.dtype == W.BF16:
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        xt = torch.from_numpy(x).cuda()
    idt = torch.from_numpy(ids).cuda()
    gt = torch.from_numpy(gates).cuda()

    measured = {p: time_path(torch, a2av, w, xt, idt, gt, p, args.steps, args.warmup) for p in paths}
    head = measured[paths[0]]

    # achievable references for one stage's bytes (read + write): torch's device copy and
    # the library's reference row copy (the path's own row movement, identity mapping)
    ref_elems = w.assignments * w.row_bytes // 2
    src = torch.empty(ref_elems, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    copy_gbps = 2 * ref_elems * 2 / (timed(lambda: dst.copy_(src)) * 1e-3) / 1e9
    row_copy_gbps = 2 * ref_elems * 2 / (timed(lambda: a2av.a2av_copy_reference(src, dst, w.assignments, w.row_bytes))
                                         * 1e-3) / 1e9
    del src, dst
    read_gbps, write_gbps = stream_ceilings(torch, a2av, w.assignments * w.row_bytes, timed)
    for p in paths:
        annotate_ceilings(measured[p], w, path_config(a2av, p)[0] == a2av.PATH_DIRECT, read_gbps, write_gbps)

    result = {
        "metric": "dispatch+combine µs/step and effective HBM GB/s (% of peak), 1 MI355X",
        "value": head["GBps"],
        "unit": "GB/s",
        "us_per_step": head["us_per_step"],
        "us_per_step_min": head["us_per_step_min"],
        "us_per_step_kernels": head["us_per_step_kernels"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 4),
        "ms_per_step_with_expert_stand_in": head["ms_per_step_full"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded numpy; no model weights or traces)",
        "config": {
            "workload": w.describe(),
            "virtual_ranks": w.num_ranks, "tokens_per_rank": w.tokens_per_rank, "hidden": w.hidden,
            "experts": w.num_experts, "top_k": w.top_k, "path": paths[0],
            "algorithmic_bytes_per_step": head["bytes_per_step"],
        },
        "stage_us": head["stage_us"],
        "stage_frac_of_mix_ceiling": head["stage_frac_of_mix_ceiling"],
        "roofline": dict(head["roofline"], copy_reference_GBps=round(copy_gbps, 1),
                         row_copy_reference_GBps=round(row_copy_gbps, 1),
                         frac_of_row_copy=round(head["roofline"]["achieved"] / row_copy_gbps, 4),
                         read_stream_GBps=read_gbps, write_stream_GBps=write_gbps),
    }
    for p in paths[1:]:
        result[f"{p.replace('-', '_')}_path"] = {k: v for k, v in measured[p].items()
                                                 if k not in ("ms_per_step_wall", "ms_per_step_full")}
    del xt
    torch.cuda.empty_cache()

    if not args.no_wide and w.name != "wide":
        ww = W.workload("wide")
        log(f"workload {ww.describe()}; generating inputs")
        xw, idw, gw = W.make_inputs(ww)
        xwt = torch.from_numpy(xw.view(np.int16)).view(torch.bfloat16).cuda()
        idwt, gwt = torch.from_numpy(idw).cuda(), torch.from_numpy(gw).cuda()
        worst = ww.num_ranks * ww.tokens_per_rank * min(ww.top_k, ww.experts_per_rank)
        wide = {"workload": ww.describe(), "steps": 10, "warmup": 3}
        wide["read_stream_GBps"], wide["write_stream_GBps"] = stream_ceilings(
            torch, a2av, ww.assignments * ww.row_bytes, timed)
        for label, cap in (("capacity_2x_mean", ww.capacity), ("capacity_worst_case", worst)):
            runs = {}
            for p in paths:
                m = time_path(torch, a2av, ww, xwt, idwt, gwt, p, 10, 3, cap=cap)
                annotate_ceilings(m, ww, path_config(a2av, p)[0] == a2av.PATH_DIRECT, wide["read_stream_GBps"],
                                  wide["write_stream_GBps"])
                runs[p] = {k: m[k] for k in ("us_per_step", "us_per_step_min", "GBps", "pct_hbm_peak",
                                             "bytes_per_step", "stage_us", "stage_frac_of_mix_ceiling", "roofline")}
            wide[label] = {"recv_capacity_rows_per_rank": cap,
                           "recv_bytes": ww.num_ranks * cap * ww.row_bytes, "paths": runs}
        # the identity row copy of A rows of this shape, the achievable figure its kernels
        # are compared with (as at the headline shape)
        wsrc = torch.empty(ww.assignments * ww.row_bytes // 2, dtype=torch.int16, device="cuda")
        wdst = torch.empty_like(wsrc)
        wide["row_copy_reference_GBps"] = round(2 * ww.assignments * ww.row_bytes / (timed(
            lambda: a2av.a2av_copy_reference(wsrc, wdst, ww.assignments, ww.row_bytes)) * 1e-3) / 1e9, 1)
        del wsrc, wdst
        result["wide"] = wide
        del xwt, idwt, gwt
        torch.cuda.empty_cache()

    if not args.no_decode_graph:
        result["graph_kernel_node_us"] = graph_kernel_node_us(torch, a2av)
        result["decode_graph"] = {p: decode_graph(np, torch, a2av, W, p) for p in paths}
        result["edge_graph"] = {p: decode_graph(np, torch, a2av, W, p, workload="edge") for p in paths}
        # decode latency against batch size: tokens per rank from 16 to 1024 at the decode
        # shape, zero-copy path (the one-launch dispatch up to 512 tokens per rank here)
        sweep_path = "direct" if "direct" in paths else paths[0]
        result["decode_sweep"] = {"path": sweep_path, "workload": W.workload("decode").describe(), "points": [
            decode_graph(np, torch, a2av, W, sweep_path, steps=50, over={"tokens_per_rank": t}, light=True)
            for t in (16, 32, 64, 128, 256, 384, 512, 768, 1024)]}
        # the same for the top-8 shape (16 ranks, 14 KiB rows, 256 experts) at decode batch sizes
        result["decode_sweep_top8"] = {"path": sweep_path, "workload": W.workload("wide").describe(), "points": [
            decode_graph(np, torch, a2av, W, sweep_path, workload="wide", steps=50, over={"tokens_per_rank": t},
                         light=True)
            for t in (4, 8, 16, 32, 64, 128)]}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)

    print(json.dumps(result), flush=True)


def path_config(a2av, name):
    """'staged' | 'direct', optionally with '-expert-major': (path, receive layout)."""
    path = a2av.PATH_DIRECT if name.startswith("direct") else a2av.PATH_STAGED
    layout = a2av.LAYOUT_EXPERT_MAJOR if name.endswith("expert-major") else a2av.LAYOUT_SOURCE_MAJOR
    return path, layout


def time_path(torch, a2av, w, xt, idt, gt, name, steps, warmup, trials=5, cap=None):
    """One path: warm-up; `steps` steps with HIP events recorded between the library's
    kernels (on the stream they run on) for the per-kernel breakdown and the roofline;
    then `trials` end-to-end runs with events only around the whole loop: `steps`
    dispatch+combine pairs (the headline: median trial, launch gaps included, no event
    between kernels; the minimum beside it), and `steps` full steps with the expert
    stand-in between them.  `cap` overrides the workload's receive capacity."""
    from moe_alltoallv_resident_amd import workloads as W
    path_id, layout = path_config(a2av, name)
    direct = path_id == a2av.PATH_DIRECT
    path = name
    at_own_capacity = (w.capacity if cap is None else cap) == W.workload(w.name).capacity
    s = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k,
                     w.recv_capacity_rows if cap is None else cap, path=path_id, recv_layout=layout)
    y = torch.empty_like(xt)

    def step():
        s.dispatch(xt, idt)
        s.expert(s.recv, s.recv, w.expert_mode)
        s.combine(s.recv, gt, y)

    def dispatch_combine():
        s.dispatch(xt, idt)
        s.combine(s.recv, gt, y)

    def loop_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    log(f"{path}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"{path}: timing {steps} steps")
    a2av.a2av_timing_begin(s.handle, steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_sum, launches = a2av.a2av_timing_end(s.handle)
    full_ms, dc_trials = [], []
    for _ in range(trials):
        full_ms.append(loop_ms(step))
        dc_trials.append(loop_ms(dispatch_combine))
    status = int(s.status.item())
    if status != 0:
        raise RuntimeError(f"device status {status} during the benchmark")
    full_ms.sort()
    dc_trials.sort()
    dc_ms = dc_trials[len(dc_trials) // 2]
    # per step (a stage may launch more than one kernel), and per launch
    stage_ms = {n: ms_sum[i] / steps for i, n in enumerate(a2av.STAGE_NAMES) if launches[i]}
    launch_ms = {n: ms_sum[i] / launches[i] for i, n in enumerate(a2av.STAGE_NAMES) if launches[i]}
    nbytes = step_bytes(w, direct)
    gbps = nbytes / (dc_ms * 1e-3) / 1e9
    sb = stage_bytes(w, direct)
    dom = max((n for n in launch_ms if n != "plan"), key=lambda n: launch_ms[n])
    dom_gbps = sb[dom] / (launch_ms[dom] * 1e-3) / 1e9
    log(f"{path}: dispatch+combine {dc_ms * 1e3:.1f} us per step (median of {trials}); stages (us/launch): "
        + ", ".join(f"{n} {v * 1e3:.1f}" for n, v in stage_ms.items()))
    s.close()
    del y, s
    torch.cuda.empty_cache()
    return {
        "GBps": round(gbps, 1),
        "us_per_step": round(dc_ms * 1e3, 2),
        "us_per_step_min": round(dc_trials[0] * 1e3, 2),
        "us_per_step_kernels": round(sum(stage_ms.values()) * 1e3, 2),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "ms_per_step_full": round(full_ms[len(full_ms) // 2], 4),
        "ms_per_step_wall": round(wall / steps * 1e3, 4),
        "bytes_per_step": nbytes,
        "stage_us": {n: round(v * 1e3, 2) for n, v in stage_ms.items()},
        "roofline": {
            "bound": "hbm", "kernel": dom, "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            # the counter passes run at the workload's own receive capacity
            "traffic": measured_traffic(w.name, path, dom) if at_own_capacity else None,
            "bytes_per_launch": sb[dom],
            "us_per_launch": round(launch_ms[dom] * 1e3, 2),
        },
    }


def decode_graph(np, torch, a2av, W, path, workload="decode", steps=100, per_graph=10, replays=None, over=None,
                 light=False):
    """A latency-bound shape captured in hipGraphs and replayed with routing that changes
    on the device every step (router stand-in -> dispatch -> expert stand-in -> combine),
    one event pair around all replays and no host synchronisation between them.

    Each graph holds `per_graph` consecutive steps, so the per-step time is GPU time and
    not the host's graph-launch rate (a one-step graph is also timed: that figure
    includes the launch rate).  The dispatch+combine share is the full step minus a graph
    of the router and expert stand-ins alone; the combine therefore reads rows that
    another kernel has just written, as it would after a real expert.  The flushed
    variant writes 512 MiB before every step, so each step starts with its inputs out of
    the 256 MiB last-level cache.  With `replays`, only the one-step graph is captured
    and replayed that many times (for API tracing).  `over` replaces workload fields;
    `light` keeps only the dispatch, combine and reference-copy figures."""
    w = W.workload(workload, **(over or {}))
    log(f"graph latency ({path}): {w.describe()}, {steps} steps")
    x = W.make_x(w)
    n = w.tokens * w.top_k
    ids_table = torch.from_numpy(np.stack([W.make_ids(w, i).reshape(n) for i in range(steps)])).cuda()
    gates_table = torch.from_numpy(np.stack([W.make_gates(w, i).reshape(n) for i in range(steps)])).cuda()
    xt = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if w.dtype == W.BF16
          else torch.from_numpy(x)).cuda()
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids = torch.empty((w.num_ranks, w.tokens_per_rank, w.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((w.num_ranks, w.tokens_per_rank, w.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty_like(xt)
    path_id, layout = path_config(a2av, path)
    s = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k,
                     path=path_id, recv_layout=layout)
    flush_buf = None

    def route():
        a2av.a2av_route_step(ids_table, gates_table, steps, n, counter, ids, gates)

    def full():
        route()
        s.dispatch(xt, ids)
        s.expert(s.recv, s.recv, w.expert_mode)
        s.combine(s.recv, gates, y)

    def harness():
        # the router and expert stand-ins alone (the expert reuses the last routing)
        route()
        s.expert(s.recv, s.recv, w.expert_mode)

    def route_dispatch():
        route()
        s.dispatch(xt, ids)

    def route_dispatch_expert():
        route()
        s.dispatch(xt, ids)
        s.expert(s.recv, s.recv, w.expert_mode)

    # a reference row copy of the bytes one dispatch (or one combine) moves: it reads N
    # rows and writes A (the combine reads A and writes N), so (N + A) / 2 rows each way
    ref_rows = (w.tokens + w.assignments) // 2
    ref_src = torch.empty((ref_rows, w.row_bytes // 2), dtype=torch.int16, device="cuda")
    ref_dst = torch.empty_like(ref_src)

    def reference_copy():
        a2av.a2av_copy_reference(ref_src, ref_dst, ref_rows, w.row_bytes)

    def flushed(fn):
        def g():
            flush_buf.fill_(1)
            fn()
        return g

    def capture(fn, count):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(count):
                fn()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        return graph

    def us_per_step(fn, count, total, routed=True):
        """Median over 5 trials of (time of total/count replays) / total."""
        graph = capture(fn, count)
        trials = []
        for _ in range(5):
            counter.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(total // count):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            if routed and int(counter.item()) != total:
                raise RuntimeError("router stand-in did not run once per step")
            trials.append(e0.elapsed_time(e1) * 1e3 / total)
        del graph
        return float(np.median(trials))

    if replays is not None:
        us = us_per_step(full, 1, replays)
        ok = int(s.status.item()) == 0
        s.close()
        return {"workload": w.describe(), "path": path, "replays": replays, "us_per_step": round(us, 2),
                "counter_ok": ok}
    t_full = us_per_step(full, per_graph, steps)
    t_harness = us_per_step(harness, per_graph, steps)
    t_route = us_per_step(route, per_graph, steps)
    t_route_dispatch = us_per_step(route_dispatch, per_graph, steps)
    t_route_dispatch_expert = us_per_step(route_dispatch_expert, per_graph, steps)
    t_copy = us_per_step(reference_copy, per_graph, steps, routed=False)
    if light:
        ok = int(s.status.item()) == 0
        t_dispatch, t_combine = t_route_dispatch - t_route, t_full - t_route_dispatch_expert
        # how many launches the library's dispatch made, from its own stage timing (no
        # planning launch: the one-launch form)
        route()
        a2av.a2av_timing_begin(s.handle, 1)
        s.dispatch(xt, ids)
        _, launches = a2av.a2av_timing_end(s.handle)
        del ref_src, ref_dst
        s.close()
        torch.cuda.empty_cache()
        return {"tokens_per_rank": w.tokens_per_rank, "assignments": w.assignments,
                "one_launch_dispatch": launches[0] == 0,
                "us_dispatch": round(t_dispatch, 2), "us_combine": round(t_combine, 2),
                "us_reference_copy": round(t_copy, 2), "bytes_dispatch": (w.tokens + w.assignments) * w.row_bytes,
                "status_ok": ok}
    t_one = us_per_step(full, 1, steps)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    t_full_f = us_per_step(flushed(full), per_graph, steps)
    t_harness_f = us_per_step(flushed(harness), per_graph, steps)
    ok = int(s.status.item()) == 0
    t_dispatch = t_route_dispatch - t_route
    t_combine = t_full - t_route_dispatch_expert
    direct = path_id == a2av.PATH_DIRECT
    sb = stage_bytes(w, direct)
    out = {"workload": w.describe(), "steps": steps, "steps_per_graph": per_graph,
           "us_per_step_with_expert_and_router": round(t_full, 2),
           "us_router_and_expert_only": round(t_harness, 2),
           "us_dispatch_combine_estimate": round(t_full - t_harness, 2),
           # dispatch: (router, dispatch) minus (router); combine: (router, dispatch, expert,
           # combine) minus (router, dispatch, expert), so the combine reads rows the expert
           # kernel has just written, as after a real expert
           "us_dispatch": round(t_dispatch, 2),
           "us_combine": round(t_combine, 2),
           "us_dispatch_plus_combine": round(t_dispatch + t_combine, 2),
           "reference_copy": {"rows": ref_rows, "bytes": 2 * ref_rows * w.row_bytes, "us": round(t_copy, 2),
                              "dispatch_gap_us": round(t_dispatch - t_copy, 2),
                              "combine_gap_us": round(t_combine - t_copy, 2)},
           "us_per_step_one_step_graphs": round(t_one, 2),
           "flushed_512MiB": {"us_per_step_with_expert_and_router": round(t_full_f, 2),
                              "us_router_and_expert_only": round(t_harness_f, 2),
                              "us_dispatch_combine_estimate": round(t_full_f - t_harness_f, 2)},
           "status_ok": ok,
           "algorithmic_bytes_per_step": step_bytes(w, direct),
           "algorithmic_bytes_dispatch": sb["pack"] + (sb["exchange"] if not direct else 0),
           "algorithmic_bytes_combine": sb["combine"] + (sb["return"] if not direct else 0)}
    log(f"graph latency ({path}, {workload}): dispatch {t_dispatch:.2f} us, combine {t_combine:.2f} us, "
        f"reference copy of the same bytes {t_copy:.2f} us; dispatch+combine {t_full - t_harness:.2f} us warm, "
        f"{t_full_f - t_harness_f:.2f} us flushed")
    del flush_buf, ref_src, ref_dst
    s.close()
    torch.cuda.empty_cache()
    return out


def graph_kernel_node_us(torch, a2av, nodes=8, per_graph=10, replays=20):
    """What one kernel node costs inside a replayed graph when it has nearly nothing to
    do: graphs of `per_graph` steps, each step a chain of 1 or `nodes` launches of the
    router stand-in with no ids to copy; the difference per step over nodes - 1 is the
    launch gap a dependent kernel adds at decode sizes."""
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = torch.zeros(1, dtype=torch.float32, device="cuda")
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")

    def per_step_us(m):
        def step():
            for _ in range(m):
                a2av.a2av_route_step(t, g, 1, 0, counter, t, g)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        trials = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            trials.append(e0.elapsed_time(e1) * 1e3 / (replays * per_graph))
        del graph
        return sorted(trials)[2]

    one, many = per_step_us(1), per_step_us(nodes)
    return round((many - one) / (nodes - 1), 3)


def cpu_baseline(w):
    """The CPU oracle as it stands (single-threaded C, fp64) on the whole workload, run in
    a child process of this script pinned to one core (the first core this process may
    use) so that it cannot touch the GPU or a second core.  Reported as effective GB/s
    over the same staged byte count as the GPU figure."""
    core = min(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle on {w.describe()}, child process pinned to core {core}")
    env = dict(os.environ, OMP_NUM_THREADS="1", HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", w.name,
                        "--cpu-core", str(core)], capture_output=True, text=True, env=env, timeout=900)
    if r.returncode != 0:
        raise RuntimeError(f"cpu baseline child failed ({r.returncode}): {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def cpu_baseline_child(name, core, reps=3):
    """Pinned to `core`: generates the workload, allocates and touches every output of the
    oracle's dispatch, return and combine, then times only those three C calls (the
    expert stand-in runs between them, untimed), median of `reps` steps."""
    os.sched_setaffinity(0, {core})
    import numpy as np

    import oracle
    from moe_alltoallv_resident_amd import workloads as W
    w = W.workload(name)
    x, ids, gates = W.make_inputs(w)
    R, T, H, k, cap = w.num_ranks, w.tokens_per_rank, w.hidden, w.top_k, w.capacity
    rows = oracle.as_rows(x)
    d = oracle.alloc_dispatch(R, T, k, w.row_bytes, w.experts_per_rank, cap)
    ret = np.zeros((R, T * k, w.row_bytes), np.uint8)
    y = np.zeros_like(x)
    for a in list(d.values()) + [ret, y]:
        a.fill(0)                                   # touch every page before timing
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.dispatch(rows, ids, w.experts_per_rank, cap, out=d)
        t1 = time.perf_counter()
        recv = d["recv"].view(x.dtype).reshape(R, cap, H)
        z = oracle.expert(recv, d["cnt"], d["recv_off"], w.experts_per_rank, w.dtype, w.expert_mode)
        t2 = time.perf_counter()
        oracle.return_exchange(oracle.as_rows(z), d["send_off"], d["recv_off"], T, k, out=ret)
        oracle.combine(ret.view(x.dtype).reshape(R, T * k, H), d["pos"], gates, w.dtype, out=y)
        t3 = time.perf_counter()
        times.append((t1 - t0) + (t3 - t2))
        del z, recv
    t = float(np.median(times))
    gbps = step_bytes(w, False) / t / 1e9
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        model = "unknown"
    print(json.dumps({
        "value": round(gbps, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"the whole workload, {w.describe()} ({T} tokens per rank), staged path, median of {reps} "
                  f"steps; timed: the oracle's dispatch, return and combine calls only (outputs allocated and "
                  f"touched beforehand, expert stand-in untimed)",
        "us_per_step": round(t * 1e6, 1), "pinned_core": core,
        "affinity_after_pin": sorted(os.sched_getaffinity(0)),
        "host_cpu": model, "host_threads_available": os.cpu_count()}), flush=True)


def traffic_json(workload, fetch_db, write_db, paths="staged,direct", out_path=None):
    """Per-launch HBM bytes of the path's kernels from a FETCH_SIZE and a WRITE_SIZE pass
    of `bench.py --workload W --paths P`, scaled by what the same counters read for
    torch's device copy of A rows (the largest __amd_rocclr_copyBuffer launch, whose bytes
    are known), merged into profiles/hbm_traffic.json under the workload.  P is
    `staged,direct` or `direct-expert-major`: the kernels of the two layouts are the same
    instances, so each layout needs passes of its own."""
    import sqlite3

    from moe_alltoallv_resident_amd import workloads as W
    w = W.workload(workload)
    copy_bytes = w.assignments * w.row_bytes

    def per_kernel(db, counter):
        c = sqlite3.connect(db)
        vals = {}
        for name, gx, val in c.execute("select kernel_name, grid_size_x, value from counters_collection "
                                       "where counter_name = ?", (counter,)):
            vals.setdefault((_short_kernel_name(name), gx), []).append(val)
        return {key: sum(v) / len(v) for key, v in vals.items()}

    fetch, write = per_kernel(fetch_db, "FETCH_SIZE"), per_kernel(write_db, "WRITE_SIZE")
    copies = [key for key in fetch if key[0] == "__amd_rocclr_copyBuffer"]
    big = max(copies, key=lambda key: fetch[key])
    read_factor = copy_bytes / (fetch[big] * 1024.0)
    write_factor = copy_bytes / (write[big] * 1024.0)
    stage_of = {"plan_kernel": None, "pack_kernel": "pack", "pack_gather_kernel": "pack",
                "exchange_recv_order_kernel": "exchange", "combine_kernel": "combine"}
    names = [p.strip() for p in paths.split(",") if p.strip()]
    expert_major = all(p.endswith("-expert-major") for p in names)
    if not expert_major and any(p.endswith("-expert-major") for p in names):
        raise RuntimeError("take the counters of the source-major and expert-major paths in separate passes")
    suffix = "-expert-major" if expert_major else ""
    out = {}
    for (name, gx), kib in fetch.items():
        base, targs = name.split("<")[0], [a.strip() for a in name.split("<", 1)[-1].rstrip(">").split(",")]
        if base == "exchange_kernel":        # <V, U, NT, REVERSE, FIRST, RPB>
            stage, direct = ("return" if targs[3] == "true" else "exchange"), False
        elif base == "pack_kernel":          # <V, U, NT, NTS, DIRECT, RPB>
            stage, direct = "pack", targs[4] == "true"
        elif base == "pack_gather_kernel":   # <V, U, NT, DIRECT, RPB>
            stage, direct = "pack", targs[3] == "true"
        elif base == "combine_kernel":       # <B, DT, U, NT, DIRECT, PAIRS, RPB>
            stage, direct = "combine", targs[4] == "true"
        elif base in stage_of:
            stage, direct = stage_of[base], False
        else:
            continue
        if stage is None or (name, gx) not in write:
            continue
        key = ("direct" if direct else "staged") + suffix
        if stage in out.setdefault(key, {}):
            raise RuntimeError(f"two kernels map to {key} {stage}: one layout per counter pass")
        out[key][stage] = {
            "read": int(round(kib * 1024.0 * read_factor)),
            "write": int(round(write[(name, gx)] * 1024.0 * write_factor)),
            "kernel": name, "grid_x": gx}
    path = out_path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    sha = kernel_source_sha256()
    if rec.get("kernel_source_sha256") != sha:
        rec = {"kernel_source_sha256": sha, "workloads": {}}
    wrec = rec.setdefault("workloads", {}).setdefault(workload, {})
    wrec["calibration" + suffix.replace("-", "_")] = {
        "copy_bytes_each_way": copy_bytes, "fetch_kib": fetch[big], "write_kib": write[big],
        "read_factor": round(read_factor, 5), "write_factor": round(write_factor, 5)}
    wrec.setdefault("per_launch_bytes", {}).update(out)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec["workloads"][workload], indent=1))


def _short_kernel_name(name):
    base = name.replace("void ", "").replace("a2av::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    base = base.replace("unsigned int __vector(4)", "u32x4").replace("unsigned int __vector(2)", "u32x2")
    return base.split("(")[0]


def api_summary(paths):
    """HIP runtime API calls per function from rocprofv3 databases (--hip-trace)."""
    import sqlite3
    for path in paths:
        c = sqlite3.connect(path)
        rows = c.execute("select name, count(*) from regions where category like '%HIP%' "
                         "group by name order by count(*) desc").fetchall()
        print(f"# {os.path.basename(path)}")
        print("| HIP API call | calls |")
        print("|---|---:|")
        for name, n in rows:
            print(f"| {name} | {n} |")
        print()


def profile_summary(paths):
    """Per (kernel, grid size) statistics from rocprofv3 rocpd databases: launches,
    average / min / max duration, and the average of every hardware counter collected
    (FETCH_SIZE / WRITE_SIZE are KiB per dispatch)."""
    import sqlite3
    for path in paths:
        c = sqlite3.connect(path)
        print(f"# {os.path.basename(path)}")
        rows = c.execute("select name, grid_x, workgroup_x, duration from kernels").fetchall()
        groups = {}
        for name, gx, wx, dur in rows:
            groups.setdefault((_short_kernel_name(name), gx, wx), []).append(dur)
        pmc = {}
        try:
            for name, gx, cname, val in c.execute(
                    "select kernel_name, grid_size_x, counter_name, value from counters_collection"):
                pmc.setdefault((_short_kernel_name(name), gx), {}).setdefault(cname, []).append(val)
        except sqlite3.Error:
            pass
        cnames = sorted({n for v in pmc.values() for n in v})
        print("| kernel | grid x | block | launches | avg us | min us | max us |"
              + "".join(f" avg {n} |" for n in cnames))
        print("|---|---:|---:|---:|---:|---:|---:|" + "---:|" * len(cnames))
        for key in sorted(groups, key=lambda k: -sum(groups[k])):
            d = groups[key]
            vals = pmc.get((key[0], key[1]), {})
            extra = "".join(f" {sum(vals[n]) / len(vals[n]):.1f} |" if n in vals else " |" for n in cnames)
            print(f"| {key[0]} | {key[1]} | {key[2]} | {len(d)} | {sum(d) / len(d) / 1e3:.2f} | "
                  f"{min(d) / 1e3:.2f} | {max(d) / 1e3:.2f} |{extra}")
        print()


if __name__ == "__main__":
    main()
