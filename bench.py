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
per-kernel event times, `stage_us` their breakdown); `ms_per_step` is a whole step
(expert stand-in included).  `roofline` is for the slowest kernel of the step, from its
per-kernel event time; `cpu_baseline` is the CPU oracle on a bounded sample of
the same workload; `decode_graph` and `edge_graph` are the decode and edge shapes
captured in hipGraphs and replayed with routing that changes on the device each step;
`graph_kernel_node_us` is what one nearly empty dependent kernel adds to a replayed
graph step (the launch gap); `wide` is the top-8 shape (16 x 2048 tokens, hidden 7168,
256 experts) timed the same way as the headline, 10 steps per path.
"""
import argparse
import json
import os
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
    if rec.get("kernel_source_sha256") != sha or rec.get("workload") != workload:
        return None
    b = rec.get("per_launch_bytes", {}).get(path, {}).get(kernel)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-graph", action="store_true")
    ap.add_argument("--no-wide", action="store_true",
                    help="skip the top-8 wide shape (16 x 2048 tokens, hidden 7168) timed after the headline")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
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
    w = W.workload(args.workload)
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
        "ms_per_step": head["ms_per_step_full"],
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
        "roofline": dict(head["roofline"], copy_reference_GBps=round(copy_gbps, 1),
                         row_copy_reference_GBps=round(row_copy_gbps, 1),
                         frac_of_row_copy=round(head["roofline"]["achieved"] / row_copy_gbps, 4)),
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
        wide = {}
        for p in paths:
            m = time_path(torch, a2av, ww, xwt, idwt, gwt, p, 10, 3)
            wide[p] = {k: m[k] for k in ("us_per_step", "us_per_step_min", "GBps", "pct_hbm_peak", "bytes_per_step",
                                         "stage_us")}
        result["wide"] = {"workload": ww.describe(), "steps": 10, "warmup": 3, "paths": wide}
        del xwt, idwt, gwt
        torch.cuda.empty_cache()

    if not args.no_decode_graph:
        result["graph_kernel_node_us"] = graph_kernel_node_us(torch, a2av)
        result["decode_graph"] = {p: decode_graph(np, torch, a2av, W, p) for p in paths}
        result["edge_graph"] = {p: decode_graph(np, torch, a2av, W, p, workload="edge") for p in paths}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, W, w, args.cpu_sample_tokens)

    print(json.dumps(result), flush=True)


def path_config(a2av, name):
    """'staged' | 'direct', optionally with '-expert-major': (path, receive layout)."""
    path = a2av.PATH_DIRECT if name.startswith("direct") else a2av.PATH_STAGED
    layout = a2av.LAYOUT_EXPERT_MAJOR if name.endswith("expert-major") else a2av.LAYOUT_SOURCE_MAJOR
    return path, layout


def time_path(torch, a2av, w, xt, idt, gt, name, steps, warmup, trials=5):
    """One path: warm-up; `steps` steps with HIP events recorded between the library's
    kernels (on the stream they run on) for the per-kernel breakdown and the roofline;
    then `trials` end-to-end runs with events only around the whole loop: `steps`
    dispatch+combine pairs (the headline: median trial, launch gaps included, no event
    between kernels; the minimum beside it), and `steps` full steps with the expert
    stand-in between them."""
    path_id, layout = path_config(a2av, name)
    direct = path_id == a2av.PATH_DIRECT
    path = name
    s = a2av.Session(w.num_ranks, w.tokens_per_rank, w.hidden, w.dtype, w.experts_per_rank, w.top_k,
                     w.recv_capacity_rows, path=path_id, recv_layout=layout)
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
            "traffic": measured_traffic(w.name, path, dom), "bytes_per_launch": sb[dom],
            "us_per_launch": round(launch_ms[dom] * 1e3, 2),
        },
    }


def decode_graph(np, torch, a2av, W, path, workload="decode", steps=100, per_graph=10, replays=None):
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
    and replayed that many times (for API tracing)."""
    w = W.workload(workload)
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

    def us_per_step(fn, count, total):
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
            if int(counter.item()) != total:
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
    t_one = us_per_step(full, 1, steps)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    t_full_f = us_per_step(flushed(full), per_graph, steps)
    t_harness_f = us_per_step(flushed(harness), per_graph, steps)
    ok = int(s.status.item()) == 0
    out = {"workload": w.describe(), "steps": steps, "steps_per_graph": per_graph,
           "us_per_step_with_expert_and_router": round(t_full, 2),
           "us_router_and_expert_only": round(t_harness, 2),
           "us_dispatch_combine_estimate": round(t_full - t_harness, 2),
           "us_dispatch_only_estimate": round(t_route_dispatch - t_route, 2),
           "us_per_step_one_step_graphs": round(t_one, 2),
           "flushed_512MiB": {"us_per_step_with_expert_and_router": round(t_full_f, 2),
                              "us_router_and_expert_only": round(t_harness_f, 2),
                              "us_dispatch_combine_estimate": round(t_full_f - t_harness_f, 2)},
           "host_syncs_between_replays": 0, "status_ok": ok,
           "algorithmic_bytes_per_step": step_bytes(w, path_id == a2av.PATH_DIRECT)}
    log(f"graph latency ({path}, {workload}): dispatch+combine {t_full - t_harness:.2f} us warm, "
        f"{t_full_f - t_harness_f:.2f} us flushed")
    del flush_buf
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


def cpu_baseline(np, W, w, sample_tokens):
    """The CPU oracle as it stands (single-threaded C, fp64) on the same workload with
    fewer tokens per rank: dispatch + return + combine timed (expert stand-in excluded),
    reported as effective GB/s over the same staged byte count."""
    import oracle
    ws = W.workload(w.name, tokens_per_rank=min(sample_tokens, w.tokens_per_rank))
    log(f"cpu baseline: oracle on {ws.describe()}")
    x, ids, gates = W.make_inputs(ws)
    rows = oracle.as_rows(x)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        d = oracle.dispatch(rows, ids, ws.experts_per_rank, ws.capacity)
        t1 = time.perf_counter()
        R, cap, H = ws.num_ranks, ws.capacity, ws.hidden
        recv = d["recv"].view(x.dtype).reshape(R, cap, H)
        z = oracle.expert(recv, d["cnt"], d["recv_off"], ws.experts_per_rank, ws.dtype, ws.expert_mode)
        t2 = time.perf_counter()
        ret = oracle.return_exchange(oracle.as_rows(z), d["send_off"], d["recv_off"], ws.tokens_per_rank, ws.top_k)
        oracle.combine(ret.view(x.dtype).reshape(R, -1, H), d["pos"], gates, ws.dtype)
        t3 = time.perf_counter()
        times.append((t1 - t0) + (t3 - t2))
    t = float(np.median(times))
    gbps = step_bytes(ws, False) / t / 1e9
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        model = "unknown"
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{ws.describe()} ({ws.tokens_per_rank} of {w.tokens_per_rank} tokens per rank), "
                      f"median of 3, dispatch+return+combine, {t * 1e3:.0f} ms per step",
            "host_cpu": model, "host_threads_available": os.cpu_count()}


def _short_kernel_name(name):
    base = name.replace("void ", "").replace("a2av::(anonymous namespace)::", "")
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
