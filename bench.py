"""Benchmark of the fused producer/consumer gather-GEMM on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload tp|large|ep|tiny]

A step is one pass of the hot path over one batch: layout (route) step, one
persistent kernel that moves the rows, counts arrivals, elects publishers,
publishes slots, gates and runs the bf16 contraction. Inputs are resident in
HBM before timing starts. Prints ONE JSON line.

Beside the fused throughput it reports the three timings of the measurement
method ("Know your platform" §5: T_comp alone with the same workgroups, T_comm
alone, T_total), overlap efficiency and compute interference, the gather's
HBM rate, slot-signal latency (ping-pong round trip, slot barrier), the
protocol-stress signal rate, the roofline of the fused kernel and the CPU
oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "fused gather-GEMM TFLOP/s + overlap efficiency; slot-signal latency (\u00b5s)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 29          # plain device copy used to calibrate the HBM byte counters


def kernel_source_hash():
    """sha256 of the code of the HIP sources and the C header (comments and
    white space removed): traffic counters recorded for other code do not
    describe the kernel that runs; an edited comment does not change it."""
    import hashlib
    import re

    def code(text):
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        return " ".join(text.split()).encode()

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sync_protocols_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code(f.read()))
    with open(os.path.join(ROOT, "include", "fg.h"), encoding="utf-8") as f:
        h.update(code(f.read()))
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch of the fused kernel from the committed counter
    summary, or None if there is none for this workload and these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _events_time(fn, n, torch):
    """Per-call device time (ms) of n calls, HIP events on the current stream."""
    times = []
    for _ in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    return times


def _pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))]


def setup_workload(name, torch, fg, W):
    dev = "cuda:0"
    c = dict(W.CONFIGS[name])
    if c["kind"] == "dense":
        d = W.dense_inputs(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"], gather=c["gather"])
        S, R, K, N = c["n_shards"], c["rows"], c["K"], c["N"]
        shards = [s.to(dev) for s in d.shards]
        w = d.w.to(dev)
        if c["gather"] == "contiguous":
            route = fg.route_contig(R)
        else:
            src = torch.arange(R, dtype=torch.int32).repeat(S, 1).contiguous().to(dev)
            dst = d.perm.reshape(S, R).contiguous().to(dev)
            route = fg.route_explicit([R] * S, src, dst, S * R, R)
        m_real = S * R
        stream_len = [R] * S
        n_groups = 1
        max_rows = R
        info = dict(n_shards=S, rows_per_shard=R, M=m_real, K=K, N=N, gather=c["gather"])
        inputs = dict(dense=d)
    else:
        e = W.ep_inputs(c["seed"], n_shards=c["n_shards"], tokens=c["tokens"], K=c["K"], N=c["N"],
                        n_experts=c["n_experts"], topk=c["topk"], n_local=c["n_local"],
                        expert_base=c["expert_base"])
        S, K, N = c["n_shards"], c["K"], c["N"]
        shards = [s.to(dev) for s in e.shards]
        w = e.w.to(dev)
        topk = e.topk.to(dev).contiguous()
        route = fg.route_topk(topk, c["tokens"], c["expert_base"])
        local = ((e.topk >= c["expert_base"]) & (e.topk < c["expert_base"] + c["n_local"]))
        m_real = int(local.sum())
        stream_len = [int(x) for x in local.reshape(S, -1).sum(dim=1)]
        n_groups = c["n_local"]
        max_rows = c["tokens"] * min(c["topk"], c["n_local"])
        info = dict(n_shards=S, tokens_per_shard=c["tokens"], M=m_real, K=K, N=N, topk=c["topk"],
                    experts=c["n_experts"], local_experts=c["n_local"])
        inputs = dict(ep=e)
    return dict(name=name, shards=shards, w=w, route=route, m_real=m_real, stream_len=stream_len, n_groups=n_groups,
                max_rows=max_rows, K=K, N=N, S=S, info=info, inputs=inputs, iters=c["iters"], cfg=c)


def cpu_baseline(wl, budget_s=12.0):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    workload: whole steps (layout, gather of every row, float64 contraction of
    every real row), repeated until about `budget_s` of CPU work; if one step
    would take much longer, the contraction is restricted to a prefix of the
    real rows. Returns contraction TFLOP/s of the sample."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    c = wl["cfg"]
    K, N = wl["K"], wl["N"]

    def bits(t):
        return t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)

    if c["kind"] == "dense":
        d = wl["inputs"]["dense"]
        shards = [bits(s) for s in d.shards]
        wb = bits(d.w)[None]
        perm = d.perm.numpy() if c["gather"] != "contiguous" else None

        def layout():
            if perm is None:
                return O.layout_contiguous(c["n_shards"], c["rows"])
            return O.layout_permutation(perm, c["n_shards"], c["rows"])
    else:
        e = wl["inputs"]["ep"]
        shards = [bits(s) for s in e.shards]
        wb = bits(e.w)
        topk = e.topk.numpy()

        def layout():
            return O.layout_topk(topk, c["expert_base"], c["n_local"])

    def one_step(rows):
        lay = layout()
        G = O.gather(shards, lay)
        O.seeds(lay)
        O.signal_counts(lay)
        real_idx = np.nonzero(O.real_rows(lay))[0]
        sel = real_idx if rows is None else real_idx[:rows]
        O.gemm(G, wb, lay, rows=None if rows is None else sel)
        return len(sel)

    # warm-up (first-touch, thread pool start), then steps on 64 and 512 rows
    # give the fixed and the per-row cost
    one_step(64)
    t0 = time.perf_counter()
    one_step(64)
    t1 = time.perf_counter()
    one_step(512)
    t2 = time.perf_counter()
    per_row = max(((t2 - t1) - (t1 - t0)) / 448, 1e-9)
    fixed = max((t1 - t0) - 64 * per_row, 0.0)
    rows = None if fixed + wl["m_real"] * per_row <= budget_s else max(64, int((budget_s - fixed) / per_row))
    t0 = time.perf_counter()
    steps, done_rows = 0, 0
    while True:
        done_rows += one_step(rows)
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flop = 2.0 * done_rows * K * N
    what = "every real row" if rows is None else f"the first {rows} real rows"
    return dict(value=round(flop / dt / 1e12, 6), unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"{steps} whole step(s) of the oracle (layout, gather of all rows, float64 contraction of "
                       f"{what} x K={K} x N={N}) in {dt:.1f} s; value = contraction FLOP / wall time")


def two_stage_bench(args, wl, ctx, gathered, out, torch, fg):
    """The two-stage dispatch (fg_gather_gemm_staged) on the same workload and
    context, with shard 0 as the self shard: T_total and the copy roles alone
    (push + scatter), each the mean of back-to-back steps between one event
    pair; algorithmic copy bytes = push (2 x remote rows x K x 2) + scatter
    (2 x M x K x 2)."""
    S, K = wl["S"], wl["K"]
    staging = [None if s == 0 else torch.empty(ctx.cfg.max_rows_per_shard, K, dtype=torch.bfloat16, device="cuda:0")
               for s in range(S)]

    def step(flags=0):
        rc = ctx.gather_gemm_staged(wl["shards"], wl["w"], staging, gathered, out, self_shard=0, route=wl["route"],
                                    flags=flags)
        if rc != fg.OK:
            raise RuntimeError(f"fg_gather_gemm_staged: {fg.strerror(rc)}")

    def back_to_back(flags, n):
        step(flags)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            step(flags)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / n

    for _ in range(3):
        step()
    n = max(10, args.steps)
    Tt = back_to_back(0, n)
    Tc = back_to_back(fg.CALL_COMM_ONLY, n)
    st = ctx.stats()
    if st.error_code:
        raise RuntimeError(f"device error {st.error_code} id {st.error_id}")
    M = wl["m_real"]
    remote = M - wl["stream_len"][0]
    copy_bytes = 2.0 * remote * K * 2 + 2.0 * M * K * 2
    flop = 2.0 * M * K * wl["N"]
    step()
    torch.cuda.synchronize()
    return {"self_shard": 0, "T_total_us": round(Tt, 2), "T_copy_alone_us": round(Tc, 2),
            "TFLOPs": round(flop / (Tt * 1e-6) / 1e12, 2), "copy_bytes": copy_bytes,
            "copy_GBps": round(copy_bytes / (Tc * 1e-6) / 1e9, 1)}


def ring_bench(args, wl, ctx, gathered, out, torch, fg):
    """The dispatch through bounded FIFO rings (fg_gather_gemm_ring) on the same
    workload and context, shard 0 as the self shard, as many rings per shard
    as the copy workgroups serve, one 64-row slot each: T_total and the copy
    roles alone, each the mean of back-to-back steps, and the ring memory
    against the whole streams."""
    S, K = wl["S"], wl["K"]
    n_ch = max(1, ctx.views().ring_cap // S)
    slots = 1
    nbytes = fg.ring_bytes(ctx.cfg, n_ch, slots)
    ring = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda:0")

    def step(flags=0):
        rc = ctx.gather_gemm_ring(wl["shards"], wl["w"], ring, gathered, out, n_channels=n_ch, ring_chunks=slots,
                                  self_shard=0, route=wl["route"], flags=flags)
        if rc != fg.OK:
            raise RuntimeError(f"fg_gather_gemm_ring: {fg.strerror(rc)}")

    def back_to_back(flags, n):
        step(flags)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            step(flags)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / n

    for _ in range(3):
        step()
    n = max(10, args.steps)
    Tt = back_to_back(0, n)
    Tc = back_to_back(fg.CALL_COMM_ONLY, n)
    st = ctx.stats()
    if st.error_code:
        raise RuntimeError(f"device error {st.error_code} id {st.error_id}")
    flop = 2.0 * wl["m_real"] * K * wl["N"]
    stream_bytes = sum(wl["stream_len"][1:]) * K * 2.0
    step()
    torch.cuda.synchronize()
    return {"self_shard": 0, "rings_per_shard": n_ch, "slots_per_ring": slots, "ring_MB": round(nbytes / 1e6, 1),
            "remote_streams_MB": round(stream_bytes / 1e6, 1), "T_total_us": round(Tt, 2),
            "T_copy_alone_us": round(Tc, 2), "TFLOPs": round(flop / (Tt * 1e-6) / 1e12, 2)}


def combine_bench(args, wl, ctx, gathered, out, torch, fg, W):
    """The combine step on the EP workload (8 x 1024 tokens, top-8 of 64 experts,
    8 local, N = 2048): T_total (push + weighted sums in one kernel), push alone,
    sums alone (each the mean of back-to-back calls between one event pair),
    overlap, and the HBM rate over the algorithmic bytes
    3 * M * N * 2 (expert rows read, staging written, staging read) +
    S * T * N * 2 (outputs written) + M * 4 (gate weights)."""
    if wl["name"] != "ep":
        wl = setup_workload("ep", torch, fg, W)
        cfg = fg.make_config(wl["S"], wl["max_rows"], wl["K"], wl["N"], n_groups=wl["n_groups"])
        ctx = fg.Context(cfg)
        cap = fg.capacity(cfg)
        gathered = torch.zeros(cap, wl["K"], dtype=torch.bfloat16, device="cuda:0")
        out = torch.zeros(cap, wl["N"], dtype=torch.bfloat16, device="cuda:0")
        own = True
    else:
        own = False
    c = wl["cfg"]
    S, T, KK, N = wl["S"], c["tokens"], c["topk"], wl["N"]
    rc = ctx.gather_gemm(wl["shards"], wl["w"], gathered, out, route=wl["route"])
    if rc != fg.OK:
        raise RuntimeError(f"fg_gather_gemm: {fg.strerror(rc)}")
    _, weights = W.combine_inputs(c["seed"] + 1, 1, N, S, T, KK)
    weights = weights.to("cuda:0")
    staging = [torch.empty(ctx.cfg.max_rows_per_shard, N, dtype=torch.bfloat16, device="cuda:0") for _ in range(S)]
    ys = [torch.empty(T, N, dtype=torch.bfloat16, device="cuda:0") for _ in range(S)]

    call = ctx.prepare_combine(out, weights, staging, ys)   # arguments marshalled outside the timed loops

    def comb(flags=0):
        r = call(flags)
        if r != fg.OK:
            raise RuntimeError(f"fg_combine: {fg.strerror(r)}")

    def back_to_back(flags, n):
        """Mean device time (us) of n back-to-back calls between one event pair."""
        comb(flags)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            comb(flags)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / n

    for _ in range(5):
        comb()
    torch.cuda.synchronize()
    n_rep = max(50, args.steps)
    Tt = back_to_back(0, n_rep)
    Tp = back_to_back(fg.CALL_COMM_ONLY, n_rep)
    Ts = back_to_back(fg.CALL_GEMM_ONLY, n_rep)
    t_single = _events_time(comb, 20, torch)
    st = ctx.stats()
    if st.error_code:
        raise RuntimeError(f"device error {st.error_code} id {st.error_id}")
    M = wl["m_real"]
    alg = 3.0 * M * N * 2 + float(S) * T * N * 2 + M * 4.0
    if own:
        ctx.close()
    gbs = alg / (Tt * 1e-6) / 1e9
    return {"workload": "ep", "M": M, "tokens": S * T, "N": N, "kernel": "combine_kernel",
            "T_total_us": round(Tt, 2),
            "T_single_call_incl_launch_us": round(statistics.median(t_single) * 1000, 2),
            "T_push_alone_us": round(Tp, 2), "T_sums_alone_us": round(Ts, 2),
            "overlap_efficiency": round((Tp + Ts - Tt) / min(Tp, Ts), 4),
            "algorithmic_bytes_per_launch": alg,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The first 75-100 back-to-back steps after an idle GPU run 5-30 % slower
    # while the clock settles under the load; 150 warm-up steps (about 40 ms on
    # TP) put the timed region in the steady state that continuous use sees.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--workload", default="tp", choices=["tp", "large", "ep", "tiny"])
    ap.add_argument("--n-comm", type=int, default=0)
    ap.add_argument("--tile-n", type=int, default=0)
    ap.add_argument("--no-extras", action="store_true", help="fused timing only (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of a known size (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X "
              "(source shards are HBM regions on that GPU); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from sync_protocols_amd import fg
    from sync_protocols_amd import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    wl = setup_workload(args.workload, torch, fg, W)
    cfg = fg.make_config(wl["S"], wl["max_rows"], wl["K"], wl["N"], n_groups=wl["n_groups"],
                         n_comm_wg=args.n_comm, tile_n=args.tile_n)
    log(f"bench: workload {args.workload}, {args.warmup} warmup + {args.steps} timed steps")
    ctx = fg.Context(cfg)
    cap = fg.capacity(cfg)
    gathered = torch.zeros(cap, wl["K"], dtype=torch.bfloat16, device="cuda:0")
    out = torch.zeros(cap, wl["N"], dtype=torch.bfloat16, device="cuda:0")
    flop = 2.0 * wl["m_real"] * wl["K"] * wl["N"]
    gather_bytes = 2.0 * wl["m_real"] * wl["K"] * 2

    def step(flags=0):
        rc = ctx.gather_gemm(wl["shards"], wl["w"], gathered, out, route=wl["route"], flags=flags)
        if rc != fg.OK:
            raise RuntimeError(f"fg_gather_gemm: {fg.strerror(rc)}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` back-to-back steps between one pair of
    # HIP events on the stream the kernels run on (torch's current stream, which
    # the library is bound to). With a cached CONTIG layout a step is one launch
    # of the fused kernel; otherwise the step's layout kernels are included.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = ctx.stats()
    if st.error_code:
        raise RuntimeError(f"device error {st.error_code} id {st.error_id}")
    ms_per_step = wall * 1000.0 / args.steps
    avg_launch_ms = e0.elapsed_time(e1) / args.steps
    value = flop * args.steps / wall / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(workload=f"{args.workload}", **wl["info"], n_comm_wg=st.n_comm_wg,
                       n_gemm_wg=st.n_gemm_wg, tiles_whole=st.tiles_whole, tiles_split=st.tiles_split,
                       split_parts=st.split_parts),
    }
    achieved = flop / (avg_launch_ms * 1e-3) / 1e12
    traffic = recorded_traffic(args.workload)
    result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                          "traffic": None if traffic is None else int(traffic),
                          "kernel": "fused_kernel", "avg_launch_us": round(avg_launch_ms * 1000, 2),
                          "algorithmic_flop_per_launch": flop,
                          "algorithmic_gather_bytes_per_launch": gather_bytes}

    if not args.no_extras:
        n_rep = max(10, args.steps)
        t_total = _events_time(lambda: step(), n_rep, torch)
        st_f = ctx.stats()
        busy_fused = st_f.t_gemm_busy_us
        t_comp = _events_time(lambda: step(fg.CALL_GEMM_ONLY), n_rep, torch)
        st_c = ctx.stats()
        busy_alone = st_c.t_gemm_busy_us
        t_comm = _events_time(lambda: step(fg.CALL_COMM_ONLY), n_rep, torch)
        step()  # leave the buffers in the fused state
        torch.cuda.synchronize()
        med = lambda xs: statistics.median(xs) * 1000.0  # noqa: E731  (us)
        Tt, Tc, Tm = med(t_total), med(t_comp), med(t_comm)
        ov = (Tc + Tm - Tt) / min(Tc, Tm)
        result["overlap"] = {
            "T_comp_alone_us": round(Tc, 2), "T_comm_alone_us": round(Tm, 2), "T_total_us": round(Tt, 2),
            "T_total_p10_p90_us": [round(_pct(t_total, 10) * 1000, 2), round(_pct(t_total, 90) * 1000, 2)],
            "overlap_efficiency": round(ov, 4),
            "compute_interference": round(busy_fused / busy_alone, 4) if busy_alone else None,
            "wall_interference": round(Tt / Tc, 4),
            "gather_GBps": round(gather_bytes / (Tm * 1e-6) / 1e9, 1),
            "gather_frac_hbm": round(gather_bytes / (Tm * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "gemm_alone_TFLOPs": round(flop / (Tc * 1e-6) / 1e12, 2),
            "gate_wait_us_mean": round(st_f.t_gate_wait_us, 2),
        }
        # slot-signal latency
        lat = fg.Context(fg.make_config(8, 256, 256, 256))
        assert lat.pingpong(10000, False) == 0
        rtt_a = lat.stats().t_rtt_us
        assert lat.pingpong(10000, True) == 0
        rtt_s = lat.stats().t_rtt_us
        assert lat.barrier(1000) == 0
        bar8 = lat.stats().t_barrier_us
        lat.close()
        lat4 = fg.Context(fg.make_config(4, 256, 256, 256))
        assert lat4.barrier(1000) == 0
        bar4 = lat4.stats().t_barrier_us
        host = _events_time(lambda: lat4.barrier(1), 50, torch)
        lat4.close()
        result["slot_latency_us"] = {"pingpong_rtt_agent": round(rtt_a, 3), "pingpong_rtt_system": round(rtt_s, 3),
                                     "barrier_4_ranks": round(bar4, 3), "barrier_8_ranks": round(bar8, 3),
                                     "barrier_4_ranks_per_call_incl_launch": round(statistics.median(host) * 1000, 2)}
        # protocol stress
        sc = W.CONFIGS["stress"]
        s_in = W.stress_inputs(sc["seed"], iters=sc["iters"])
        P, Cc, KC = s_in.chunk_rows.shape
        sctx = fg.Context(fg.make_config(4, 256, 256, 256, stress=(P, Cc, KC)))
        cr = s_in.chunk_rows.cuda()
        dl = s_in.delays_ns.cuda()
        zero = torch.zeros_like(dl[0])
        payload = torch.zeros(Cc * P * KC * 64, dtype=torch.int32, device="cuda:0")
        assert sctx.stress(cr, zero, payload) == 0
        t_nodelay = _events_time(lambda: sctx.stress(cr, zero, payload), 10, torch)
        t_delay = []
        for t in range(sc["iters"]):
            t_delay += _events_time(lambda: sctx.stress(cr, dl[t].contiguous(), payload), 1, torch)
        sst = sctx.stats()
        sctx.close()
        signals = int((s_in.chunk_rows > 0).sum())
        result["stress"] = {"signals_per_iter": signals, "iters": sc["iters"] + 11, "stale": int(sst.stale),
                            "errors": int(sst.error_code),
                            "us_per_iter_no_delay": round(statistics.median(t_nodelay) * 1000, 2),
                            "us_per_iter_delays_0_20us": round(statistics.median(t_delay) * 1000, 2),
                            "signals_per_s_no_delay": round(signals / (statistics.median(t_nodelay) * 1e-3), 0)}
        result["two_stage"] = two_stage_bench(args, wl, ctx, gathered, out, torch, fg)
        result["ring"] = ring_bench(args, wl, ctx, gathered, out, torch, fg)
        result["combine"] = combine_bench(args, wl, ctx, gathered, out, torch, fg, W)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)     # one elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        log(f"bench: copy calibration, 3 copies of {COPY_BYTES} bytes")
    if not args.no_cpu:
        log("bench: oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline(wl)
    ctx.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
