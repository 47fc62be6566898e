"""Benchmark of the fused producer/consumer gather-GEMM on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large|tp|ep|tiny]

A step is one pass of the hot path over one batch: layout (route) step, one
persistent kernel that moves the rows, counts arrivals, elects publishers,
publishes slots, gates and runs the bf16 contraction. Inputs are resident in
HBM before timing starts. Prints ONE JSON line.

The headline workload is the largest single-GPU configuration: 8 shards x
4096 rows scattered by a seeded permutation (M = 32768), K = N = 8192, bf16.
Beside its fused throughput the line reports the three timings of the
measurement method ("Know your platform" §5: T_comp alone with the same
workgroups, T_comm alone, T_total), overlap efficiency and compute
interference, the gather's HBM rate, a sweep of the copy-workgroup count
("Know your platform" §4), the publish-to-gate-observe latency from a traced
call, the same fields for the TP share and the EP dispatch workloads, the board
power of each mode with the bound a power cap puts on overlap efficiency, the
vendor library's GEMM (torch.matmul) on the same operands for context,
slot-signal latency (ping-pong round trip, slot barrier), the protocol-stress
signal rate, the two-stage, ring and combine entry points, the roofline of the
fused kernel and the CPU oracle timed on a bounded sample on the host cores.
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
PEAK_CLOCK_MHZ = 2400.0       # the clock that peak is quoted at
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


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
                host_threads=os.cpu_count() or 0, cpu_model=_cpu_model(),
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


def observe_latency(ctx, step, fg, torch):
    """Publish -> gate-observe latency from one traced call: for every whole
    tile whose row blocks completed after its workgroup took it (so that the
    workgroup was waiting), the time from the last of its blocks' counters
    reaching 128 (stamped by the copy wave whose add completed it) to the gate
    opening in the compute workgroup. Both stamps are on the device wall clock."""
    import numpy as np
    step(fg.CALL_TRACE)
    torch.cuda.synchronize()
    st = ctx.stats()
    tl = ctx.read_timeline()
    v = ctx.views()
    desc = ctx.read_i32(v.desc, 3).numpy()
    n_slabs = int(desc[1])
    slab = ctx.read_i32(v.slab, max(1, n_slabs)).numpy()[:n_slabs]
    tile_n = 256 if ctx.cfg.tile_n in (0, 256) and ctx.cfg.N % 256 == 0 else 128
    n_tn = ctx.cfg.N // tile_n
    tr, rbt, us = tl["trace"], tl["rb_time"], tl["us_per_tick"]
    lat = []
    for t in range(n_slabs * n_tn):
        entry = int(slab[t // n_tn])
        m0, bm = entry & ~1, 128 if entry & 1 else 256
        rbs = [m0 // 128] + ([m0 // 128 + 1] if bm == 256 else [])
        ready = max(int(rbt[r]) for r in rbs)
        if ready > int(tr[t, 1]) and int(tr[t, 2]) >= ready:
            lat.append((int(tr[t, 2]) - ready) * us)
    out = {"tiles": n_slabs * n_tn, "tiles_that_waited": len(lat),
           "max_wait_us": round(st.max_wait_ns / 1000.0, 2)}
    if lat:
        a = np.array(lat)
        out.update(p50_us=round(float(np.percentile(a, 50)), 3), p99_us=round(float(np.percentile(a, 99)), 3),
                   max_us=round(float(a.max()), 3))
    return out


def back_to_back_us(step, flags, n, torch):
    """Mean device time (us) of n back-to-back calls between one event pair on
    the current stream, after one untimed call."""
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


def overlap_fields(ctx, step, n_rep, flop, gather_bytes, fg, torch):
    """The three timings of "Know your platform" §5, each the median of
    separately synchronized calls with the same grid: T_comp alone (GEMM_ONLY,
    gates pre-opened), T_comm alone (COMM_ONLY), T_total (fused); overlap
    efficiency = (T_comp + T_comm - T_total) / min(T_comp, T_comm); compute
    interference = per-tile busy time fused / GEMM only."""
    t_total = _events_time(lambda: step(), n_rep, torch)
    st_f = ctx.stats()
    busy_fused = st_f.t_gemm_busy_us
    t_comp = _events_time(lambda: step(fg.CALL_GEMM_ONLY), n_rep, torch)
    busy_alone = ctx.stats().t_gemm_busy_us
    t_comm = _events_time(lambda: step(fg.CALL_COMM_ONLY), n_rep, torch)
    step()  # leave the buffers in the fused state
    torch.cuda.synchronize()
    med = lambda xs: statistics.median(xs) * 1000.0  # noqa: E731  (us)
    Tt, Tc, Tm = med(t_total), med(t_comp), med(t_comm)
    return {
        "T_comp_alone_us": round(Tc, 2), "T_comm_alone_us": round(Tm, 2), "T_total_us": round(Tt, 2),
        "T_total_p10_p90_us": [round(_pct(t_total, 10) * 1000, 2), round(_pct(t_total, 90) * 1000, 2)],
        "overlap_efficiency": round((Tc + Tm - Tt) / min(Tc, Tm), 4),
        "compute_interference": round(busy_fused / busy_alone, 4) if busy_alone else None,
        "wall_interference": round(Tt / Tc, 4),
        "gather_GBps": round(gather_bytes / (Tm * 1e-6) / 1e9, 1),
        "gather_frac_hbm": round(gather_bytes / (Tm * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "gemm_alone_TFLOPs": round(flop / (Tc * 1e-6) / 1e12, 2),
        "gemm_alone_frac": round(flop / (Tc * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "gate_wait_us_mean": round(st_f.t_gate_wait_us, 2),
        "clock_mhz_fused": round(st_f.clock_mhz, 0),
    }


class Bench:
    """One workload on one context: inputs resident on the device, the step."""

    def __init__(self, name, fg, W, torch, n_comm=0, tile_n=0, copy_mode=0):
        self.name = name
        self.fg, self.torch = fg, torch
        self.wl = setup_workload(name, torch, fg, W)
        wl = self.wl
        self.cfg = fg.make_config(wl["S"], wl["max_rows"], wl["K"], wl["N"], n_groups=wl["n_groups"],
                                  n_comm_wg=n_comm, tile_n=tile_n, copy_mode=copy_mode)
        self.ctx = fg.Context(self.cfg)
        cap = fg.capacity(self.cfg)
        self.gathered = torch.zeros(cap, wl["K"], dtype=torch.bfloat16, device="cuda:0")
        self.out = torch.zeros(cap, wl["N"], dtype=torch.bfloat16, device="cuda:0")
        self.flop = 2.0 * wl["m_real"] * wl["K"] * wl["N"]
        self.gather_bytes = 2.0 * wl["m_real"] * wl["K"] * 2

    def step(self, flags=0, ctx=None):
        c = ctx or self.ctx
        rc = c.gather_gemm(self.wl["shards"], self.wl["w"], self.gathered, self.out, route=self.wl["route"],
                           flags=flags)
        if rc != self.fg.OK:
            raise RuntimeError(f"fg_gather_gemm: {self.fg.strerror(rc)}")

    def check(self, ctx=None):
        st = (ctx or self.ctx).stats()
        if st.error_code:
            raise RuntimeError(f"device error {st.error_code} id {st.error_id}")
        return st

    def close(self):
        self.ctx.close()


def n_comm_sweep(b, t_comp_us, counts, torch, fg):
    """Sweep of the copy-workgroup count ("Know your platform" §4: the share of
    compute units given to communication must be swept), in the copy-workgroup
    mode (copy_mode 0: n_comm_wg workgroups copy every row, then compute): per
    count a context of its own on the same buffers, T_total as the mean of
    back-to-back fused steps and T_comm alone as the mean of back-to-back
    copy-only steps, overlap efficiency against the same T_comp alone (its grid
    does not change)."""
    out = []
    for n in counts:
        cfg = fg.make_config(b.wl["S"], b.wl["max_rows"], b.wl["K"], b.wl["N"], n_groups=b.wl["n_groups"],
                             n_comm_wg=n, copy_mode=fg.COPY_WORKGROUPS)
        ctx = fg.Context(cfg)
        step = lambda flags=0: b.step(flags, ctx)  # noqa: E731
        for _ in range(3):
            step()
        tt = back_to_back_us(step, 0, 10, torch)
        tm = back_to_back_us(step, fg.CALL_COMM_ONLY, 5, torch)
        b.check(ctx)
        ctx.close()
        out.append({"n_comm_wg": n, "T_total_us": round(tt, 1), "T_comm_alone_us": round(tm, 1),
                    "TFLOPs": round(b.flop / (tt * 1e-6) / 1e12, 1),
                    "overlap_efficiency": round((t_comp_us + tm - tt) / min(t_comp_us, tm), 3)})
    b.step()
    torch.cuda.synchronize()
    return out


def other_copy_mode(b, t_comp_us, mode, torch, fg):
    """The fused step with the other copy mode on the same buffers and grid:
    T_total (median of separately synchronized calls), TFLOP/s and the ratio
    to the same T_comp alone."""
    cfg = fg.make_config(b.wl["S"], b.wl["max_rows"], b.wl["K"], b.wl["N"], n_groups=b.wl["n_groups"],
                         copy_mode=mode)
    ctx = fg.Context(cfg)
    step = lambda flags=0: b.step(flags, ctx)  # noqa: E731
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    ts = _events_time(step, 20, torch)
    st = b.check(ctx)
    ctx.close()
    t = statistics.median(ts) * 1000.0
    return {"copy": "in tiles" if st.copy_in_tiles else "copy workgroups", "lead_rows": st.lead_rows,
            "T_total_us": round(t, 2), "TFLOPs": round(b.flop / (t * 1e-6) / 1e12, 1),
            "T_total_over_T_comp": round(t / t_comp_us, 4)}


def _power_files():
    """The board power sensor (microwatts) and the board's power cap, from the
    GPU's hwmon node in sysfs; None where the node is missing or unreadable."""
    import glob
    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        inp, cap = os.path.join(d, "power1_input"), os.path.join(d, "power1_cap")
        if not os.path.exists(inp):
            inp = os.path.join(d, "power1_average")
        try:
            int(open(inp).read().strip())
            c = int(open(cap).read().strip()) if os.path.exists(cap) else 0
        except (OSError, ValueError):
            continue
        return inp, c
    return None


def power_fields(ctx, step, step_us, fg, torch, secs=1.5):
    """Board power while GEMM-only, copy-only and fused steps run back to back
    (about `secs` each; the power sensor, sampled every 5 ms from a host thread,
    averages over a window, so the first third of each run is dropped), and the
    bound that a fixed power cap puts on overlap efficiency.

    Under full MFMA load the part runs at its power cap, so the copy's energy
    comes out of the same budget as the contraction's: the fused step cannot
    take less than T_comp + E_copy / P_cap, where E_copy is the energy the copy
    adds. Counted from the idle board (its incremental energy, (P_copy -
    P_idle) x T_comm) this bounds overlap efficiency by 1 - (P_copy - P_idle) /
    P_cap; counted whole (P_copy x T_comm) by 1 - P_copy / P_cap. The first
    reading ignores the static power that a busy part spends beyond idle, the
    second counts all of it, so the bound lies between the two."""
    import threading
    pf = _power_files()
    if pf is None:
        return None
    path, cap_uw = pf

    def sample(stop, out):
        while not stop.is_set():
            try:
                out.append(int(open(path).read().strip()))
            except (OSError, ValueError):
                pass
            time.sleep(0.005)

    torch.cuda.synchronize()
    time.sleep(1.0)
    idle = []
    stop = threading.Event()
    th = threading.Thread(target=sample, args=(stop, idle))
    th.start()
    time.sleep(0.3)
    stop.set()
    th.join()
    res = {"sensor": path, "cap_W": round(cap_uw / 1e6, 1), "idle_W": round(statistics.median(idle) / 1e6, 1)}
    for mode, flags in (("gemm_only", fg.CALL_GEMM_ONLY), ("comm_only", fg.CALL_COMM_ONLY), ("fused", 0)):
        n = max(20, int(secs * 1e6 / step_us[mode]))
        samples = []
        stop = threading.Event()
        th = threading.Thread(target=sample, args=(stop, samples))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        th.start()
        e0.record()
        for _ in range(n):
            step(flags)
        e1.record()
        e1.synchronize()
        stop.set()
        th.join()
        us = e0.elapsed_time(e1) * 1000.0 / n
        w = statistics.mean(samples[len(samples) // 3:]) / 1e6 if len(samples) >= 6 else float("nan")
        st = ctx.stats()
        res[mode] = {"W": round(w, 1), "us_per_step": round(us, 2), "mJ_per_step": round(w * us / 1000.0, 2),
                     "clock_mhz": round(st.clock_mhz, 0), "samples": len(samples)}
    step()
    torch.cuda.synchronize()
    res.update(power_bounds(res))
    return res


def library_gemm_fields(b, fg, torch, rounds=3, n=25, skip=8):
    """The same contraction by the vendor library (torch.matmul, which PyTorch
    hands to hipBLASLt) on the same operands: the gathered rows of the last
    fused step and W as [K][N] (grouped routes: one batched matmul over the
    groups, padded to the largest). Context for the roofline fraction, timed beside
    the fused kernel's GEMM-only and fused modes in alternating rounds (each
    round: n back-to-back launches per variant, per-launch events, the first
    `skip` dropped; medians over the rounds), plus the largest difference
    between the two outputs."""
    wl = b.wl
    same = fg.CALL_SAME_ROUTE if wl["route"].mode != fg.ROUTE_CONTIG else 0
    K, N, G = wl["K"], wl["N"], wl["n_groups"]
    if G == 1:
        M = wl["m_real"]
        A = b.gathered[:M]
        Wt = wl["w"].reshape(N, K).t().contiguous()   # [K][N], contiguous (no transposed view)
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda:0")
        lib_call = lambda: torch.matmul(A, Wt, out=out)  # noqa: E731
        form = "one matmul"
    else:
        # grouped routes: one batched matmul over the groups, each padded to the
        # largest group (padding rows of the gathered buffer are zero)
        goff = b.ctx.read_i32(b.ctx.views().group_off, G + 1).tolist()
        P = max(goff[g + 1] - goff[g] for g in range(G))
        A = torch.zeros(G, P, K, dtype=torch.bfloat16, device="cuda:0")
        for g in range(G):
            A[g, :goff[g + 1] - goff[g]] = b.gathered[goff[g]:goff[g + 1]]
        w3 = wl["w"].reshape(G, N, K)
        Wt = torch.stack([w3[g].t().contiguous() for g in range(G)]).contiguous()   # [G][K][N]
        outb = torch.empty(G, P, N, dtype=torch.bfloat16, device="cuda:0")
        lib_call = lambda: torch.bmm(A, Wt, out=outb)  # noqa: E731
        form = f"one batched matmul over {G} groups padded to {P} rows"

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record()
        for i in range(n):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(skip, n)]

    variants = {"library": lib_call,
                "gemm_only": lambda: b.step(fg.CALL_GEMM_ONLY | same),
                "fused": lambda: b.step(same)}
    ts = {k: [] for k in variants}
    for _ in range(rounds):
        for k, fn in variants.items():
            ts[k] += timed(fn)
    b.step(fg.CALL_GEMM_ONLY | same)
    variants["library"]()
    torch.cuda.synchronize()
    if G == 1:
        diff = (b.out[:M].float() - out.float()).abs().max().item()
    else:
        diff = max((b.out[goff[g]:goff[g + 1]].float() - outb[g, :goff[g + 1] - goff[g]].float()).abs().max().item()
                   for g in range(G))
    b.step()
    torch.cuda.synchronize()
    b.check()
    med = {k: statistics.median(v) for k, v in ts.items()}
    res = {"library_form": form}
    res.update({k + "_us": round(v, 1) for k, v in med.items()})
    res.update({k + "_TFLOPs": round(b.flop / (v * 1e-6) / 1e12, 1) for k, v in med.items()})
    res["gemm_only_over_library"] = round(med["library"] / med["gemm_only"], 4)
    res["fused_over_library"] = round(med["library"] / med["fused"], 4)
    res["max_abs_diff_gemm_only_vs_library"] = diff
    return res


def power_bounds(res):
    """Overlap efficiency of the back-to-back timings in `res` and the two
    readings of its bound under the power cap (see power_fields)."""
    cap = res["cap_W"] or max(res["gemm_only"]["W"], res["fused"]["W"])
    pc = res["comm_only"]["W"]
    tc, tm, tt = res["gemm_only"]["us_per_step"], res["comm_only"]["us_per_step"], res["fused"]["us_per_step"]
    return {"overlap_efficiency_back_to_back": round((tc + tm - tt) / min(tc, tm), 4),
            "overlap_bound_incremental": round(1.0 - (pc - res["idle_W"]) / cap, 4),
            "overlap_bound_whole": round(1.0 - pc / cap, 4),
            "T_total_energy_floor_us": round(tc + pc * tm / cap, 2)}


def secondary(name, steps, fg, W, torch):
    """Fused throughput (back-to-back steps after a warm-up), the three timings
    and overlap, and the publish-to-observe latency of another workload."""
    b = Bench(name, fg, W, torch)
    for _ in range(20):
        b.step()
    t = back_to_back_us(b.step, 0, steps, torch)
    res = {"config": dict(workload=name, **b.wl["info"]), "T_step_us": round(t, 2),
           "TFLOPs": round(b.flop / (t * 1e-6) / 1e12, 2),
           "frac_bf16_peak": round(b.flop / (t * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    res["overlap"] = overlap_fields(b.ctx, b.step, 10, b.flop, b.gather_bytes, fg, torch)
    ov = res["overlap"]
    res["power"] = power_fields(b.ctx, b.step, {"gemm_only": ov["T_comp_alone_us"], "comm_only": ov["T_comm_alone_us"],
                                                "fused": ov["T_total_us"]}, fg, torch, secs=1.0)
    res["publish_observe"] = observe_latency(b.ctx, b.step, fg, torch)
    lib = library_gemm_fields(b, fg, torch)
    if lib is not None:
        res["library_gemm"] = lib
    b.check()
    return b, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the clock settles over the first ten or so launches of the fused kernel
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large", choices=["large", "tp", "ep", "tiny"])
    ap.add_argument("--n-comm", type=int, default=0)
    ap.add_argument("--copy-mode", type=int, default=0, choices=[0, 1],
                    help="0: copy workgroups; 1: rows copied in the compute tiles where the shape allows")
    ap.add_argument("--tile-n", type=int, default=0)
    ap.add_argument("--no-extras", action="store_true", help="fused timing only (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="headline workload's fields only (no other workloads, latency, stress or other entry points)")
    ap.add_argument("--mode", default="fused", choices=["fused", "gemm_only", "comm_only", "library"],
                    help="timed steps in this mode (profiling runs of the compute or copy role alone, or of the "
                         "vendor library's GEMM on the same operands)")
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

    log(f"bench: workload {args.workload}, {args.warmup} warmup + {args.steps} timed steps ({args.mode})")
    b = Bench(args.workload, fg, W, torch, n_comm=args.n_comm, tile_n=args.tile_n, copy_mode=args.copy_mode)
    wl, ctx = b.wl, b.ctx
    if args.mode == "library":
        # profiling runs only: the same contraction by torch.matmul (hipBLASLt)
        # on the gathered rows of one fused step and W as [K][N]
        if wl["n_groups"] != 1:
            print("--mode library profiles the dense workloads (large, tp) only", file=sys.stderr)
            sys.exit(2)
        b.step()
        M = wl["m_real"]
        A = b.gathered[:M]
        Wt = wl["w"].reshape(wl["N"], wl["K"]).t().contiguous()
        out = torch.empty(M, wl["N"], dtype=torch.bfloat16, device="cuda:0")
        for _ in range(args.warmup):
            torch.matmul(A, Wt, out=out)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            torch.matmul(A, Wt, out=out)
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / args.steps
        if args.copy_calibration:
            src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.mul(src, 1.0, out=dst)
            torch.cuda.synchronize()
        b.close()
        print(json.dumps({"mode": "library", "workload": args.workload, "steps": args.steps, "warmup": args.warmup,
                          "us_per_step": round(us, 2), "TFLOPs": round(b.flop / (us * 1e-6) / 1e12, 1)}), flush=True)
        return
    mode_flags = {"fused": 0, "gemm_only": fg.CALL_GEMM_ONLY, "comm_only": fg.CALL_COMM_ONLY}[args.mode]
    if mode_flags == fg.CALL_GEMM_ONLY:
        b.step()   # the gathered rows the compute role reads
    for _ in range(args.warmup):
        b.step(mode_flags)
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` back-to-back steps between one pair of
    # HIP events on the stream the kernels run on (torch's current stream, which
    # the library is bound to). With a cached CONTIG layout a step is one launch
    # of the fused kernel; otherwise the step's layout kernel is included.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        b.step(mode_flags)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = b.check()
    ms_per_step = wall * 1000.0 / args.steps
    step_ms = e0.elapsed_time(e1) / args.steps
    value = b.flop * args.steps / wall / 1e12
    # the fused kernel's own launch duration for the roofline: with an EXPLICIT
    # or TOPK route a step also runs the layout kernel, so the same number of
    # launches is timed again with the route marked unchanged (fused kernel only)
    layout_per_step = wl["route"].mode != fg.ROUTE_CONTIG
    if layout_per_step:
        e2 = torch.cuda.Event(enable_timing=True)
        e3 = torch.cuda.Event(enable_timing=True)
        e2.record()
        for i in range(args.steps):
            b.step(mode_flags | fg.CALL_SAME_ROUTE)
        e3.record()
        torch.cuda.synchronize()
        b.check()
        avg_launch_ms = e2.elapsed_time(e3) / args.steps
    else:
        avg_launch_ms = step_ms

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
        "config": dict(workload=f"{args.workload}", **wl["info"],
                       copy="in tiles" if st.copy_in_tiles else "copy workgroups",
                       lead_rows=st.lead_rows, n_comm_wg=st.n_comm_wg if not st.copy_in_tiles else None,
                       tiles_whole=st.tiles_whole, tiles_split=st.tiles_split, split_parts=st.split_parts),
    }
    if args.mode != "fused":
        result["mode"] = args.mode
    achieved = b.flop / (avg_launch_ms * 1e-3) / 1e12
    traffic = recorded_traffic(args.workload)
    result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                          "traffic": None if traffic is None else int(traffic),
                          "kernel": "fused_kernel", "avg_launch_us": round(avg_launch_ms * 1000, 2),
                          "step_us_incl_layout": round(step_ms * 1000, 2),
                          "algorithmic_flop_per_launch": b.flop,
                          "algorithmic_gather_bytes_per_launch": b.gather_bytes,
                          "clock_mhz": round(st.clock_mhz, 0)}
    if st.clock_mhz > 0:
        # context, not the contract's frac: the same peak scaled to the shader
        # clock the part held under this load (it is power-limited below 2.4 GHz)
        peak_clk = PEAK_BF16_TFLOPS * st.clock_mhz / PEAK_CLOCK_MHZ
        result["roofline"].update(peak_at_clock=round(peak_clk, 1), frac_at_clock=round(achieved / peak_clk, 4))

    if not args.no_extras and args.mode == "fused":
        n_rep = max(10, args.steps)
        ov = overlap_fields(ctx, b.step, n_rep, b.flop, b.gather_bytes, fg, torch)
        result["overlap"] = ov
        result["power"] = power_fields(ctx, b.step, {"gemm_only": ov["T_comp_alone_us"],
                                                     "comm_only": ov["T_comm_alone_us"],
                                                     "fused": ov["T_total_us"]}, fg, torch)
        result["publish_observe"] = observe_latency(ctx, b.step, fg, torch)
        result["library_gemm"] = library_gemm_fields(b, fg, torch)
        log("bench: copy-workgroup sweep")
        result["n_comm_sweep"] = n_comm_sweep(b, ov["T_comp_alone_us"], [8, 16, 32, 64, 128, 192, 224], torch, fg)
        result["other_copy_mode"] = other_copy_mode(b, ov["T_comp_alone_us"], 1 - args.copy_mode, torch, fg)
    if not args.no_extras and args.mode == "fused" and not args.no_secondary:
        others = {}
        tp_b = ep_b = None
        for name in ("tp", "ep"):
            if name == args.workload:
                continue
            log(f"bench: secondary workload {name}")
            sb, others[name] = secondary(name, 50, fg, W, torch)
            if name == "tp":
                tp_b = sb
            else:
                ep_b = sb
        result["workloads"] = others
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
                            "errors": int(sst.error_code), "timeouts": int(sst.timeouts),
                            "us_per_iter_no_delay": round(statistics.median(t_nodelay) * 1000, 2),
                            "us_per_iter_delays_0_20us": round(statistics.median(t_delay) * 1000, 2),
                            "signals_per_s_no_delay": round(signals / (statistics.median(t_nodelay) * 1e-3), 0)}
        if tp_b is not None:
            result["two_stage"] = two_stage_bench(args, tp_b.wl, tp_b.ctx, tp_b.gathered, tp_b.out, torch, fg)
            result["ring"] = ring_bench(args, tp_b.wl, tp_b.ctx, tp_b.gathered, tp_b.out, torch, fg)
            tp_b.close()
        if ep_b is not None:
            result["combine"] = combine_bench(args, ep_b.wl, ep_b.ctx, ep_b.gathered, ep_b.out, torch, fg, W)
            ep_b.close()
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
    b.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
