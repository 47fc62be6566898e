"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare every result with the CPU oracle."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W

DEV = "cuda:0"
POISON = 0x7FC1          # a bf16 NaN; a gate that opens early lets it into the output


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def misaligned_like(t: torch.Tensor, shift_bytes: int = 2) -> torch.Tensor:
    """A copy of t whose first element sits shift_bytes past a 16-byte boundary."""
    es = t.element_size()
    assert shift_bytes % es == 0
    flat = torch.empty(t.numel() + 16 // es, dtype=t.dtype, device=t.device)
    view = flat[shift_bytes // es:shift_bytes // es + t.numel()].view(t.shape)
    view.copy_(t)
    assert view.data_ptr() % 16 == shift_bytes
    return view


def poison_(t: torch.Tensor) -> None:
    t.view(torch.int16).fill_(POISON)


class Case:
    """One workload instance: inputs on the device, the oracle's layout, a route."""

    def __init__(self, kind, shards, w, lay, route, n_groups, sigma_x, sigma_w, rows_per_shard,
                 topk=None, expert_base=0):
        self.kind = kind
        self.shards_cpu = shards
        self.w_cpu = w
        self.lay = lay
        self.route = route
        self.n_groups = n_groups
        self.sigma_x, self.sigma_w = sigma_x, sigma_w
        self.rows_per_shard = rows_per_shard
        self.K = shards[0].shape[1]
        self.N = w.shape[-2]
        self.shards = [s.to(DEV) for s in shards]
        self.w = w.to(DEV).contiguous()
        self.topk = topk
        self.expert_base = expert_base
        self._oracle_G = None

    @property
    def oracle_G(self):
        if self._oracle_G is None:
            self._oracle_G = O.gather([bits(s) for s in self.shards_cpu], self.lay)
        return self._oracle_G


def dense_case(seed, n_shards, rows, K, N, gather="contiguous", use_explicit=False) -> Case:
    d = W.dense_inputs(seed, n_shards, rows, K, N, gather=gather)
    if gather == "contiguous":
        lay = O.layout_contiguous(n_shards, rows)
        if use_explicit:
            src = torch.arange(rows, dtype=torch.int32).repeat(n_shards, 1)
            dst = (torch.arange(n_shards, dtype=torch.int32)[:, None] * rows + torch.arange(rows, dtype=torch.int32))
            route = fg.route_explicit([rows] * n_shards, src.contiguous().to(DEV), dst.contiguous().to(DEV),
                                      lay.m_pad, rows)
        else:
            route = fg.route_contig(rows)
    else:
        lay = O.layout_permutation(d.perm.numpy(), n_shards, rows)
        src = torch.arange(rows, dtype=torch.int32).repeat(n_shards, 1).contiguous()
        dst = d.perm.reshape(n_shards, rows).contiguous()
        route = fg.route_explicit([rows] * n_shards, src.to(DEV), dst.to(DEV), lay.m_pad, rows)
    return Case("dense", d.shards, d.w, lay, route, 1, d.sigma_x, d.sigma_w, rows)


def holes_case(seed, lens, R, K, N, hole_frac) -> Case:
    """An explicit route whose streams (lengths `lens`, at most R rows per
    shard) land on a seeded random subset of the gathered rows: about
    `hole_frac` of them stay padding, scattered over every row block."""
    S = len(lens)
    d = W.dense_inputs(seed, S, R, K, N)
    rng = np.random.default_rng(seed)
    m = sum(lens)
    m_pad = max(128, -(-int(m / (1 - hole_frac)) // 128) * 128)
    dst_all = rng.permutation(m_pad)[:m]
    src = np.zeros((S, R), np.int32)
    dst = np.zeros((S, R), np.int32)
    src_l, dst_l, j = [], [], 0
    for s in range(S):
        srow = rng.permutation(R)[:lens[s]]
        src[s, :lens[s]] = srow
        dst[s, :lens[s]] = dst_all[j:j + lens[s]]
        src_l.append(srow.astype(np.int64))
        dst_l.append(dst_all[j:j + lens[s]].astype(np.int64))
        j += lens[s]
    lay = O.Layout(src_l, dst_l, m_pad, np.array([0, m_pad]))
    route = fg.route_explicit(lens, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV), m_pad, R)
    return Case("dense", d.shards, d.w, lay, route, 1, d.sigma_x, d.sigma_w, R)


def ep_case(seed, n_shards, tokens, K, N, n_experts=64, topk=8, n_local=8, expert_base=0) -> Case:
    e = W.ep_inputs(seed, n_shards=n_shards, tokens=tokens, K=K, N=N, n_experts=n_experts, topk=topk,
                    n_local=n_local, expert_base=expert_base)
    lay = O.layout_topk(e.topk.numpy(), expert_base, n_local)
    topk_dev = e.topk.to(DEV).contiguous()
    route = fg.route_topk(topk_dev, tokens, expert_base)
    return Case("ep", e.shards, e.w, lay, route, n_local, e.sigma_x, e.sigma_w, tokens, topk=topk_dev,
                expert_base=expert_base)


def make_ctx(case: Case, *, n_comm=0, n_gemm=0, tile_n=0, timeout_ns=0, max_rows=None, split_parts=0,
             split_tiles=0, tile_order=0, combine_wg=0, copy_rows=0, copy_mode=fg.COPY_WORKGROUPS) -> fg.Context:
    max_rows = max_rows or max(int(case.lay.stream_len.max()), case.rows_per_shard)
    cfg = fg.make_config(len(case.shards), max_rows, case.K, case.N, n_groups=case.n_groups,
                         n_comm_wg=n_comm, n_gemm_wg=n_gemm, tile_n=tile_n, timeout_ns=timeout_ns,
                         split_parts=split_parts, split_tiles=split_tiles, tile_order=tile_order,
                         combine_wg=combine_wg, copy_rows=copy_rows, copy_mode=copy_mode)
    return fg.Context(cfg)


def buffers(ctx: fg.Context, case: Case):
    cap = fg.capacity(ctx.cfg)
    gathered = torch.zeros(cap, case.K, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(cap, case.N, dtype=torch.bfloat16, device=DEV)
    return gathered, out


def run_iters(ctx, case, gathered, out, iters, flags=0, poison=True):
    for t in range(iters):
        if poison:
            poison_(gathered)
            poison_(out)
        rc = ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=flags)
        assert rc == fg.OK, fg.strerror(rc)
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st.error_code == 0, (st.error_code, hex(st.error_id))
    return st


def control_plane(ctx: fg.Context, n_shards: int):
    v = ctx.views()
    S, cc, rbc = n_shards, v.chunk_cap, v.rb_cap
    return dict(
        slot=ctx.read_i32(v.slot, S * cc).numpy().reshape(S, cc),
        counter=ctx.read_i32(v.counter, 2 * rbc * fg.COUNTER_STRIDE).numpy().reshape(2, rbc, -1)[:, :, 0].copy(),
        elect=ctx.read_i32(v.elect, 2 * S * cc).numpy().reshape(2, S, cc),
        pub_count=ctx.read_i32(v.pub_count, S * cc).numpy().reshape(S, cc),
        seed=ctx.read_i32(v.seed, rbc).numpy(),
        inv=ctx.read_inverse_map().numpy(),
        stream_len=ctx.read_i32(v.stream_len, S).numpy(),
        group_off=ctx.read_i32(v.group_off, 65).numpy(),
        desc=ctx.read_i32(v.desc, 3).numpy(),
        slab=ctx.read_i32(v.slab, v.rb_cap).numpy(),
        group_slab=ctx.read_i32(v.group_slab, 65).numpy(),
        src_row=ctx.read_i32(v.src_row, S * ctx.cfg.max_rows_per_shard).numpy().reshape(S, -1),
        dst_row=ctx.read_i32(v.dst_row, S * ctx.cfg.max_rows_per_shard).numpy().reshape(S, -1),
        src_of=ctx.read_i32(v.src_of, v.m_pad_cap).numpy(),
        chunk_cap=cc, rb_cap=rbc)


def expected_group_slabs(lay) -> np.ndarray:
    """First slab of each group, then the slab count."""
    counts = [(int(lay.group_off[g + 1]) - int(lay.group_off[g]) + 255) // 256 for g in range(lay.n_groups)]
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def expected_slabs(lay) -> np.ndarray:
    """Row slabs of the compute role for a layout: every group cut into 256-row
    slabs plus a 128-row slab when its size is an odd number of row blocks;
    entry = first row | 1 for a 128-row slab."""
    out = []
    for g in range(lay.n_groups):
        a, b = int(lay.group_off[g]), int(lay.group_off[g + 1])
        for m0 in range(a, b, 256):
            out.append(m0 | (1 if b - m0 == 128 else 0))
    return np.array(out, dtype=np.int64)


def check_route(case: Case, cp) -> None:
    lay = case.lay
    assert np.array_equal(cp["stream_len"], lay.stream_len), "stream lengths"
    for s in range(lay.n_shards):
        n = int(lay.stream_len[s])
        assert np.array_equal(cp["src_row"][s, :n], lay.src_row[s]), f"src_row shard {s}"
        assert np.array_equal(cp["dst_row"][s, :n], lay.dst_row[s]), f"dst_row shard {s}"
        # the per-row source table the in-tile copy reads
        assert np.array_equal(cp["src_of"][np.asarray(lay.dst_row[s], dtype=np.int64)], lay.src_row[s]), \
            f"source row of the gathered rows of shard {s}"
    assert np.array_equal(cp["group_off"][:lay.n_groups + 1], lay.group_off), "group offsets"
    want = expected_slabs(lay)
    assert int(cp["desc"][0]) == lay.m_pad and int(cp["desc"][1]) == len(want), "m_pad / slab count"
    assert np.array_equal(cp["slab"][:len(want)], want), "row slab table"
    assert int(cp["desc"][2]) == lay.n_groups, "group count"
    gs = expected_group_slabs(lay)
    assert np.array_equal(cp["group_slab"][:len(gs)], gs), "first slab of each group"
    assert np.array_equal(cp["seed"][:lay.n_rb], O.seeds(lay)), "padding seeds"
    real = O.real_rows(lay)
    assert np.array_equal(cp["inv"][:lay.m_pad] >= 0, real), "padding rows of the inverse map"


def check_control_plane(case: Case, cp, t: int, verify_iters: int | None) -> None:
    lay = case.lay
    want = O.state_after(lay, t, cp["chunk_cap"])
    n_rb = lay.n_rb
    assert np.array_equal(cp["slot"], want.slot), "slots"
    assert np.array_equal(cp["counter"][:, :n_rb], want.counter), "arrival counters (both parities)"
    assert np.array_equal(cp["elect"], want.elect), "election counts (both parities)"
    if verify_iters is not None:
        exp_pub = (want.pub_count > 0) * verify_iters
        assert np.array_equal(cp["pub_count"], exp_pub), "one publisher per chunk per iteration"


class EveryCallCheck:
    """Checks after every call of a full-size run, on the device: the gathered
    real rows equal the oracle's gather bit for bit and the padding rows still
    hold the poison; the output bits equal the first call's (the summation
    order does not depend on which workgroup runs which item); every output
    element is compared with the fp64 oracle product (computed once) on the
    first call and on the call numbered `last`."""

    def __init__(self, case: Case, last: int, label: str):
        real = O.real_rows(case.lay)
        self.case, self.last, self.label = case, last, label
        self.real_idx = torch.from_numpy(np.nonzero(real)[0]).to(DEV)
        self.pad_idx = torch.from_numpy(np.nonzero(~real)[0]).to(DEV)
        self.G = torch.from_numpy(case.oracle_G.view(np.int16)).to(DEV)
        self.C64 = None
        self.ref = None
        self.calls = 0

    def __call__(self, gathered: torch.Tensor, out: torch.Tensor) -> None:
        case, m_pad = self.case, self.case.lay.m_pad
        self.calls += 1
        t = self.calls
        g = gathered[:m_pad].view(torch.int16)
        assert torch.equal(g.index_select(0, self.real_idx), self.G.index_select(0, self.real_idx)), \
            f"{self.label} call {t}: gathered rows differ from the oracle"
        if self.pad_idx.numel():
            assert bool((g.index_select(0, self.pad_idx) == POISON).all()), f"{self.label} call {t}: padding written"
        o = out[:m_pad].view(torch.int16)
        if t == 1 or t == self.last:
            if self.C64 is None:
                wb = bits(case.w_cpu)
                self.C64 = O.gemm(case.oracle_G, wb if wb.ndim == 3 else wb[None], case.lay)
            real = O.real_rows(case.lay)
            r = O.gemm_check(bits(out[:m_pad]), self.C64, case.K, case.sigma_x, case.sigma_w,
                             np.repeat(real[:, None], case.N, 1))
            assert r["ok"], (self.label, t, r)
        if self.ref is None:
            self.ref = o.clone()
        else:
            assert torch.equal(o, self.ref), f"{self.label} call {t}: output bits differ from call 1"


def check_gathered(case: Case, gathered: torch.Tensor, poisoned: bool) -> None:
    lay = case.lay
    G = bits(gathered[:lay.m_pad])
    real = O.real_rows(lay)
    assert np.array_equal(G[real], case.oracle_G[real]), "gathered real rows bit-exact"
    pad_val = POISON if poisoned else 0
    assert np.all(G[~real] == pad_val), "padding rows never written"


def check_out(case: Case, out: torch.Tensor, rows=None) -> dict:
    lay = case.lay
    real = O.real_rows(lay)
    wb = bits(case.w_cpu)
    if wb.ndim == 2:
        wb = wb[None]
    if rows is None:
        C64 = O.gemm(case.oracle_G, wb, lay)
        ob = bits(out[:lay.m_pad])
        mask = np.repeat(real[:, None], case.N, 1)
    else:
        rows = np.asarray(rows)
        C64 = O.gemm(case.oracle_G, wb, lay, rows=rows)
        ob = bits(out[torch.as_tensor(rows, device=out.device)])
        mask = np.repeat(real[rows][:, None], case.N, 1)
    r = O.gemm_check(ob, C64, case.K, case.sigma_x, case.sigma_w, mask)
    assert r["ok"], r
    return r
