"""The two top-k layout paths against the CPU oracle.

A top-k route is laid out by one kernel whose workgroups count, the last one
scans and the others then place, or by two kernels (count + scan, then place;
`FG_CALL_LAYOUT_TWO_PASS`). Each path must give the oracle's tables bit for
bit ("DeepEP FIFO pipeline" dispatch notify stage: per-expert counts fix the
offsets; rows ordered per expert by shard and token): stream lengths, source
and destination rows, group offsets, slabs, seeds, the inverse map, the
source-row table, the first stream entry of each token and the top-k position
of each entry. A token that names one local expert twice is rejected by both
paths."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W
from fg_harness import DEV, Case, buffers, check_control_plane, check_gathered, check_out, check_route, control_plane, \
    ep_case, log, make_ctx, poison_

pytestmark = pytest.mark.gpu

PATHS = [("one_kernel", 0), ("two_pass", fg.CALL_LAYOUT_TWO_PASS)]


def _expected_combine_tables(topk_np, base, n_local):
    picks = O.combine_picks(topk_np, base, n_local)
    S, T, _ = topk_np.shape
    tok_first = np.zeros((S, T + 1), dtype=np.int64)
    src_k = []
    for s in range(S):
        ts = np.array([t for t, _ in picks[s]], dtype=np.int64)
        tok_first[s] = np.searchsorted(ts, np.arange(T + 1), side="left")
        src_k.append(np.array([k for _, k in picks[s]], dtype=np.int64))
    return tok_first, src_k


def _check_tables(ctx, case, topk_np):
    cp = control_plane(ctx, len(case.shards))
    check_route(case, cp)
    v = ctx.views()
    S, T, rs_cap = len(case.shards), case.rows_per_shard, ctx.cfg.max_rows_per_shard
    tf = ctx.read_i32(v.tok_first, S * (rs_cap + 1)).numpy().reshape(S, rs_cap + 1)
    sk = ctx.read_i32(v.src_k, S * rs_cap).numpy().reshape(S, rs_cap)
    wtf, wsk = _expected_combine_tables(topk_np, case.expert_base, case.n_groups)
    assert np.array_equal(tf[:, :T + 1], wtf), "first stream entry of each token"
    for s in range(S):
        assert np.array_equal(sk[s, :len(wsk[s])], wsk[s]), f"top-k position of the entries of shard {s}"
    return cp


def _misaligned(topk: torch.Tensor) -> torch.Tensor:
    """The same lists at an address 4 bytes past a 16-byte boundary."""
    flat = torch.empty(topk.numel() + 1, dtype=torch.int32, device=DEV)
    view = flat[1:].view(topk.shape)
    view.copy_(topk)
    assert view.data_ptr() % 16 == 4
    return view


CASES = [
    # (seed, shards, tokens, K, N, experts, topk, local, base)
    (1003, 8, 1024, 256, 256, 64, 8, 8, 0),    # the EP routing at its full token count
    (1103, 4, 300, 256, 256, 16, 4, 4, 4),     # experts 4..7 local
    (1113, 3, 777, 256, 512, 32, 5, 16, 8),    # ragged token count, 16 local experts
    (1123, 8, 1100, 256, 256, 64, 8, 8, 0),    # tokens not a multiple of the layout's 256-token blocks
    (1133, 1, 64, 256, 256, 8, 8, 8, 0),       # every token picks every local expert
    (1163, 2, 640, 256, 256, 64, 12, 16, 16),  # 12 choices per token
    (1183, 3, 500, 256, 256, 32, 5, 8, 0),     # 5 choices per token
    (1173, 8, 4096, 256, 256, 64, 8, 8, 0),    # 128 layout workgroups
]


@pytest.mark.parametrize("seed,S,T,K,N,E,KK,L,base", CASES)
def test_topk_layout_paths_match_oracle(seed, S, T, K, N, E, KK, L, base):
    log(f"top-k layout paths: {S} x {T} tokens, top-{KK} of {E}, {L} local from {base}")
    case = ep_case(seed, S, T, K, N, n_experts=E, topk=KK, n_local=L, expert_base=base)
    topk_np = case.topk.cpu().numpy()
    ctx = make_ctx(case)
    g, o = buffers(ctx, case)
    t = 0
    for name, flags in PATHS:
        t += 1
        rc = ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=flags | fg.CALL_VERIFY)
        assert rc == fg.OK, (name, fg.strerror(rc))
        torch.cuda.synchronize()
        st = ctx.stats()
        assert st.error_code == 0, (name, st.error_code, hex(st.error_id))
        cp = _check_tables(ctx, case, topk_np)
        check_control_plane(case, cp, t, t)
        check_out(case, o)
    ctx.close()


def test_topk_layout_misaligned_lists():
    log("top-k lists 4 bytes past a 16-byte boundary, both layout paths")
    case = ep_case(1143, 4, 500, 256, 256, n_experts=32, topk=6, n_local=8, expert_base=0)
    topk_np = case.topk.cpu().numpy()
    mis = _misaligned(case.topk)
    route = fg.route_topk(mis, case.rows_per_shard, case.expert_base)
    case2 = Case("ep", case.shards_cpu, case.w_cpu, case.lay, route, case.n_groups, case.sigma_x, case.sigma_w,
                 case.rows_per_shard, topk=mis, expert_base=case.expert_base)
    ctx = make_ctx(case2)
    g, o = buffers(ctx, case2)
    for name, flags in PATHS:
        assert ctx.gather_gemm(case2.shards, case2.w, g, o, route=route, flags=flags | fg.CALL_VERIFY) == fg.OK
        torch.cuda.synchronize()
        assert ctx.stats().error_code == 0, name
        _check_tables(ctx, case2, topk_np)
        check_out(case2, o)
    ctx.close()


@pytest.mark.parametrize("name,flags", PATHS)
def test_topk_duplicate_local_expert_rejected(name, flags):
    log(f"top-k list naming one local expert twice -> FG_EPROTOCOL ({name} layout)")
    case = ep_case(1153, 2, 128, 256, 256, n_experts=16, topk=4, n_local=4)
    bad = case.topk.clone()
    bad[1, 5, 1] = bad[1, 5, 0] = 2          # token 5 of shard 1 picks local expert 2 twice
    route = fg.route_topk(bad, case.rows_per_shard, case.expert_base)
    ctx = make_ctx(case, timeout_ns=20_000_000)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=route, flags=flags) == fg.OK
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st.error_code == fg.EPROTOCOL, (st.error_code, hex(st.error_id))
    assert (st.error_id & 0x7F000000) == 0x48000000 and (st.error_id & 0xFFFFFF) == 1, hex(st.error_id)
    ctx.close()


def test_topk_route_changes_on_one_context():
    """One context, a new top-k routing of the same tokens on every call (three
    routings drawn from different seeds, in the order 1 2 3 1 3 2, the layout
    path alternating): each call's route tables, combine tables, gathered rows
    and output must be the oracle's for its own routing, with one publisher per
    chunk per call."""
    S, T, K, N, E, KK, L = 4, 300, 256, 256, 32, 4, 8
    log(f"top-k route changes on one context: {S} x {T} tokens, top-{KK} of {E}, {L} local, routings 1 2 3 1 3 2")
    base = ep_case(1190, S, T, K, N, n_experts=E, topk=KK, n_local=L)
    cases = {1: base}
    for i, seed in ((2, 1191), (3, 1192)):
        tk = W.ep_inputs(seed, n_shards=S, tokens=T, K=K, N=N, n_experts=E, topk=KK, n_local=L).topk
        lay = O.layout_topk(tk.numpy(), 0, L)
        tk_dev = tk.to(DEV).contiguous()
        cases[i] = Case("ep", base.shards_cpu, base.w_cpu, lay, fg.route_topk(tk_dev, T, 0), L, base.sigma_x,
                        base.sigma_w, T, topk=tk_dev, expert_base=0)
    max_rows = max(int(c.lay.stream_len.max()) for c in cases.values())
    ctx = make_ctx(base, max_rows=max(max_rows, T))
    g, o = buffers(ctx, base)
    expected = 0
    for t, i in enumerate((1, 2, 3, 1, 3, 2)):
        case = cases[i]
        name, flags = PATHS[t % len(PATHS)]
        poison_(g)
        poison_(o)
        rc = ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=flags | fg.CALL_VERIFY)
        assert rc == fg.OK, (i, name, fg.strerror(rc))
        torch.cuda.synchronize()
        st = ctx.stats()
        assert st.error_code == 0, (i, name, st.error_code, hex(st.error_id))
        _check_tables(ctx, case, case.topk.cpu().numpy())
        check_gathered(case, g, poisoned=True)
        check_out(case, o)
        expected += O.signal_counts(case.lay)["publishes"]
        assert st.publishes == expected == st.expected_publishes, (i, name)
    ctx.close()
