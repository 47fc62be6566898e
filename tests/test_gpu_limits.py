"""Parity at the limits of the configuration: the most shards and expert
groups the interface allows, the largest K, one row per shard, a full top-64
list, and the combine on such routes."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from fg_harness import (DEV, buffers, check_control_plane, check_gathered, check_out, check_route, control_plane,
                        dense_case, ep_case, log, make_ctx, run_iters)

pytestmark = pytest.mark.gpu


def _run(case, iters=2, **ctx_kw):
    ctx = make_ctx(case, **ctx_kw)
    gathered, out = buffers(ctx, case)
    st = run_iters(ctx, case, gathered, out, iters, flags=fg.CALL_VERIFY)
    cp = control_plane(ctx, len(case.shards))
    check_route(case, cp)
    check_control_plane(case, cp, iters, iters)
    check_gathered(case, gathered, poisoned=True)
    r = check_out(case, out)
    assert st.publishes == iters * O.signal_counts(case.lay)["publishes"]
    return ctx, r


def test_most_shards():
    log(f"contiguous: {fg.MAX_SHARDS} shards x 16 rows (the most shards), K=128, N=128")
    case = dense_case(81, fg.MAX_SHARDS, 16, 128, 128)
    ctx, _ = _run(case)
    ctx.close()


def test_one_row_per_shard():
    log("contiguous: 4 shards x 1 row (a 128-row block of 4 real rows and 124 padding rows)")
    case = dense_case(82, 4, 1, 256, 256)
    ctx, _ = _run(case, iters=3)
    ctx.close()


def test_largest_k():
    log("contiguous: 2 x 64 rows, K=16384 (the largest K), N=256")
    case = dense_case(83, 2, 64, 16384, 256)
    ctx, r = _run(case)
    log(f"max|d|={r['max_abs']:.3g} tol={r['tol']:.3g}")
    ctx.close()


def test_most_expert_groups():
    log(f"EP: {fg.MAX_GROUPS} local experts (the most groups), top-8 of 64, 8 x 64 tokens: "
        "every group is one 128-row slab")
    case = ep_case(84, 8, 64, 128, 256, n_experts=64, topk=8, n_local=fg.MAX_GROUPS)
    ctx, _ = _run(case)
    ctx.close()


def test_full_top64_list_and_combine():
    log("EP: every token picks all 64 experts, all local (top-k = 64), then the combine over 64 picks per token")
    case = ep_case(85, 2, 40, 128, 128, n_experts=64, topk=64, n_local=64)
    ctx, _ = _run(case)
    from sync_protocols_amd import workloads as W
    from fg_harness import bits, poison_
    S, T, KK, N = 2, 40, 64, case.N
    out = torch.zeros(fg.capacity(ctx.cfg), N, dtype=torch.bfloat16, device=DEV)
    out_cpu, w_cpu = W.combine_inputs(86, out.shape[0], N, S, T, KK)
    out.copy_(out_cpu.to(DEV))
    staging = [torch.empty(ctx.cfg.max_rows_per_shard, N, dtype=torch.bfloat16, device=DEV) for _ in range(S)]
    y = [torch.empty(T, N, dtype=torch.bfloat16, device=DEV) for _ in range(S)]
    for t in staging + y:
        poison_(t)
    assert ctx.combine(out, w_cpu.to(DEV), staging, y) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    topk = case.topk.cpu().numpy()
    ob = bits(out_cpu)
    y64 = O.combine(ob, w_cpu.numpy(), topk, 0, 64, case.lay)
    tol = O.combine_tolerance(ob, w_cpu.numpy(), topk, 0, 64, case.lay)
    for s in range(S):
        assert np.all(np.abs(O.bf16_to_f64(bits(y[s])) - y64[s]) <= tol[s])
    ctx.close()


def test_combine_most_shards():
    log(f"combine on {fg.MAX_SHARDS} shards x 24 tokens, top-2 of 8 experts, 8 local")
    case = ep_case(87, fg.MAX_SHARDS, 24, 128, 256, n_experts=8, topk=2, n_local=8)
    ctx, _ = _run(case, iters=1)
    from sync_protocols_amd import workloads as W
    from fg_harness import bits, poison_
    S, T, KK, N = fg.MAX_SHARDS, 24, 2, case.N
    out = torch.zeros(fg.capacity(ctx.cfg), N, dtype=torch.bfloat16, device=DEV)
    out_cpu, w_cpu = W.combine_inputs(88, out.shape[0], N, S, T, KK)
    out.copy_(out_cpu.to(DEV))
    staging = [torch.empty(ctx.cfg.max_rows_per_shard, N, dtype=torch.bfloat16, device=DEV) for _ in range(S)]
    y = [torch.empty(T, N, dtype=torch.bfloat16, device=DEV) for _ in range(S)]
    for t in staging + y:
        poison_(t)
    assert ctx.combine(out, w_cpu.to(DEV), staging, y) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    topk = case.topk.cpu().numpy()
    ob = bits(out_cpu)
    y64 = O.combine(ob, w_cpu.numpy(), topk, 0, 8, case.lay)
    tol = O.combine_tolerance(ob, w_cpu.numpy(), topk, 0, 8, case.lay)
    for s in range(S):
        assert np.all(np.abs(O.bf16_to_f64(bits(y[s])) - y64[s]) <= tol[s])
    ctx.close()
