"""Parity of the two-stage dispatch (fg_gather_gemm_staged, through the C ABI)
with the CPU oracle: staged rows, gathered rows, route tables and the control
plane bit-exact; the contraction within the stated tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W
from fg_harness import (DEV, POISON, EveryCallCheck, bits, buffers, check_gathered, check_out, check_route,
                        control_plane, dense_case, ep_case, log, make_ctx, poison_)

pytestmark = pytest.mark.gpu


def _staging(ctx, case, self_shard):
    rs = ctx.cfg.max_rows_per_shard
    return [None if s == self_shard else torch.empty(rs, case.K, dtype=torch.bfloat16, device=DEV)
            for s in range(len(case.shards))]


def _run(case, iters, *, self_shard=-1, flags=0, ctx_kw=None, sample_rows=None, per_call=None):
    ctx = make_ctx(case, **(ctx_kw or {}))
    gathered, out = buffers(ctx, case)
    staging = _staging(ctx, case, self_shard)
    for t in range(iters):
        poison_(gathered)
        poison_(out)
        for x in staging:
            if x is not None:
                poison_(x)
        rc = ctx.gather_gemm_staged(case.shards, case.w, staging, gathered, out, self_shard=self_shard,
                                    route=case.route, flags=flags | fg.CALL_VERIFY)
        assert rc == fg.OK, fg.strerror(rc)
        if per_call is not None:
            torch.cuda.synchronize()
            assert ctx.stats().error_code == 0, t
            per_call(gathered, out)
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st.error_code == 0, (st.error_code, hex(st.error_id))
    lay = case.lay
    cp = control_plane(ctx, len(case.shards))
    check_route(case, cp)
    want = O.state_after_two_stage(lay, iters, cp["chunk_cap"], self_shard)
    assert np.array_equal(cp["slot"], want.slot), "watermark slots"
    assert np.array_equal(cp["counter"][:, :lay.n_rb], want.counter), "arrival counters (both parities)"
    assert np.array_equal(cp["elect"], want.elect), "election counts (both parities)"
    assert np.array_equal(cp["pub_count"], (want.slot > 0) * iters), "one publisher per remote chunk per call"
    remote_chunks = sum(-(-int(lay.stream_len[s]) // lay.chunk_rows) for s in range(lay.n_shards) if s != self_shard)
    assert st.publishes == iters * remote_chunks
    staged = O.push_staging([bits(s) for s in case.shards_cpu], lay, self_shard)
    for s in range(lay.n_shards):
        if s == self_shard:
            continue
        n = int(lay.stream_len[s])
        assert np.array_equal(bits(staging[s][:n]), staged[s]), f"staged rows of shard {s}"
    check_gathered(case, gathered, poisoned=True)
    r = check_out(case, out, rows=sample_rows)
    ctx.close()
    return r


def test_two_stage_tiny_contiguous():
    log("two-stage: tiny contiguous, every shard remote, 3 iterations")
    c = W.CONFIGS["tiny"]
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _run(case, 3)


@pytest.mark.parametrize("self_shard", [0, 2])
def test_two_stage_self_shard_read_directly(self_shard):
    log(f"two-stage: 3 x 100 rows (ragged), shard {self_shard} read directly by the scatter")
    case = dense_case(51, 3, 100, 256, 256)
    _run(case, 2, self_shard=self_shard)


def test_two_stage_permutation_scatter():
    log("two-stage: 4 x 96 rows scattered by a seeded permutation, K=384, N=384 (BN 128)")
    case = dense_case(52, 4, 96, 384, 384, gather="permutation")
    _run(case, 2, ctx_kw=dict(tile_n=128))


def test_two_stage_expert_dispatch():
    log("two-stage: EP top-4 of 16, 4 local, 4 x 200 tokens, self shard 1")
    case = ep_case(53, 4, 200, 256, 256, n_experts=16, topk=4, n_local=4)
    _run(case, 2, self_shard=1)


def test_two_stage_strict_fences():
    log("two-stage with formal fences")
    case = dense_case(54, 2, 130, 256, 256)
    _run(case, 2, flags=fg.CALL_STRICT)


def test_two_stage_comm_only_then_gemm_only():
    log("two-stage roles: push + scatter only, then the compute role only")
    case = dense_case(55, 3, 128, 256, 512)
    ctx = make_ctx(case)
    gathered, out = buffers(ctx, case)
    staging = _staging(ctx, case, -1)
    poison_(out)
    assert ctx.gather_gemm_staged(case.shards, case.w, staging, gathered, out, route=case.route,
                                  flags=fg.CALL_COMM_ONLY) == fg.OK
    torch.cuda.synchronize()
    check_gathered(case, gathered, poisoned=False)
    assert np.all(bits(out) == POISON)
    assert ctx.gather_gemm_staged(case.shards, case.w, staging, gathered, out, route=case.route,
                                  flags=fg.CALL_GEMM_ONLY) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    check_out(case, out)
    ctx.close()


def test_two_stage_tp_full_size():
    c = W.CONFIGS["tp"]
    log(f"two-stage at the TP size: 4 x 2048 rows, K=N=4096, self shard 0, {c['iters']} calls, each checked")
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _run(case, c["iters"], self_shard=0, per_call=EveryCallCheck(case, c["iters"], "tp/two-stage"))


def test_two_stage_dropped_watermark_times_out():
    log("two-stage fault: the watermark of chunk (0,0) is never stored -> the scatter times out, FG_ETIMEOUT")
    case = dense_case(56, 2, 128, 256, 256)
    ctx = make_ctx(case, timeout_ns=20_000_000)
    gathered, out = buffers(ctx, case)
    staging = _staging(ctx, case, -1)
    assert ctx.gather_gemm_staged(case.shards, case.w, staging, gathered, out, route=case.route,
                                  flags=fg.FAULT_DROP_PUBLISH) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == fg.ETIMEOUT
    ctx.close()


def test_two_stage_invalid_arguments():
    log("two-stage: staging pointers required for every remote shard; self shard in range")
    case = dense_case(57, 2, 128, 256, 256)
    ctx = make_ctx(case)
    gathered, out = buffers(ctx, case)
    staging = _staging(ctx, case, 0)
    assert ctx.gather_gemm_staged(case.shards, case.w, staging, gathered, out, self_shard=-1,
                                  route=case.route) == fg.EINVAL
    assert ctx.gather_gemm_staged(case.shards, case.w, staging, gathered, out, self_shard=2,
                                  route=case.route) == fg.EINVAL
    assert ctx.gather_gemm_staged(case.shards, case.w, staging, gathered, out, self_shard=0,
                                  route=case.route) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    ctx.close()


@pytest.mark.parametrize("seed", list(range(520, 528)))
def test_two_stage_random_configuration(seed):
    """Seeded random two-stage dispatches: shard and row counts, K, N, the
    self shard, the copy workgroup count and the route kind drawn per seed;
    staged rows, gathered rows, the control plane and output against the
    oracle."""
    rng = np.random.default_rng(seed)
    kind = ["contig", "perm", "ep"][seed % 3]
    K = int(rng.choice([256, 512, 1024]))
    N = 128 * int(rng.integers(1, 5))
    S = int(rng.integers(1, 7))
    self_shard = int(rng.integers(-1, S))
    n_comm = int(rng.choice([0, 8, 24, 64]))
    if kind == "ep":
        case = ep_case(seed, S, int(rng.integers(8, 300)), K, N, n_experts=16, topk=int(rng.integers(1, 5)),
                       n_local=4)
    else:
        case = dense_case(seed, S, int(rng.integers(1, 600)), K, N,
                          gather="permutation" if kind == "perm" else "contiguous")
    log(f"seed {seed}: two-stage {kind}, {S} shards, K={K} N={N}, self shard {self_shard}, n_comm {n_comm}")
    _run(case, 2, self_shard=self_shard, ctx_kw=dict(n_comm=n_comm))
