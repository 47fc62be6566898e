"""Parity of the dispatch through bounded FIFO rings (fg_gather_gemm_ring,
through the C ABI) with the CPU oracle: gathered rows, counters and the ring
tail / head words bit-exact, the contraction within the stated tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W
from fg_harness import (DEV, EveryCallCheck, bits, buffers, check_gathered, check_out, check_route, control_plane,
                        dense_case, ep_case, log, make_ctx, poison_)

pytestmark = pytest.mark.gpu

TAIL_STRIDE = 32


def _ring_state(ctx, rings):
    v = ctx.views()
    cap = v.ring_cap
    t = ctx.read_i32(v.ring_tail, 2 * cap * TAIL_STRIDE * 2).numpy().view(np.int64).reshape(2, cap, TAIL_STRIDE)
    h = ctx.read_i32(v.ring_head, 2 * cap * fg.COUNTER_STRIDE).numpy().reshape(2, cap, fg.COUNTER_STRIDE)
    return t[:, :rings, 0].copy(), h[:, :rings, 0].copy()


def _run(case, iters, *, n_channels, ring_chunks, self_shard=-1, flags=0, ctx_kw=None, sample_rows=None,
         per_call=None):
    ctx = make_ctx(case, **(ctx_kw or {}))
    gathered, out = buffers(ctx, case)
    nbytes = fg.ring_bytes(ctx.cfg, n_channels, ring_chunks)
    ring = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=DEV)
    for t in range(iters):
        poison_(gathered)
        poison_(out)
        poison_(ring)
        rc = ctx.gather_gemm_ring(case.shards, case.w, ring, gathered, out, n_channels=n_channels,
                                  ring_chunks=ring_chunks, self_shard=self_shard, route=case.route, flags=flags)
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
    want = O.state_after(lay, iters, cp["chunk_cap"])
    assert np.array_equal(cp["counter"][:, :lay.n_rb], want.counter), "arrival counters (both parities)"
    tail, head = _ring_state(ctx, len(case.shards) * n_channels)
    wt, wh = O.ring_state_after(lay, n_channels, iters, self_shard)
    assert np.array_equal(tail, wt), "ring tails (both parities)"
    assert np.array_equal(head, wh), "ring heads (both parities)"
    check_gathered(case, gathered, poisoned=True)
    r = check_out(case, out, rows=sample_rows)
    ctx.close()
    return r


@pytest.mark.parametrize("n_channels,ring_chunks", [(1, 1), (2, 2), (3, 1)])
def test_ring_tiny_contiguous(n_channels, ring_chunks):
    log(f"ring: tiny contiguous, {n_channels} rings per shard of {ring_chunks} slots, 3 iterations")
    c = W.CONFIGS["tiny"]
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _run(case, 3, n_channels=n_channels, ring_chunks=ring_chunks)


@pytest.mark.parametrize("self_shard", [0, 2])
def test_ring_self_shard_read_directly(self_shard):
    log(f"ring: 3 x 300 rows (ragged), shard {self_shard} read directly, 4 rings per shard of 2 slots")
    case = dense_case(61, 3, 300, 256, 256)
    _run(case, 2, n_channels=4, ring_chunks=2, self_shard=self_shard)


def test_ring_permutation_scatter():
    log("ring: 4 x 200 rows scattered by a seeded permutation, 2 rings per shard of 1 slot")
    case = dense_case(62, 4, 200, 384, 384, gather="permutation")
    _run(case, 2, n_channels=2, ring_chunks=1, ctx_kw=dict(tile_n=128))


def test_ring_expert_dispatch():
    log("ring: EP top-4 of 16, 4 local, 4 x 300 tokens, self shard 3, 3 rings per shard of 2 slots")
    case = ep_case(63, 4, 300, 256, 256, n_experts=16, topk=4, n_local=4)
    _run(case, 2, n_channels=3, ring_chunks=2, self_shard=3)


def test_ring_strict_fences():
    log("ring with formal fences")
    case = dense_case(64, 2, 260, 256, 256)
    _run(case, 2, n_channels=2, ring_chunks=1, flags=fg.CALL_STRICT)


def test_ring_tp_full_size():
    c = W.CONFIGS["tp"]
    log(f"ring at the TP size: 4 x 2048 rows, K=N=4096, 8 rings per shard of 2 slots (1/4 of the streams), "
        f"self shard 0, {c['iters']} calls, each checked")
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _run(case, c["iters"], n_channels=8, ring_chunks=2, self_shard=0,
         per_call=EveryCallCheck(case, c["iters"], "tp/ring"))


def test_ring_arguments():
    log("ring: size helper, rings within the copy workgroups, slots >= 1")
    case = dense_case(65, 2, 128, 256, 256)
    ctx = make_ctx(case)
    assert fg.ring_bytes(ctx.cfg, 3, 2) == 2 * 3 * 2 * 64 * 256 * 2
    gathered, out = buffers(ctx, case)
    ring = torch.empty(fg.ring_bytes(ctx.cfg, 1, 1) // 2, dtype=torch.bfloat16, device=DEV)
    cap = ctx.views().ring_cap
    assert ctx.gather_gemm_ring(case.shards, case.w, ring, gathered, out, n_channels=cap // 2 + 1, ring_chunks=1,
                                route=case.route) == fg.EINVAL
    assert ctx.gather_gemm_ring(case.shards, case.w, ring, gathered, out, n_channels=1, ring_chunks=0,
                                route=case.route) == fg.EINVAL
    assert ctx.gather_gemm_ring(case.shards, case.w, ring, gathered, out, n_channels=1, ring_chunks=1,
                                self_shard=2, route=case.route) == fg.EINVAL
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    ctx.close()


def _draw_ring(seed):
    rng = np.random.default_rng(seed)
    kind = ["contig", "perm", "ep"][seed % 3]
    K = int(rng.choice([256, 512, 1024]))
    N = 128 * int(rng.integers(1, 5))
    S = int(rng.integers(1, 7))
    n_channels = int(rng.integers(1, 4))
    ring_chunks = int(rng.integers(1, 4))
    self_shard = int(rng.integers(-1, S))
    n_comm = 8 * int(np.ceil(2 * S * n_channels / 8)) + 8 * int(rng.integers(0, 3))   # every ring served
    return kind, K, N, S, n_channels, ring_chunks, self_shard, n_comm, rng


@pytest.mark.parametrize("seed", list(range(500, 508)))
def test_ring_random_configuration(seed):
    """Seeded random ring dispatches: shard, row and ring counts, slots per
    ring, the self shard and the route kind drawn per seed; gathered rows,
    counters, ring words and output against the oracle."""
    kind, K, N, S, n_channels, ring_chunks, self_shard, n_comm, rng = _draw_ring(seed)
    if kind == "ep":
        case = ep_case(seed, S, int(rng.integers(8, 300)), K, N, n_experts=16, topk=int(rng.integers(1, 5)),
                       n_local=4)
    else:
        case = dense_case(seed, S, int(rng.integers(1, 600)), K, N,
                          gather="permutation" if kind == "perm" else "contiguous")
    log(f"seed {seed}: ring {kind}, {S} shards, K={K} N={N}, {n_channels} rings x {ring_chunks} slots per shard, "
        f"self shard {self_shard}, {n_comm} copy workgroups")
    _run(case, 2, n_channels=n_channels, ring_chunks=ring_chunks, self_shard=self_shard,
         ctx_kw=dict(n_comm=n_comm))
