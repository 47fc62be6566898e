"""Parity of the in-tile copy (copy_mode 1, fg_plan.hpp) with the CPU oracle.

Every workgroup copies the lead rows first; each compute item copies rows of
a later round's slabs inside its K loop and counts and publishes them. The
results must be those of the oracle, bit for bit for the gathered rows, the
route tables and the whole control plane after every call, and within the
stated tolerance for every output element; and the outputs must equal, bit
for bit, those of the copy-workgroup mode (copy_mode 0) on the same inputs
when neither splits a tile: each whole tile is computed the same way
whichever workgroup copies its rows.

Shapes: only lead rows; several groups of non-lead slabs; a 128-row last slab
with padding rows; seeded permutation routes; a per-item share long enough
that the copy is finished after the K loop; and 16 seeded random shapes with
both tile widths, smaller grids, a grid that is not a multiple of the XCDs
(which falls back to copy workgroups), strict fences and tracing."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from fg_harness import (DEV, POISON, bits, buffers, check_control_plane, check_gathered, check_out, check_route,
                        control_plane, dense_case, log, make_ctx, poison_)

pytestmark = pytest.mark.gpu


def _calls(case, ctx, iters, flags=0):
    gathered, out = buffers(ctx, case)
    want_pubs = O.signal_counts(case.lay)["publishes"]
    ref = None
    t_first = ctx.stats(wait=False).seq + 1     # the context's sequence numbers run on across calls
    for t in range(t_first, t_first + iters):
        poison_(gathered)
        poison_(out)
        rc = ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=flags | fg.CALL_VERIFY)
        assert rc == fg.OK, fg.strerror(rc)
        torch.cuda.synchronize()
        st = ctx.stats()
        assert st.error_code == 0, (t, st.error_code, hex(st.error_id))
        cp = control_plane(ctx, len(case.shards))
        check_route(case, cp)
        check_control_plane(case, cp, t, t)      # every call of the context ran with VERIFY
        assert st.publishes == t * want_pubs and st.expected_publishes == st.publishes
        check_gathered(case, gathered, poisoned=True)
        o = out[:case.lay.m_pad].view(torch.int16).clone()
        if ref is None:
            check_out(case, out)
            ref = o
        else:
            assert torch.equal(o, ref), f"call {t}: output bits differ from call 1"
    return st, ref


SHAPES = [
    # (seed, shards, rows, K, N, gather): what the plan does on it (256 workgroups, 32 per XCD list)
    (601, 4, 512, 1536, 512, "contiguous"),      # 8 slabs: every row is a lead row
    (602, 8, 1000, 1536, 4096, "contiguous"),    # 31.5 slabs, 2 lead slabs per list, 128-row last slab
    (603, 8, 2048, 2048, 8192, "permutation"),   # 64 slabs, 1 lead slab per list, two groups of 4 slabs
    (604, 3, 1777, 2560, 4096, "permutation"),   # ragged: 42 slabs, 5 segments per row, padding rows
    (605, 8, 4096, 1536, 1024, "contiguous"),    # 64 rows per round-0 item: the copy ends after the K loop
]


@pytest.mark.parametrize("seed,S,R,K,N,gather", SHAPES)
def test_tile_copy_matches_oracle_and_copy_workgroups(seed, S, R, K, N, gather):
    log(f"in-tile copy: {S} x {R} rows ({gather}), K={K}, N={N}, 4 calls")
    case = dense_case(seed, S, R, K, N, gather=gather)
    ctx = make_ctx(case, copy_mode=fg.COPY_IN_TILES)
    st, bits_tiles = _calls(case, ctx, 4)
    assert st.copy_in_tiles == 1 and st.lead_rows > 0
    log(f"  lead rows {st.lead_rows} of {case.lay.m_pad}")
    ctx.close()
    ctx2 = make_ctx(case, copy_mode=fg.COPY_WORKGROUPS)
    st2, bits_wg = _calls(case, ctx2, 2)
    assert st2.copy_in_tiles == 0
    ctx2.close()
    if st.tiles_split == 0 and st2.tiles_split == 0:
        # the split-K tail takes the last tiles of each list, which differ between the two tile orders (a
        # split tile sums its k-range partials in another order); with no split every tile is computed alike
        assert torch.equal(bits_tiles, bits_wg), "in-tile copy and copy workgroups give different output bits"
    else:
        log(f"  split tail ({st.tiles_split} / {st2.tiles_split} tiles): both modes checked against the oracle")


def test_tile_copy_strict_fences_same_bits():
    log("in-tile copy with the formal fences: 8 x 2048 rows permuted, K=2048, N=8192")
    case = dense_case(603, 8, 2048, 2048, 8192, gather="permutation")
    ctx = make_ctx(case, copy_mode=fg.COPY_IN_TILES)
    _, b1 = _calls(case, ctx, 2)
    _, b2 = _calls(case, ctx, 2, flags=fg.CALL_STRICT)
    assert torch.equal(b1, b2)
    ctx.close()


def test_tile_copy_trace_stamps_every_block():
    log("in-tile copy with TRACE: every row block has a publish stamp within the kernel's span")
    case = dense_case(602, 8, 1000, 1536, 4096)
    ctx = make_ctx(case, copy_mode=fg.COPY_IN_TILES)
    gathered, out = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route) == fg.OK
    assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=fg.CALL_TRACE) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    tl = ctx.read_timeline()
    wg = tl["wg"]
    t0, t1 = int(wg[:, 0].min()), int(wg[:, 1].max())
    rbt = tl["rb_time"][:case.lay.n_rb]
    assert np.all((rbt >= t0) & (rbt <= t1)), "a row block without a publish stamp from this call"
    check_out(case, out)
    ctx.close()


def test_tile_copy_comm_only_then_gemm_only():
    log("in-tile copy context: COMM_ONLY copies every row; GEMM_ONLY then computes from them")
    case = dense_case(603, 8, 2048, 2048, 8192, gather="permutation")
    ctx = make_ctx(case, copy_mode=fg.COPY_IN_TILES)
    gathered, out = buffers(ctx, case)
    poison_(gathered)
    poison_(out)
    assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route,
                           flags=fg.CALL_COMM_ONLY | fg.CALL_VERIFY) == fg.OK
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st.error_code == 0
    check_gathered(case, gathered, poisoned=True)
    check_control_plane(case, control_plane(ctx, len(case.shards)), 1, 1)
    assert bool((out.view(torch.int16) == POISON).all())
    assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=fg.CALL_GEMM_ONLY) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    check_out(case, out)
    ctx.close()


def test_tile_copy_not_used_where_the_shape_does_not_allow_it():
    log("copy_mode 1 falls back to copy workgroups: K=256 (under three segments per row), watermark gating")
    case = dense_case(606, 4, 256, 256, 512)
    ctx = make_ctx(case, copy_mode=fg.COPY_IN_TILES)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().copy_in_tiles == 0
    ctx.close()
    case = dense_case(602, 8, 1000, 1536, 4096)
    ctx = make_ctx(case, copy_mode=fg.COPY_IN_TILES)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=fg.CALL_GATE_WATERMARK) == fg.OK
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st.error_code == 0 and st.copy_in_tiles == 0
    check_out(case, o)
    ctx.close()


def _draw_tile_case(seed):
    rng = np.random.default_rng(seed)
    kind = ["contiguous", "permutation", "explicit"][seed % 3]
    K = int(rng.choice([1536, 2048, 2560, 3072, 4096]))
    tile_n = int(rng.choice([128, 256]))
    N = tile_n * int(rng.integers(1, 9))
    S = int(rng.integers(1, 9))
    R = int(rng.integers(1, 1500))
    # grid: the default 256, 72 and 136 workgroups, or 201 (not a multiple of the 8 XCDs: copy workgroups instead)
    n_comm, n_gemm = [(0, 0), (0, 0), (8, 64), (8, 128), (1, 200)][int(rng.integers(0, 5))]
    flags = 0
    if rng.random() < 0.3:
        flags |= fg.CALL_STRICT
    if rng.random() < 0.3:
        flags |= fg.CALL_TRACE
    return kind, K, tile_n, N, S, R, n_comm, n_gemm, flags


@pytest.mark.parametrize("seed", range(700, 716))
def test_tile_copy_random_shapes(seed):
    kind, K, tile_n, N, S, R, n_comm, n_gemm, flags = _draw_tile_case(seed)
    log(f"seed {seed}: in-tile copy, {S} x {R} rows ({kind}), K={K}, N={N}, tile_n={tile_n}, "
        f"grid {n_comm}+{n_gemm}, flags={flags:#x}")
    case = dense_case(seed, S, R, K, N, gather="permutation" if kind == "permutation" else "contiguous",
                      use_explicit=kind == "explicit")
    ctx = make_ctx(case, copy_mode=fg.COPY_IN_TILES, tile_n=tile_n, n_comm=n_comm, n_gemm=n_gemm)
    st, _ = _calls(case, ctx, 2, flags=flags)
    log(f"  copied in tiles: {st.copy_in_tiles}, lead rows {st.lead_rows}, whole tiles {st.tiles_whole}, "
        f"split {st.tiles_split} x {st.split_parts}")
    assert st.copy_in_tiles == (0 if n_gemm == 200 else 1), "the in-tile copy where the grid allows it"
    ctx.close()
