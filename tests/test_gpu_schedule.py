"""The compute schedule: ticket-dispatched tiles, communication workgroups that
join the compute role, and the split-K tail (tail tiles cut into k-ranges whose
fp32 partials are summed in a fixed order). Every case is checked against the
CPU oracle element by element; the split path must also be deterministic."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from fg_harness import (bits, buffers, check_control_plane, check_gathered, check_out, check_route, control_plane,
                        dense_case, ep_case, expected_group_slabs, expected_slabs, log, make_ctx, run_iters)

pytestmark = pytest.mark.gpu


def _check(case, ctx, iters, flags=fg.CALL_VERIFY):
    gathered, out = buffers(ctx, case)
    st = run_iters(ctx, case, gathered, out, iters, flags=flags)
    cp = control_plane(ctx, len(case.shards))
    check_route(case, cp)
    check_control_plane(case, cp, iters, iters if flags & fg.CALL_VERIFY else None)
    check_gathered(case, gathered, poisoned=True)
    r = check_out(case, out)
    return st, out, r


def _schedule(case, grid, split_parts, split_tiles, bn=256, tile_order=0):
    """(whole tiles, split tiles, parts per split tile) of the documented
    schedule. Lists: 8 (XCD-grouped, when the grid is a multiple of 8 and
    tile_order = 0) or 1. Default: list x splits its leftover len_x mod
    (workgroups per list) tiles into P = min(split_parts, K / 128, grid / R)
    parts; with split_tiles given, split_tiles / lists tiles of every list,
    P = min(split_parts, K / 128, grid)."""
    n_tn = case.N // bn
    n_slabs = len(expected_slabs(case.lay))
    n_tiles = n_slabs * n_tn
    nx = 8 if (tile_order == 0 and grid % 8 == 0) else 1
    per_list = grid // nx
    if nx == 8 and case.lay.n_groups == 8:      # list x = the slabs of group x
        gs = expected_group_slabs(case.lay)
        lens = [int(gs[x + 1] - gs[x]) * n_tn for x in range(8)]
    else:
        lens = [((n_slabs - x + nx - 1) // nx) * n_tn for x in range(nx)]
    min_len = min(lens) if split_tiles else 0
    r = [min(split_tiles // nx, min_len)] * nx if split_tiles else [l % per_list for l in lens]
    R, P = sum(r), 1
    if R > 0 and n_tiles > grid:
        P = min(split_parts, case.K // 128, grid if split_tiles else grid // R)
    if P <= 1:
        R, P = 0, 1
    return n_tiles - R, R, P


@pytest.mark.parametrize("P,split_tiles", [(2, 4), (3, 4), (4, 4), (8, 4), (4, 32), (3, 5)])
def test_split_tail_matches_oracle(P, split_tiles):
    log(f"split-K tail: 4 x 512 rows (32 tiles), K=N=1024, grid 2+5, P={P}, split_tiles={split_tiles}")
    case = dense_case(51, 4, 512, 1024, 1024)
    ctx = make_ctx(case, n_comm=2, n_gemm=5, split_parts=P, split_tiles=split_tiles)
    st, _, r = _check(case, ctx, 3)
    assert (st.tiles_whole, st.tiles_split, st.split_parts) == _schedule(case, 7, P, split_tiles)
    assert st.tiles_split > 0
    log(f"split ok: whole={st.tiles_whole} split={st.tiles_split} P={st.split_parts} max|d|={r['max_abs']:.3g}")
    ctx.close()


@pytest.mark.parametrize("rows,N,n_comm,n_gemm", [(640, 768, 2, 14), (896, 768, 4, 12), (512, 1280, 1, 2)])
def test_default_split_of_leftover_tiles(rows, N, n_comm, n_gemm):
    grid = n_comm + n_gemm
    log(f"default split of each list's leftover tiles: 4 x {rows} rows, K=1024, N={N}, grid {n_comm}+{n_gemm}")
    case = dense_case(80 + rows // 128, 4, rows, 1024, N)
    ctx = make_ctx(case, n_comm=n_comm, n_gemm=n_gemm, split_parts=8)
    st, _, _ = _check(case, ctx, 3)
    want = _schedule(case, grid, 8, 0)
    assert (st.tiles_whole, st.tiles_split, st.split_parts) == want
    assert want[1] > 0
    ctx.close()


def test_split_tail_is_deterministic():
    log("split-K tail: outputs of repeated calls are bit-identical")
    case = dense_case(52, 4, 512, 1024, 1024)
    ctx = make_ctx(case, n_comm=2, n_gemm=5, split_parts=4, split_tiles=32)
    gathered, out = buffers(ctx, case)
    outs = []
    for _ in range(3):
        run_iters(ctx, case, gathered, out, 1, flags=0)
        outs.append(bits(out[:case.lay.m_pad]).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    check_out(case, out)
    ctx.close()


def test_split_parts_capped_by_k():
    log("split-K tail with fewer k-iteration pairs than parts: K=256 -> 2 parts")
    case = dense_case(53, 4, 512, 256, 1024)
    ctx = make_ctx(case, n_comm=2, n_gemm=5, split_parts=4, split_tiles=32)
    st, _, _ = _check(case, ctx, 2)
    assert (st.tiles_whole, st.tiles_split, st.split_parts) == _schedule(case, 7, 4, 32)
    assert st.split_parts == 2 and st.tiles_split > 0
    ctx.close()


def test_no_split_whole_tiles_only():
    log("split-K off (split_parts=1): whole tiles only")
    case = dense_case(54, 4, 512, 1024, 1024)
    ctx = make_ctx(case, n_comm=2, n_gemm=5, split_parts=1)
    st, _, _ = _check(case, ctx, 2)
    assert st.tiles_split == 0 and st.tiles_whole == 32
    ctx.close()


def test_split_tail_tile_n_128_ragged():
    log("split-K tail, BN 128, ragged rows: 5 x 77 rows, K=512, N=384")
    case = dense_case(55, 5, 77, 512, 384)
    ctx = make_ctx(case, n_comm=1, n_gemm=3, tile_n=128, split_parts=4, split_tiles=6)
    st, _, _ = _check(case, ctx, 3)
    assert st.tiles_split > 0
    ctx.close()


def test_split_tail_expert_groups():
    log("split-K tail on grouped expert tiles: 8 shards x 64 tokens, grid 1+3")
    case = ep_case(56, 8, 64, 512, 256)
    n_tiles = len(expected_slabs(case.lay))
    grid = next(g for g in (4, 3, 5, 6, 7) if n_tiles > g and n_tiles % g)
    ctx = make_ctx(case, n_comm=1, n_gemm=grid - 1, split_parts=4, split_tiles=8)
    st, _, _ = _check(case, ctx, 3)
    assert (st.tiles_whole, st.tiles_split, st.split_parts) == _schedule(case, grid, 4, 8)
    assert st.tiles_split > 0
    ctx.close()


def test_strict_split_tail():
    log("split-K tail with formal release fences")
    case = dense_case(57, 4, 512, 1024, 1024)
    ctx = make_ctx(case, n_comm=2, n_gemm=5, split_parts=4, split_tiles=8)
    _check(case, ctx, 2, flags=fg.CALL_VERIFY | fg.CALL_STRICT)
    ctx.close()


def test_comm_workgroups_join_compute():
    log("one communication workgroup, one compute workgroup: the comm workgroup takes tiles after its rows")
    case = dense_case(58, 2, 512, 512, 512)
    ctx = make_ctx(case, n_comm=1, n_gemm=1, split_parts=1)
    st, _, _ = _check(case, ctx, 2)
    assert st.tiles_whole == (1024 // 256) * (512 // 256)
    ctx.close()


@pytest.mark.parametrize("rows,n_comm,n_gemm,split_tiles", [(1024, 2, 14, 0), (1024, 1, 7, 0), (640, 2, 14, 16),
                                                             (640, 2, 14, 0), (896, 4, 12, 24), (1024, 2, 14, 16)])
def test_xcd_grouped_lists(rows, n_comm, n_gemm, split_tiles):
    grid = n_comm + n_gemm
    log(f"XCD-grouped lists: 4 x {rows} rows, K=512, N=1024, grid {n_comm}+{n_gemm}, split_tiles={split_tiles}")
    case = dense_case(60 + rows // 128, 4, rows, 512, 1024)
    ctx = make_ctx(case, n_comm=n_comm, n_gemm=n_gemm, split_parts=4, split_tiles=split_tiles)
    st, _, _ = _check(case, ctx, 3)
    assert (st.tiles_whole, st.tiles_split, st.split_parts) == _schedule(case, grid, 4, split_tiles)
    ctx.close()


def test_xcd_grouped_expert_groups():
    log("XCD-grouped lists on grouped expert tiles: 8 shards x 128 tokens, grid 2+14")
    case = ep_case(70, 8, 128, 512, 512)
    ctx = make_ctx(case, n_comm=2, n_gemm=14, split_parts=4, split_tiles=16)
    st, _, _ = _check(case, ctx, 3)
    assert (st.tiles_whole, st.tiles_split, st.split_parts) == _schedule(case, 16, 4, 16)
    ctx.close()


def test_single_list_order_at_full_grid():
    log("one row-block-major list (tile_order=1) on the default grid: TP-like 4 x 512 rows, K=N=1024")
    case = dense_case(71, 4, 512, 1024, 1024)
    cfg_ctx = make_ctx(case, tile_order=1)
    _check(case, cfg_ctx, 2)
    cfg_ctx.close()
