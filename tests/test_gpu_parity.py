"""Parity of the HIP path (through the C ABI) with the CPU oracle: bit-exact
gathered rows, route tables and control-plane state; the contraction within the
stated tolerance, element by element (the full workload sizes are in
test_gpu_full_size.py)."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W
from fg_harness import (DEV, POISON, bits, buffers, check_control_plane, check_gathered, check_out,
                        check_route, control_plane, dense_case, ep_case, holes_case, log, make_ctx, poison_,
                        run_iters)

pytestmark = pytest.mark.gpu


def _run_and_check(case, iters, *, flags=0, ctx_kw=None, full_out=True, sample_rows=None, verify=True):
    ctx = make_ctx(case, **(ctx_kw or {}))
    gathered, out = buffers(ctx, case)
    f = flags | (fg.CALL_VERIFY if verify else 0)
    st = run_iters(ctx, case, gathered, out, iters, flags=f)
    cp = control_plane(ctx, len(case.shards))
    check_route(case, cp)
    check_control_plane(case, cp, iters, iters if verify else None)
    check_gathered(case, gathered, poisoned=True)
    r = check_out(case, out, rows=None if full_out else sample_rows)
    if verify:
        assert st.publishes == iters * O.signal_counts(case.lay)["publishes"]
        assert st.expected_publishes == st.publishes
        assert st.timeouts == 0 and st.first_timeout_id == -1
    ctx.close()
    return r


def test_tiny_contiguous_three_iterations():
    log("tiny contiguous: 4 x 256 rows, K=256, N=512, 3 iterations")
    c = W.CONFIGS["tiny"]
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    r = _run_and_check(case, c["iters"])
    log(f"tiny ok: max|d|={r['max_abs']:.3g} tol={r['tol']:.3g}")


def test_tiny_strict_fences_same_result():
    log("tiny contiguous, formal release fences on every signal")
    c = W.CONFIGS["tiny"]
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _run_and_check(case, 3, flags=fg.CALL_STRICT)


def test_ragged_contiguous_padding():
    log("ragged contiguous: 3 x 50 rows (150 real of 256), K=256, N=256")
    case = dense_case(31, 3, 50, 256, 256)
    _run_and_check(case, 4)


def test_ragged_rows_128_tile():
    log("ragged contiguous: 5 x 77 rows (385 real of 512 -> BM 256), K=384, N=384 (BN 128)")
    case = dense_case(32, 5, 77, 384, 384)
    _run_and_check(case, 3, ctx_kw=dict(tile_n=128))


@pytest.mark.parametrize("tile_n", [256, 128])
def test_every_output_element_of_full_tiles_each_call(tile_n):
    """Whole 256-row tiles in every column tile, every output element checked
    after each of five calls: the tile's store path writes each wave's rows
    through LDS in 16-byte pieces, and a wrong row, chunk or half-chunk there
    shows up as scattered elements, which sampled checks would miss."""
    log(f"contiguous: 4 x 512 rows, K=256, N=1024, BN {tile_n}: five calls, full check after each")
    case = dense_case(35, 4, 512, 256, 1024)
    ctx = make_ctx(case, tile_n=tile_n)
    gathered, out = buffers(ctx, case)
    for _ in range(5):
        run_iters(ctx, case, gathered, out, 1, flags=fg.CALL_VERIFY)
        check_gathered(case, gathered, poisoned=True)
        check_out(case, out)
    ctx.close()


def test_ragged_odd_row_blocks():
    log("ragged contiguous: 3 x 100 rows (m_pad 384 -> BM 128 tiles), K=256, N=256")
    case = dense_case(33, 3, 100, 256, 256)
    _run_and_check(case, 3)


@pytest.mark.parametrize("K,copy_rows", [(256, 1), (256, 4), (1024, 1), (1024, 2), (4096, 2), (7168, 1)])
def test_copy_batches_shorter_than_register_set(K, copy_rows):
    """Copy batches of fewer rows than the register set holds (the copy_rows
    setting): the unused register rows must neither load nor store, and every
    row block and chunk still gets its signals."""
    log(f"copy batches of {copy_rows} rows: 3 x 200 rows (ragged), K={K}, N=256, 8 copy workgroups")
    case = dense_case(90 + copy_rows, 3, 200, K, 256)
    _run_and_check(case, 3, ctx_kw=dict(copy_rows=copy_rows, n_comm=8, n_gemm=24))


def test_explicit_route_equals_contiguous():
    log("explicit route carrying the contiguous layout")
    case = dense_case(34, 4, 256, 256, 512, use_explicit=True)
    _run_and_check(case, 3)


def test_permutation_scatter():
    log("permutation scatter: 4 x 200 rows, K=512, N=256")
    case = dense_case(35, 4, 200, 512, 256, gather="permutation")
    _run_and_check(case, 5)


def test_ep_topk_small():
    log("expert dispatch: 8 shards x 64 tokens, top-8 of 64, 8 local experts, K=256, N=256")
    case = ep_case(36, 8, 64, 256, 256)
    r = _run_and_check(case, 3)
    log(f"ep small ok: m_pad={case.lay.m_pad} max|d|={r['max_abs']:.3g}")


@pytest.mark.parametrize("n_shards,rows", [(4, 256), (3, 100), (5, 77)])
def test_contiguous_watermark_gating(n_shards, rows):
    log(f"contiguous {n_shards} x {rows} rows, the GEMM gated on the 64-row chunk watermarks")
    case = dense_case(70 + rows, n_shards, rows, 256, 256)
    _run_and_check(case, 3, flags=fg.CALL_GATE_WATERMARK)


def test_watermark_gating_full_tp():
    log("TP size, GEMM gated on chunk watermarks: 4 x 2048 rows, K=N=4096, 3 calls, every output element")
    c = W.CONFIGS["tp"]
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _run_and_check(case, 3, flags=fg.CALL_GATE_WATERMARK)


def test_watermark_gating_needs_contiguous_route():
    log("watermark gating is refused for other routes")
    case = dense_case(75, 2, 128, 256, 256, gather="permutation")
    ctx = make_ctx(case)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=fg.CALL_GATE_WATERMARK) == fg.EINVAL
    ctx.close()


def test_ep_topk_two_pass_layout():
    log("EP top-k with the layout as two kernels (count + scan, then place): same tables and results")
    case = ep_case(1103, 4, 300, 256, 256, n_experts=16, topk=4, n_local=4, expert_base=4)
    _run_and_check(case, 3, flags=fg.CALL_LAYOUT_TWO_PASS)


def test_ep_topk_other_base():
    log("expert dispatch: local experts 24..31, 4 shards x 200 tokens")
    case = ep_case(37, 4, 200, 256, 256, expert_base=24)
    _run_and_check(case, 3)


def test_fifty_iterations_poisoned():
    log("tiny contiguous, 50 iterations, NaN poison before each")
    c = W.CONFIGS["tiny"]
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _run_and_check(case, 50)


def test_comm_only_and_gemm_only_roles():
    log("role-only modes: comm only then gemm only")
    case = dense_case(38, 4, 256, 256, 512)
    ctx = make_ctx(case)
    gathered, out = buffers(ctx, case)
    poison_(gathered)
    poison_(out)
    assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=fg.CALL_COMM_ONLY) == 0
    torch.cuda.synchronize()
    check_gathered(case, gathered, poisoned=True)
    assert np.all(bits(out) == POISON), "comm-only must not write the output"
    cp = control_plane(ctx, 4)
    assert np.all(cp["counter"][1, :case.lay.n_rb] == 128)
    assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=fg.CALL_GEMM_ONLY) == 0
    torch.cuda.synchronize()
    check_out(case, out)
    assert ctx.stats().error_code == 0
    ctx.close()


def test_zero_length_shard_streams():
    log("explicit route with empty and ragged shard streams")
    torch.manual_seed(0)
    S, R, K, N = 4, 96, 256, 256
    d = W.dense_inputs(39, S, R, K, N)
    lens = [0, 96, 17, 65]
    rng = np.random.default_rng(39)
    m = sum(lens)
    m_pad = -(-m // 128) * 128
    dst_all = rng.permutation(m_pad)[:m]
    src = np.zeros((S, R), np.int32)
    dst = np.zeros((S, R), np.int32)
    j = 0
    src_l, dst_l = [], []
    for s in range(S):
        srow = rng.permutation(R)[:lens[s]]
        src[s, :lens[s]] = srow
        dst[s, :lens[s]] = dst_all[j:j + lens[s]]
        src_l.append(srow.astype(np.int64))
        dst_l.append(dst_all[j:j + lens[s]].astype(np.int64))
        j += lens[s]
    lay = O.Layout(src_l, dst_l, m_pad, np.array([0, m_pad]))
    route = fg.route_explicit(lens, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV), m_pad, R)
    from fg_harness import Case
    case = Case("dense", d.shards, d.w, lay, route, 1, d.sigma_x, d.sigma_w, R)
    _run_and_check(case, 3)


@pytest.mark.parametrize("seed,lens,R,hole_frac", [
    (4101, [3000, 2500, 2999, 1], 3000, 0.10),   # 12,000 stream slots: 47 layout workgroups
    (4102, [4096, 0, 4096, 333], 4096, 0.30),    # a third of the gathered rows are padding
])
def test_explicit_route_scattered_padding(seed, lens, R, hole_frac):
    """An explicit route whose padding rows are scattered over the whole
    gathered buffer, laid out by many workgroups: every row block's real-row
    count is assembled from the adds of several workgroups, and the seeds,
    counters, gathered rows and output must match the oracle."""
    log(f"explicit route, {sum(lens)} rows over {len(lens)} shards, {hole_frac:.0%} padding")
    case = holes_case(seed, lens, R, 256, 256, hole_frac)
    assert int(np.count_nonzero(O.seeds(case.lay))) > case.lay.m_pad // 128 // 2, "padding in most row blocks"
    _run_and_check(case, 3)


def test_route_changes_on_one_context():
    """One context, the route switched between calls: contiguous (A), a
    permutation (B) and an explicit route with scattered padding and another
    padded size (C), in the order A B C A C B B A. Every call must give the
    oracle's route tables, gathered rows and output for the route it was
    given: entries of an earlier route read as padding (versioned inverse
    map), a cached contiguous layout is rebuilt after another route, and each
    layout arms the parity its call uses; one publisher per chunk per call."""
    seed, S, R, K, N = 4201, 4, 500, 512, 256
    log(f"route changes on one context: {S} x {R} rows, K={K}, N={N}, routes A B C A C B B A")
    cases = {"A": dense_case(seed, S, R, K, N),
             "B": dense_case(seed, S, R, K, N, gather="permutation"),
             "C": holes_case(seed, [R // 2, R // 3, R, 7], R, K, N, 0.3)}
    assert cases["C"].lay.m_pad != cases["A"].lay.m_pad
    ctx = make_ctx(cases["A"])
    gathered, out = buffers(ctx, cases["A"])
    expected = 0
    for name in "ABCACBBA":
        case = cases[name]
        poison_(gathered)
        poison_(out)
        assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=fg.CALL_VERIFY) == fg.OK
        torch.cuda.synchronize()
        st = ctx.stats()
        assert st.error_code == 0, (name, st.error_code, hex(st.error_id))
        cp = control_plane(ctx, S)
        check_route(case, cp)
        check_gathered(case, gathered, poisoned=True)
        check_out(case, out)
        expected += O.signal_counts(case.lay)["publishes"]
        assert st.publishes == expected == st.expected_publishes, name
    ctx.close()


def test_two_contexts_share_one_stream():
    """Two contexts of different shapes used alternately on one stream (A B A B
    A B): each call matches the oracle for its own context and inputs, and each
    context's control plane stays exact (its sequence runs on its own)."""
    log("two contexts on one stream, alternating calls")
    ca = dense_case(4301, 4, 300, 512, 256, gather="permutation")
    cb = dense_case(4302, 2, 640, 256, 512)
    xa, xb = make_ctx(ca), make_ctx(cb)
    ga, oa = buffers(xa, ca)
    gb, ob = buffers(xb, cb)
    ta = tb = 0
    for i in range(6):
        case, ctx, g, o = (ca, xa, ga, oa) if i % 2 == 0 else (cb, xb, gb, ob)
        poison_(g)
        poison_(o)
        assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=fg.CALL_VERIFY) == fg.OK
        torch.cuda.synchronize()
        st = ctx.stats()
        assert st.error_code == 0, (i, st.error_code, hex(st.error_id))
        if i % 2 == 0:
            ta += 1
            t = ta
        else:
            tb += 1
            t = tb
        cp = control_plane(ctx, len(case.shards))
        check_route(case, cp)
        check_control_plane(case, cp, t, t)
        check_gathered(case, g, poisoned=True)
        check_out(case, o)
    xa.close()
    xb.close()
