"""Parity of the combine entry point (fg_combine, through the C ABI) with the
CPU oracle: staging rows and the combine control plane bit-exact, the weighted
top-k sums within the stated tolerance, element by element.

The expert outputs fed to the combine are seeded synthetic rows written into
the output buffer after the dispatch call that builds the route, so that no
oracle input comes from the HIP path."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W
from fg_harness import DEV, Case, bits, buffers, ep_case, log, make_ctx, misaligned_like, poison_

pytestmark = pytest.mark.gpu


def _manual_case(seed, topk_np, K, N, n_local, expert_base=0):
    S, T, KK = topk_np.shape
    e = W.ep_inputs(seed, n_shards=S, tokens=T, K=K, N=N, n_experts=max(n_local + expert_base, KK), topk=KK,
                    n_local=n_local, expert_base=expert_base)
    topk_t = torch.from_numpy(topk_np.astype(np.int32)).contiguous()
    lay = O.layout_topk(topk_np, expert_base, n_local)
    topk_dev = topk_t.to(DEV)
    route = fg.route_topk(topk_dev, T, expert_base)
    return Case("ep", e.shards, e.w, lay, route, n_local, e.sigma_x, e.sigma_w, T, topk=topk_dev,
                expert_base=expert_base)


def _expected_tables(lay, topk_np, base, n_local, rs_cap):
    picks = O.combine_picks(topk_np, base, n_local)
    S, T, _ = topk_np.shape
    tok_first = np.zeros((S, T + 1), dtype=np.int64)
    src_k = []
    for s in range(S):
        ts = np.array([t for t, _ in picks[s]], dtype=np.int64)
        tok_first[s] = np.searchsorted(ts, np.arange(T + 1), side="left")
        src_k.append(np.array([k for _, k in picks[s]], dtype=np.int64))
    return tok_first, src_k


class CombineRun:
    def __init__(self, case, *, ctx_kw=None, timeout_ns=0):
        kw = dict(ctx_kw or {})
        if timeout_ns:
            kw["timeout_ns"] = timeout_ns
        self.case = case
        self.ctx = make_ctx(case, **kw)
        self.gathered, self.out = buffers(self.ctx, case)
        S, T = len(case.shards), case.rows_per_shard
        self.S, self.T, self.KK = S, T, int(case.topk.shape[2])
        rs_cap = self.ctx.cfg.max_rows_per_shard
        self.staging = [torch.empty(rs_cap, case.N, dtype=torch.bfloat16, device=DEV) for _ in range(S)]
        self.y = [torch.empty(T, case.N, dtype=torch.bfloat16, device=DEV) for _ in range(S)]
        self.topk_np = case.topk.cpu().numpy()

    def dispatch(self):
        rc = self.ctx.gather_gemm(self.case.shards, self.case.w, self.gathered, self.out, route=self.case.route)
        assert rc == fg.OK, fg.strerror(rc)

    def combine(self, seed, flags=0, poison=True, check=True):
        out_cpu, w_cpu = W.combine_inputs(seed, self.out.shape[0], self.case.N, self.S, self.T, self.KK)
        self.out.copy_(out_cpu.to(DEV))
        wd = w_cpu.to(DEV)
        if poison:
            for t in self.staging + self.y:
                poison_(t)
        rc = self.ctx.combine(self.out, wd, self.staging, self.y, flags=flags)
        assert rc == fg.OK, fg.strerror(rc)
        torch.cuda.synchronize()
        st = self.ctx.stats()
        assert st.error_code == 0, (st.error_code, hex(st.error_id))
        self.last = (bits(out_cpu), w_cpu.numpy())
        if check:
            self.check_staging()
            self.check_y()
        return st

    def check_staging(self):
        ob, _ = self.last
        lay = self.case.lay
        want = O.combine_staging(ob, lay)
        for s in range(self.S):
            n = int(lay.stream_len[s])
            assert np.array_equal(bits(self.staging[s][:n]), want[s]), f"staging rows of shard {s}"

    def check_y(self):
        ob, w = self.last
        c = self.case
        y64 = O.combine(ob, w, self.topk_np, c.expert_base, c.n_groups, c.lay)
        tol = O.combine_tolerance(ob, w, self.topk_np, c.expert_base, c.n_groups, c.lay)
        worst = 0.0
        lo, hi = c.expert_base, c.expert_base + c.n_groups
        for s in range(self.S):
            yb = O.bf16_to_f64(bits(self.y[s]))
            d = np.abs(yb - y64[s])
            assert np.all(d <= tol[s]), f"shard {s}: max excess {float((d - tol[s]).max()):.3g}"
            worst = max(worst, float((d / tol[s]).max()))
            # tokens with no local pick: exactly zero rows
            none = ~np.any((self.topk_np[s] >= lo) & (self.topk_np[s] < hi), axis=1)
            assert np.all(yb[none] == 0.0), f"shard {s}: a token without a local pick has a nonzero row"
        return worst

    def check_plane(self, t, verify_iters=None):
        v = self.ctx.views()
        S, cc = self.S, v.chunk_cap
        lay = self.case.lay
        want = O.state_after(lay, t, cc)
        cs = fg.COUNTER_STRIDE
        slot = self.ctx.read_i32(v.combine_slot, S * cc * cs).numpy().reshape(S, cc, cs)[:, :, 0]
        elect = self.ctx.read_i32(v.combine_elect, 2 * S * cc * cs).numpy().reshape(2, S, cc, cs)[:, :, :, 0]
        assert np.array_equal(slot, want.slot), "combine slots"
        assert np.array_equal(elect, want.elect), "combine election counts (both parities)"
        if verify_iters is not None:
            pub = self.ctx.read_i32(v.combine_pub, S * cc).numpy().reshape(S, cc)
            assert np.array_equal(pub, (want.slot > 0) * verify_iters), "one combine publisher per chunk per call"
        rs_cap = self.ctx.cfg.max_rows_per_shard
        tf = self.ctx.read_i32(v.tok_first, S * (rs_cap + 1)).numpy().reshape(S, rs_cap + 1)
        sk = self.ctx.read_i32(v.src_k, S * rs_cap).numpy().reshape(S, rs_cap)
        wtf, wsk = _expected_tables(lay, self.topk_np, self.case.expert_base, self.case.n_groups, rs_cap)
        assert np.array_equal(tf[:, :self.T + 1], wtf), "first stream entry of each token"
        for s in range(S):
            assert np.array_equal(sk[s, :len(wsk[s])], wsk[s]), f"top-k position of the entries of shard {s}"

    def close(self):
        self.ctx.close()


def test_combine_small_ep_three_calls():
    log("combine: 4 shards x 200 tokens, top-4 of 16 experts, 4 local, N=512, 3 calls")
    case = ep_case(2001, 4, 200, 256, 512, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case)
    r.dispatch()
    for t in range(3):
        st = r.combine(3000 + t, flags=fg.CALL_VERIFY)
    assert st.combine_seq == 3
    r.check_plane(3, verify_iters=3)
    r.close()


@pytest.mark.parametrize("N", [128, 384, 2560])
def test_combine_ragged_widths_and_tokens(N):
    log(f"combine: 3 shards x 203 tokens (ragged), top-3 of 12 experts, 5 local at base 2, N={N}")
    case = ep_case(2002, 3, 203, 128, N, n_experts=12, topk=3, n_local=5, expert_base=2)
    r = CombineRun(case)
    r.dispatch()
    r.combine(3100, flags=fg.CALL_VERIFY)
    r.check_plane(1, verify_iters=1)
    r.close()


@pytest.mark.parametrize("combine_wg", [1, 3, 37])
def test_combine_small_grids_stride_over_items(combine_wg):
    log(f"combine with {combine_wg} workgroups: every wave loops over many push and sum items")
    case = ep_case(2011, 4, 300, 128, 256, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case, ctx_kw=dict(combine_wg=combine_wg))
    r.dispatch()
    for t in range(2):
        r.combine(3800 + t, flags=fg.CALL_VERIFY)
    r.check_plane(2, verify_iters=2)
    r.close()


def test_combine_grid_beyond_residency_rejected():
    log("combine grid larger than the resident capacity -> FG_ERESIDENCY at init")
    case = ep_case(2012, 2, 64, 128, 256, n_experts=16, topk=4, n_local=4)
    cfg = fg.make_config(2, 64, 128, 256, n_groups=4, combine_wg=65536)
    with pytest.raises(fg.FgError) as e:
        fg.Context(cfg)
    assert e.value.code == fg.ERESIDENCY


def test_combine_more_than_sixteen_local_picks():
    log("combine: every token picks 20 of 32 local experts (weights beyond the first 16 picks)")
    g = np.random.default_rng(2003)
    S, T, KK, E = 2, 40, 20, 32
    topk = np.stack([np.stack([g.permutation(E)[:KK] for _ in range(T)]) for _ in range(S)])
    case = _manual_case(2003, topk, 128, 256, n_local=E)
    r = CombineRun(case)
    r.dispatch()
    r.combine(3200)
    r.check_plane(1)
    r.close()


def test_combine_shard_without_local_picks():
    log("combine: shard 1 routes nothing here (empty stream); tokens with no local pick give 0")
    g = np.random.default_rng(2004)
    S, T, KK = 3, 90, 4
    topk = np.stack([np.stack([g.permutation(16)[:KK] for _ in range(T)]) for _ in range(S)])
    topk[1] = np.stack([4 + g.permutation(12)[:KK] for _ in range(T)])   # experts 4..15 only
    case = _manual_case(2004, topk, 128, 256, n_local=4)
    assert int(case.lay.stream_len[1]) == 0
    r = CombineRun(case)
    r.dispatch()
    r.combine(3300, flags=fg.CALL_VERIFY)
    assert np.all(bits(r.y[1]) == 0), "tokens without a local pick are zero rows"
    r.check_plane(1, verify_iters=1)
    r.close()


def test_combine_push_only_then_sums_only():
    log("combine roles: push only (staging written, y untouched), then sums only from that staging")
    case = ep_case(2005, 4, 160, 128, 512, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case)
    r.dispatch()
    r.combine(3400, flags=fg.CALL_COMM_ONLY, check=False)
    r.check_staging()
    for y in r.y:
        assert np.all(bits(y) == 0x7FC1), "push-only call wrote y"
    rc = r.ctx.combine(r.out, torch.from_numpy(r.last[1]).to(DEV), r.staging, r.y, flags=fg.CALL_GEMM_ONLY)
    assert rc == fg.OK
    torch.cuda.synchronize()
    r.check_y()
    r.close()


def test_combine_follows_a_route_change():
    log("combine after a new dispatch route (other top-k draw): tables and sums follow the route")
    a = ep_case(2006, 4, 150, 128, 256, n_experts=16, topk=4, n_local=4)
    b = ep_case(2007, 4, 150, 128, 256, n_experts=16, topk=4, n_local=4)
    r = CombineRun(a, ctx_kw=dict(max_rows=600))
    r.dispatch()
    r.combine(3500)
    r.case = b
    r.topk_np = b.topk.cpu().numpy()
    rc = r.ctx.gather_gemm(b.shards, b.w, r.gathered, r.out, route=b.route)
    assert rc == fg.OK
    r.combine(3501)
    v = r.ctx.views()
    S, cc = r.S, v.chunk_cap
    cs = fg.COUNTER_STRIDE
    slot = r.ctx.read_i32(v.combine_slot, S * cc * cs).numpy().reshape(S, cc, cs)[:, :, 0]
    for s in range(S):
        n_ch = -(-int(b.lay.stream_len[s]) // 64)
        assert np.all(slot[s, :n_ch] == 2), "every chunk of the new route published in call 2"
    r.close()


def test_combine_strict_fences_same_bits():
    log("combine with formal release / acquire fences gives the same bits as the default")
    case = ep_case(2013, 4, 180, 128, 512, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case)
    r.dispatch()
    r.combine(3900)
    y1 = [bits(y).copy() for y in r.y]
    r.combine(3900, flags=fg.CALL_STRICT | fg.CALL_VERIFY)
    for a, b in zip(y1, r.y):
        assert np.array_equal(a, bits(b))
    r.close()


def test_combine_is_deterministic():
    log("combine: two calls on the same inputs give identical bits")
    case = ep_case(2008, 4, 128, 128, 1024, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case)
    r.dispatch()
    r.combine(3600)
    y1 = [bits(y).copy() for y in r.y]
    r.combine(3600)
    for a, b in zip(y1, r.y):
        assert np.array_equal(a, bits(b))
    r.close()


def test_combine_full_ep_size():
    """The configured EP call count, each call on new expert outputs and gate
    weights: its staging rows bit-exact and every y element within the
    tolerance (exact zero rows for tokens with no local pick); the combine
    slots, election counts and publisher counts exact after the last."""
    c = W.CONFIGS["ep"]
    log(f"combine at the EP workload size: 8 x 1024 tokens, top-8 of 64, 8 local, N=2048, {c['iters']} calls, "
        f"every element of each")
    case = ep_case(c["seed"], c["n_shards"], c["tokens"], c["K"], c["N"], n_experts=c["n_experts"],
                   topk=c["topk"], n_local=c["n_local"], expert_base=c["expert_base"])
    r = CombineRun(case)
    r.dispatch()
    for t in range(c["iters"]):
        r.combine(3700 + t, flags=fg.CALL_VERIFY)
    r.check_plane(c["iters"], verify_iters=c["iters"])
    r.close()


def test_combine_dropped_publish_times_out():
    log("combine fault: the publisher of chunk (0,0) skips its slot store -> FG_ETIMEOUT, every wave exits")
    case = ep_case(2009, 2, 128, 128, 256, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case, timeout_ns=20_000_000)
    r.dispatch()
    out_cpu, w_cpu = W.combine_inputs(1, r.out.shape[0], case.N, r.S, r.T, r.KK)
    rc = r.ctx.combine(r.out, w_cpu.to(DEV), r.staging, r.y, flags=fg.FAULT_DROP_PUBLISH)
    assert rc == fg.OK
    torch.cuda.synchronize()
    st = r.ctx.stats()
    assert st.error_code == fg.ETIMEOUT
    assert r.ctx.combine(r.out, w_cpu.to(DEV), r.staging, r.y) in (fg.ETIMEOUT, fg.ESTATE)
    r.close()


def test_combine_invalid_arguments():
    log("combine: needs a TOPK route; one role flag at most; no NULL buffers")
    case = ep_case(2010, 2, 64, 128, 256, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case)
    w = torch.zeros(r.S, r.T, r.KK, dtype=torch.float32, device=DEV)
    assert r.ctx.combine(r.out, w, r.staging, r.y) == fg.EINVAL          # no route yet
    contig = fg.route_contig(64)
    assert r.ctx.gather_gemm(case.shards, case.w, r.gathered, r.out, route=contig) == fg.OK
    assert r.ctx.combine(r.out, w, r.staging, r.y) == fg.EINVAL          # route is not top-k
    r.dispatch()
    assert r.ctx.combine(r.out, w, r.staging, r.y, flags=fg.CALL_COMM_ONLY | fg.CALL_GEMM_ONLY) == fg.EINVAL
    lib = fg.load_library()
    assert lib.fg_combine(r.ctx._h, None, None, None, None, 0, None) == fg.EINVAL
    torch.cuda.synchronize()
    assert r.ctx.stats().error_code == 0
    r.close()


@pytest.mark.parametrize("seed", list(range(400, 412)))
def test_combine_random_configuration(seed):
    """Seeded random combine configurations: shards, tokens, row widths, expert
    counts, top-k, the local expert window and its base, and the combine grid;
    two calls, staging rows, outputs and the combine control plane checked."""
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 9))
    T = int(rng.integers(1, 400))
    n_experts = int(rng.choice([8, 16, 64]))
    topk = int(rng.integers(1, min(8, n_experts) + 1))
    n_local = int(rng.integers(1, min(16, n_experts) + 1))
    base = int(rng.integers(0, n_experts - n_local + 1))
    N = 128 * int(rng.integers(1, 24))
    combine_wg = int(rng.choice([0, 1, 7, 64]))
    log(f"seed {seed}: combine {S} shards x {T} tokens, top-{topk} of {n_experts}, {n_local} local at {base}, "
        f"N={N}, combine_wg={combine_wg}")
    case = ep_case(seed, S, T, 128, N, n_experts=n_experts, topk=topk, n_local=n_local, expert_base=base)
    r = CombineRun(case, ctx_kw=dict(combine_wg=combine_wg))
    r.dispatch()
    for t in range(2):
        r.combine(seed * 10 + t, flags=fg.CALL_VERIFY)
    r.check_plane(2, verify_iters=2)
    r.close()


def test_combine_misaligned_buffers_rejected():
    """The combine's expert outputs, staging and result rows start on 16-byte
    boundaries and its gate weights on 4-byte ones; otherwise FG_EINVAL, and a
    valid combine on the same context still matches the oracle."""
    log("combine: misaligned buffers -> FG_EINVAL, then a valid call")
    case = ep_case(2014, 4, 160, 128, 256, n_experts=16, topk=4, n_local=4)
    r = CombineRun(case)
    r.dispatch()
    wd = torch.rand(r.S, r.T, r.KK, device=DEV)
    ctx = r.ctx
    assert ctx.combine(misaligned_like(r.out), wd, r.staging, r.y) == fg.EINVAL
    assert ctx.combine(r.out, wd, [r.staging[0], misaligned_like(r.staging[1])] + r.staging[2:], r.y) == fg.EINVAL
    assert ctx.combine(r.out, wd, r.staging, r.y[:3] + [misaligned_like(r.y[3], 8)]) == fg.EINVAL
    flat = torch.empty(wd.numel() + 1, dtype=torch.uint8, device=DEV)
    assert ctx.combine(r.out, flat[1:], r.staging, r.y) == fg.EINVAL     # weights 1 byte past a boundary
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    r.combine(2015)
    ctx.close()
