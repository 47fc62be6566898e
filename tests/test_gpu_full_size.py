"""Parity at the full workload sizes, over the configured iteration counts
(TP 20, EP 20, Large 50), checked after every call.

Before each call the gathered and output buffers are poisoned with a bf16
NaN, so a gate that opens early, a stale read or a lost signal in any call
leaves NaN or old bits behind. After every call:
  - the gathered rows are compared bit for bit with the oracle's gather
    (padding rows must still hold the poison: they are never written);
  - the route tables and the whole control plane (slots, both parities of
    the arrival counters and election counts, publisher counts) are compared
    bit for bit with the oracle's state after iteration t;
  - the publish count equals the device's expected count and the oracle's
    closed form, with no timeout.
Every output element is compared with the oracle's fp64 product on the first
and the last call. The calls in between must give the same output bits as
the first one: the contraction's summation order, split-K parts included,
does not depend on which workgroup runs which item, so any difference is a
wrong read. A final call with formal release/acquire fences must give the
same bits again ("PCIe sync protocols" §7: repeated iterations with the
intermediate buffers reconciled byte for byte against a host-side table).

The oracle's gathered rows are uploaded once and compared on the device
(torch.equal), which keeps 50 checks of 512 MB affordable; the expected
values themselves are computed on the CPU by the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W
from fg_harness import (DEV, POISON, bits, buffers, check_control_plane, check_out, check_route, control_plane,
                        dense_case, ep_case, log, make_ctx, poison_)

pytestmark = pytest.mark.gpu


def _full_size(case, iters, label, copy_mode=fg.COPY_WORKGROUPS):
    ctx = make_ctx(case, copy_mode=copy_mode)
    gathered, out = buffers(ctx, case)
    lay = case.lay
    m_pad, S = lay.m_pad, lay.n_shards
    real = O.real_rows(lay)
    real_idx = torch.from_numpy(np.nonzero(real)[0]).to(DEV)
    pad_idx = torch.from_numpy(np.nonzero(~real)[0]).to(DEV)
    G_dev = torch.from_numpy(case.oracle_G.view(np.int16)).to(DEV)
    want_pubs = O.signal_counts(lay)["publishes"]
    C64 = None
    ref = None
    for t in range(1, iters + 1):
        poison_(gathered)
        poison_(out)
        rc = ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route, flags=fg.CALL_VERIFY)
        assert rc == fg.OK, (label, t, fg.strerror(rc))
        torch.cuda.synchronize()
        st = ctx.stats()
        assert st.error_code == 0, (label, t, st.error_code, hex(st.error_id))
        assert st.timeouts == 0
        g = gathered[:m_pad].view(torch.int16)
        assert torch.equal(g.index_select(0, real_idx), G_dev.index_select(0, real_idx)), \
            f"{label} call {t}: gathered rows differ from the oracle"
        if pad_idx.numel():
            assert bool((g.index_select(0, pad_idx) == POISON).all()), f"{label} call {t}: a padding row was written"
        cp = control_plane(ctx, S)
        check_route(case, cp)
        check_control_plane(case, cp, t, t)
        assert st.publishes == t * want_pubs and st.expected_publishes == st.publishes, (label, t)
        o = out[:m_pad].view(torch.int16)
        if t == 1 or t == iters:
            if C64 is None:
                log(f"{label}: fp64 oracle product ({m_pad} x {case.N} x {case.K})")
                wb = bits(case.w_cpu)
                C64 = O.gemm(case.oracle_G, wb if wb.ndim == 3 else wb[None], lay)
            ob = bits(out[:m_pad])
            r = O.gemm_check(ob, C64, case.K, case.sigma_x, case.sigma_w, np.repeat(real[:, None], case.N, 1))
            assert r["ok"], (label, t, r)
            log(f"{label} call {t}: every output element within tolerance, max|d|={r['max_abs']:.3g} "
                f"(tol {r['tol']:.3g})")
        if ref is None:
            ref = o.clone()
        else:
            assert torch.equal(o, ref), f"{label} call {t}: output bits differ from call 1"
    # one more call with the formal agent-scope release and acquire fences
    poison_(gathered)
    poison_(out)
    rc = ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route,
                         flags=fg.CALL_VERIFY | fg.CALL_STRICT)
    assert rc == fg.OK
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st.error_code == 0 and st.publishes == (iters + 1) * want_pubs
    g = gathered[:m_pad].view(torch.int16)
    assert torch.equal(g.index_select(0, real_idx), G_dev.index_select(0, real_idx)), f"{label}: strict gather"
    assert torch.equal(out[:m_pad].view(torch.int16), ref), f"{label}: strict fences changed the output bits"
    check_control_plane(case, control_plane(ctx, S), iters + 1, iters + 1)
    log(f"{label}: {iters} calls + 1 strict call bit-identical, control plane exact after each")
    st = ctx.stats()
    ctx.close()
    return st, ref


def test_tp_full_size_every_call():
    c = W.CONFIGS["tp"]
    log(f"TP share: 4 x 2048 rows, K=N=4096, contiguous, {c['iters']} calls")
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"])
    _full_size(case, c["iters"], "tp")


def test_ep_full_size_every_call():
    c = W.CONFIGS["ep"]
    log(f"EP dispatch: 8 x 1024 tokens, top-8/64, 8 local experts, K=7168, N=2048, {c['iters']} calls")
    case = ep_case(c["seed"], c["n_shards"], c["tokens"], c["K"], c["N"])
    _full_size(case, c["iters"], "ep")


def test_large_full_size_every_call():
    c = W.CONFIGS["large"]
    log(f"Large: 8 x 4096 rows permuted, K=N=8192, {c['iters']} calls")
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"], gather="permutation")
    _full_size(case, c["iters"], "large")


@pytest.mark.parametrize("name", ["tp", "large"])
def test_in_tile_copy_full_size_every_call(name):
    """The in-tile copy mode (the compute tiles copy the rows of later rounds
    inside their K loops) at the full TP and Large sizes over the configured
    call counts, checked after every call as above; with no split tail the
    output bits must also equal those of the copy-workgroup mode (the same
    tiles sum in the same order)."""
    c = W.CONFIGS[name]
    gather = "permutation" if name == "large" else "contiguous"
    log(f"{name}, in-tile copy: {c['n_shards']} x {c['rows']} rows ({gather}), K={c['K']}, N={c['N']}, "
        f"{c['iters']} calls")
    case = dense_case(c["seed"], c["n_shards"], c["rows"], c["K"], c["N"], gather=gather)
    st, bits_tiles = _full_size(case, c["iters"], f"{name}/in-tile", copy_mode=fg.COPY_IN_TILES)
    assert st.copy_in_tiles == 1 and st.lead_rows > 0, (st.copy_in_tiles, st.lead_rows)
    ctx = make_ctx(case, copy_mode=fg.COPY_WORKGROUPS)
    gathered, out = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, gathered, out, route=case.route) == fg.OK
    torch.cuda.synchronize()
    st2 = ctx.stats()
    assert st2.error_code == 0 and st2.copy_in_tiles == 0
    if st.tiles_split == 0 and st2.tiles_split == 0:
        assert torch.equal(out[:case.lay.m_pad].view(torch.int16), bits_tiles), \
            f"{name}: in-tile copy and copy workgroups give different output bits"
    ctx.close()
