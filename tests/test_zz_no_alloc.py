"""fg_gather_gemm_noalloc (through the C ABI) against fg_gather_gemm on the
same inputs: two calls in a row, the second with a smaller input. The
gathered rows and the outputs must equal those of the context entry point
bit for bit (neither splits a tile on these shapes, and the tiles run the
same code), and both must match the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from fg_harness import DEV, bits, check_gathered, check_out, dense_case, log, make_ctx, poison_

pytestmark = pytest.mark.gpu


def _both(case, label):
    # reference: the context entry point
    ctx = make_ctx(case)
    cap = fg.capacity(ctx.cfg)
    g_ref = torch.zeros(cap, case.K, dtype=torch.bfloat16, device=DEV)
    o_ref = torch.zeros(cap, case.N, dtype=torch.bfloat16, device=DEV)
    poison_(g_ref)
    poison_(o_ref)
    assert ctx.gather_gemm(case.shards, case.w, g_ref, o_ref, route=case.route) == fg.OK
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    cfg = ctx.cfg
    ctx.close()
    # the same iteration with no context
    g = torch.zeros(cap, case.K, dtype=torch.bfloat16, device=DEV)
    o = torch.zeros(cap, case.N, dtype=torch.bfloat16, device=DEV)
    poison_(g)
    poison_(o)
    status = torch.full((1,), 12345, dtype=torch.int32, device=DEV)
    rc = fg.gather_gemm_noalloc(cfg, case.shards, case.w, g, o, status, route=case.route)
    assert rc == fg.OK, fg.strerror(rc)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, f"{label}: device-side error {int(status.item())}"
    m_pad = case.lay.m_pad
    assert torch.equal(g[:m_pad].view(torch.int16), g_ref[:m_pad].view(torch.int16)), f"{label}: gathered rows"
    assert torch.equal(o[:m_pad].view(torch.int16), o_ref[:m_pad].view(torch.int16)), f"{label}: outputs"
    check_gathered(case, g, poisoned=True)
    r = check_out(case, o)
    log(f"{label}: no-alloc call equals the context call bit for bit; max|d| vs oracle {r['max_abs']:.3g}")


def test_noalloc_two_calls_second_smaller():
    log("no-alloc: 4 x 512 rows K=512 N=512 contiguous, then 3 x 100 rows K=256 N=256 permuted")
    _both(dense_case(501, 4, 512, 512, 512), "call 1 (4 x 512, K=512, N=512)")
    _both(dense_case(502, 3, 100, 256, 256, gather="permutation"), "call 2 (3 x 100, K=256, N=256)")


def test_noalloc_at_the_largest_documented_size():
    """The size its scratch array is sized for: 8 shards x 4096 rows gathered by
    a permutation, K = N = 8192; bit for bit as the context call, and every
    output element against the oracle."""
    log("no-alloc at 8 x 4096 rows permuted, K=N=8192")
    _both(dense_case(504, 8, 4096, 8192, 8192, gather="permutation"), "8 x 4096, K=N=8192")


def test_noalloc_rejects_what_it_cannot_hold():
    log("no-alloc: a control plane beyond the scratch size, bad flags and NULLs are refused before any launch")
    case = dense_case(503, 2, 128, 256, 256)
    cfg = fg.make_config(64, 1 << 16, 256, 256)        # 64 shards x 65536 rows: tens of MiB of route tables
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = torch.zeros(256, 256, dtype=torch.bfloat16, device=DEV)
    o = torch.zeros(256, 256, dtype=torch.bfloat16, device=DEV)
    assert fg.gather_gemm_noalloc(cfg, case.shards, case.w, g, o, status, route=case.route) == fg.EINVAL
    small = fg.make_config(2, 128, 256, 256)
    assert fg.gather_gemm_noalloc(small, case.shards, case.w, g, o, status, route=case.route,
                                  flags=fg.CALL_VERIFY) == fg.EINVAL
    assert fg.gather_gemm_noalloc(small, case.shards, case.w, g, o, status, route=case.route) == fg.OK
    torch.cuda.synchronize()
    assert int(status.item()) == 0
