"""Protocol entry points on the GPU: the all-rank slot barrier, the slot
ping-pong, the protocol-stress workload, and the error paths (bounded waits that
time out, counters that overshoot, invalid arguments)."""
import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import fg
from sync_protocols_amd import workloads as W
from fg_harness import DEV, buffers, check_out, dense_case, log, make_ctx, misaligned_like

pytestmark = pytest.mark.gpu


def _small_ctx(n_shards=4, timeout_ns=0, stress=(0, 0, 0)):
    return fg.Context(fg.make_config(n_shards, 256, 256, 256, timeout_ns=timeout_ns, stress=stress))


@pytest.mark.parametrize("n", [2, 4, 8])
def test_barrier_slots(n):
    log(f"slot barrier over {n} virtual ranks, 3 calls of 1, 10, 1000 rounds")
    ctx = _small_ctx(n)
    total = 0
    for r in (1, 10, 1000):
        assert ctx.barrier(r) == 0
        total += r
    st = ctx.stats()
    assert st.error_code == 0 and st.bseq == total
    v = ctx.views()
    bs = ctx.read_i32(v.bslot, n * n).numpy().reshape(n, n)
    assert np.array_equal(bs, O.barrier_expected(n, total))
    assert st.t_barrier_us > 0
    log(f"barrier n={n}: {st.t_barrier_us:.3f} us per barrier")
    ctx.close()


def test_pingpong_rtt():
    log("slot ping-pong across XCDs, agent and system scope")
    ctx = _small_ctx()
    for sys_scope in (False, True):
        assert ctx.pingpong(2000, sys_scope) == 0
        st = ctx.stats()
        assert st.error_code == 0 and 0 < st.t_rtt_us < 100
        log(f"rtt sys={sys_scope}: {st.t_rtt_us:.3f} us")
    ctx.close()


def _stress_ctx(st_in, timeout_ns=0):
    P, C, KC = st_in.chunk_rows.shape
    return fg.Context(fg.make_config(4, 256, 256, 256, timeout_ns=timeout_ns, stress=(P, C, KC)))


def test_stress_full_config():
    c = W.CONFIGS["stress"]
    log("protocol stress: 64 producers x 64 consumers, 10000 signals/iteration, 50 iterations, delays 0-20us")
    st_in = W.stress_inputs(c["seed"], iters=c["iters"])
    ctx = _stress_ctx(st_in)
    cr = st_in.chunk_rows.to(DEV)
    delays = st_in.delays_ns.to(DEV)
    P, C, KC = st_in.chunk_rows.shape
    payload = torch.zeros(C * P * KC * 64, dtype=torch.int32, device=DEV)
    active = st_in.chunk_rows.numpy() > 0
    for t in range(c["iters"]):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        assert ctx.stress(cr, delays[t].contiguous(), payload) == 0
        e1.record()
        e1.synchronize()
        # a producer spins its delays one chunk after another, so the call takes
        # at least the largest per-producer sum of delays (the wall clock's rate
        # is the device's own)
        d_ns = st_in.delays_ns[t].numpy().astype(np.int64) * active
        floor_ms = float(d_ns.reshape(P, -1).sum(axis=1).max()) * 1e-6
        assert e0.elapsed_time(e1) >= 0.95 * floor_ms, (t, e0.elapsed_time(e1), floor_ms)
    st = ctx.stats()
    assert st.error_code == 0 and st.stale == 0 and st.timeouts == 0
    want = O.stress_expected(st_in.chunk_rows.numpy(), c["iters"])
    v = ctx.views()
    slots = ctx.read_i32(v.stress_slot, P * C * KC).numpy().reshape(P, C, KC)
    pubs = ctx.read_i32(v.stress_pub, P * C * KC).numpy().reshape(P, C, KC)
    assert np.array_equal(slots, want["slot"])
    assert np.array_equal(pubs, want["pub_count"])
    got = payload.cpu().numpy().view(np.uint32).reshape(C, P, KC, 64)
    assert np.array_equal(got[want["valid"]], want["payload"][want["valid"]])
    log(f"stress ok: slot polls {st.slot_polls}")
    ctx.close()


def test_stress_strict_mode():
    log("protocol stress, 5 iterations with formal release fences")
    st_in = W.stress_inputs(1004, iters=5)
    ctx = _stress_ctx(st_in)
    cr = st_in.chunk_rows.to(DEV)
    delays = st_in.delays_ns.to(DEV)
    payload = torch.zeros(64 * 64 * 4 * 64, dtype=torch.int32, device=DEV)
    for t in range(5):
        assert ctx.stress(cr, delays[t].contiguous(), payload, flags=fg.CALL_STRICT) == 0
    st = ctx.stats()
    assert st.error_code == 0 and st.stale == 0
    ctx.close()


# ------------------------------------------------------------- error paths

def test_dropped_publish_times_out_in_stress():
    log("fault: dropped publish in the stress workload -> bounded wait times out")
    st_in = W.stress_inputs(1004, producers=4, consumers=4, signals=40, iters=2)
    ctx = _stress_ctx(st_in, timeout_ns=20_000_000)
    cr = st_in.chunk_rows.to(DEV)
    d = torch.zeros_like(st_in.delays_ns[0]).to(DEV)
    payload = torch.zeros(4 * 4 * 4 * 64, dtype=torch.int32, device=DEV)
    assert ctx.stress(cr, d, payload, flags=fg.FAULT_DROP_PUBLISH) == 0
    st = ctx.stats()
    assert st.error_code == fg.ETIMEOUT
    # the consumer waiting on slot 0 (producer 0, consumer 0, chunk 0) times out
    assert st.timeouts >= 1 and st.first_timeout_id == 0
    assert ctx.stress(cr, d, payload) == fg.ETIMEOUT     # reported by the next call
    assert ctx.stress(cr, d, payload) == fg.ESTATE       # then sticky
    ctx.close()


def test_seed_low_times_out():
    log("fault: padding seed one too low -> gate never opens -> FG_ETIMEOUT")
    case = dense_case(40, 3, 50, 256, 256)
    ctx = make_ctx(case, timeout_ns=20_000_000)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=fg.FAULT_SEED_LOW) == 0
    st = ctx.stats()
    assert st.error_code == fg.ETIMEOUT and st.error_id == 0
    # every compute workgroup gating on row block 0 times out; the first is block 0
    assert st.timeouts >= 1 and st.first_timeout_id == 0
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route) == fg.ETIMEOUT
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route) == fg.ESTATE
    ctx.close()


def test_seed_high_overshoots():
    log("fault: padding seed one too high -> counter overshoots -> FG_EPROTOCOL")
    case = dense_case(41, 3, 50, 256, 256)
    ctx = make_ctx(case, timeout_ns=20_000_000)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=fg.FAULT_SEED_HIGH) == 0
    st = ctx.stats()
    assert st.error_code == fg.EPROTOCOL
    assert st.first_timeout_id == -1   # an overshoot is not a timeout
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route) == fg.EPROTOCOL
    ctx.close()


def test_dropped_publish_visible_in_slots():
    log("fault: dropped publish in the gather -> slot (0,0) stays behind, nothing else changes")
    case = dense_case(42, 4, 256, 256, 512)
    ctx = make_ctx(case)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route) == 0
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=fg.FAULT_DROP_PUBLISH) == 0
    torch.cuda.synchronize()
    v = ctx.views()
    slots = ctx.read_i32(v.slot, 4 * v.chunk_cap).numpy().reshape(4, -1)
    assert slots[0, 0] == 1 and np.all(slots[:, :4][slots[:, :4] != 1] == 2)
    assert (slots[:, :4] == 2).sum() == 15
    ctx.close()


def test_duplicate_route_row_rejected():
    log("bad route: two stream rows target one gathered row -> FG_EPROTOCOL")
    case = dense_case(43, 2, 128, 256, 256)
    src = torch.arange(128, dtype=torch.int32).repeat(2, 1).contiguous().to(DEV)
    dst = torch.arange(128, dtype=torch.int32).repeat(2, 1).contiguous().to(DEV)   # both shards -> rows 0..127
    route = fg.route_explicit([128, 128], src, dst, 256, 128)
    ctx = make_ctx(case, timeout_ns=20_000_000)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=route) == 0
    st = ctx.stats()
    assert st.error_code == fg.EPROTOCOL
    ctx.close()


def test_invalid_arguments():
    log("invalid arguments: stream binding, both role flags, bad route sizes")
    case = dense_case(44, 2, 128, 256, 256)
    ctx = make_ctx(case)
    g, o = buffers(ctx, case)
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route) == 0
    s2 = torch.cuda.Stream()
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, stream=s2) == fg.EINVAL
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route,
                           flags=fg.CALL_COMM_ONLY | fg.CALL_GEMM_ONLY) == fg.EINVAL
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=fg.route_contig(1000)) == fg.EINVAL
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    ctx.close()


def test_litmus_device_scope_loads_see_signalled_data():
    log("litmus: writer on XCD 0, reader on XCD 1 with the old block cached; device-scope loads after the flag")
    ctx = fg.Context(fg.make_config(2, 256, 256, 256))
    assert ctx.litmus(5000, 0) == fg.OK
    st0 = ctx.stats()
    assert st0.error_code == 0
    assert st0.litmus_words == 5000 * 4096
    assert st0.litmus_stale == 0, "a device-scope load returned a word from before the signal"
    assert ctx.litmus(2000, 1) == fg.OK
    st1 = ctx.stats()
    log(f"plain loads without a fence: {st1.litmus_stale - st0.litmus_stale} stale words of {2000 * 4096} "
        "(the reader's caches are in reach of the test)")
    assert ctx.litmus(5000, 2) == fg.OK
    st2 = ctx.stats()
    assert st2.error_code == 0
    assert st2.litmus_stale == st1.litmus_stale, "plain loads after the acquire fence returned stale words"
    assert ctx.litmus(0, 0) == fg.EINVAL and ctx.litmus(10, 3) == fg.EINVAL
    ctx.close()


def test_misaligned_buffers_rejected():
    """Row buffers must start on 16-byte boundaries (rows move in 16-byte
    vectors): a shard, the weights, the gathered or output buffer, a staging
    buffer or a ring 2 bytes past one gives FG_EINVAL before anything is
    launched, and the context then runs a valid call as before."""
    log("misaligned row buffers -> FG_EINVAL; the context stays usable")
    case = dense_case(45, 2, 128, 256, 256)
    ctx = make_ctx(case)
    g, o = buffers(ctx, case)
    mis_shards = [case.shards[0], misaligned_like(case.shards[1])]
    assert ctx.gather_gemm(mis_shards, case.w, g, o, route=case.route) == fg.EINVAL
    assert ctx.gather_gemm(case.shards, misaligned_like(case.w), g, o, route=case.route) == fg.EINVAL
    assert ctx.gather_gemm(case.shards, case.w, misaligned_like(g), o, route=case.route) == fg.EINVAL
    assert ctx.gather_gemm(case.shards, case.w, g, misaligned_like(o, 8), route=case.route) == fg.EINVAL
    staging = [torch.empty(128, case.K, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    staging[1] = misaligned_like(staging[1], 4)
    assert ctx.gather_gemm_staged(case.shards, case.w, staging, g, o, self_shard=0, route=case.route) == fg.EINVAL
    assert ctx.views().ring_cap >= 2       # so the ring call below fails on the alignment alone
    ring = torch.empty(fg.ring_bytes(ctx.cfg, 1, 2) + 16, dtype=torch.uint8, device=DEV)[2:]
    assert ctx.gather_gemm_ring(case.shards, case.w, ring, g, o, n_channels=1, ring_chunks=2,
                                route=case.route) == fg.EINVAL
    torch.cuda.synchronize()
    assert ctx.stats().error_code == 0
    assert ctx.gather_gemm(case.shards, case.w, g, o, route=case.route, flags=fg.CALL_VERIFY) == fg.OK
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st.error_code == 0 and st.publishes == st.expected_publishes
    check_out(case, o)
    ctx.close()
