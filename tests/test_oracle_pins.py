"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked examples, closed forms, invariants, library special cases, exact
rational arithmetic and brute force; plus planted mistakes (in the oracle's
inputs, on the CPU) that each pin must catch."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from sync_protocols_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _num(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


# --------------------------------------------------------------------- bf16

def test_bf16_hand_cases():
    g = _golden("bf16_cases.json")
    for hexbits, val in g["decode"]:
        got = O.bf16_to_f64(np.array([int(hexbits, 16)], np.uint16))[0]
        assert got == _num(val) and math.copysign(1, got) == math.copysign(1, _num(val))
    for val, hexbits, _why in g["encode"]:
        assert int(O.f64_to_bf16(np.array([_num(val)]))[0]) == int(hexbits, 16), (val, _why)


def test_bf16_ulp_hand_cases():
    # grid spacing worked out from the format; zero's neighbour is the
    # smallest subnormal, so ulp(0) is 2^-133 like the rest of the subnormals
    g = _golden("bf16_cases.json")
    for val, want, why in g["ulp"]:
        got = float(O.bf16_ulp(np.array([_num(val)]))[0])
        assert got == _num(want), (val, got, why)


def test_bf16_ulp_is_the_gap_to_the_next_pattern():
    # every finite non-negative pattern except the largest: ulp equals the
    # distance to the next larger bf16 (a brute-force check over the format)
    b = np.arange(0, 0x7F7F, dtype=np.uint16)
    v = O.bf16_to_f64(b)
    nxt = O.bf16_to_f64(b + np.uint16(1))
    # at a power of two the step above is the new binade's; ulp(x) is the
    # spacing of the binade that holds x, which is the gap to the next pattern
    assert np.array_equal(O.bf16_ulp(v), nxt - v)


def test_bf16_encode_matches_torch_on_float32_values():
    # For inputs exactly representable in float32 a single RNE step equals
    # torch's float32 -> bfloat16 conversion (an independent library routine).
    g = torch.Generator().manual_seed(7)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-30, 30, (200000,), generator=g).float())
    x = torch.cat([x, torch.tensor([0.0, -0.0, float("inf"), -float("inf"), 3.3895e38, 1e-40, -1e-41])])
    want = _bits(x.to(torch.bfloat16))
    got = O.f64_to_bf16(x.double().numpy())
    assert np.array_equal(got, want)


def test_bf16_roundtrip_all_finite_patterns():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f64(b)
    fin = np.isfinite(v)
    assert np.array_equal(O.f64_to_bf16(v[fin]), b[fin])


# ------------------------------------------------------------------- layouts

def test_contiguous_gather_equals_concatenation():
    d = W.dense_inputs(11, 4, 96, 64, 64)
    lay = O.layout_contiguous(4, 96)
    G = O.gather([_bits(s) for s in d.shards], lay)
    cat = _bits(torch.cat(d.shards))
    assert lay.m_pad == 384
    assert np.array_equal(G[:384], cat)


def test_contiguous_ragged_padding_rows_zero_and_seeded():
    lay = O.layout_contiguous(3, 50)             # 150 rows -> m_pad 256, last block 22 real rows
    assert lay.m_pad == 256
    assert list(O.seeds(lay)) == [0, 128 - 22]
    shards = [np.full((50, 8), 0x3F80 + s, np.uint16) for s in range(3)]
    G = O.gather(shards, lay)
    assert np.all(G[150:] == 0)
    assert np.all(G[100:150] == 0x3F82)


def test_permutation_brute_force_tiny():
    rng = np.random.default_rng(3)
    S, R = 4, 8
    perm = rng.permutation(S * R)
    lay = O.layout_permutation(perm, S, R, row_block=4, chunk_rows=2)
    shards = [rng.integers(0, 1 << 16, (R, 5)).astype(np.uint16) for _ in range(S)]
    G = O.gather(shards, lay)
    for s in range(S):
        for i in range(R):
            assert np.array_equal(G[perm[s * R + i]], shards[s][i])
    # every gathered row received exactly one stream row
    hits = np.zeros(S * R, int)
    for d in lay.dst_row:
        hits[d] += 1
    assert np.all(hits == 1)


def test_permutation_rejects_non_injective():
    with pytest.raises(AssertionError):
        O.layout_permutation(np.array([0, 1, 1, 2]), 2, 2)


def test_ep_layout_hand_example():
    g = _golden("ep_route_tiny.json")
    lay = O.layout_topk(np.array(g["topk"]), g["expert_base"], g["n_local"],
                        row_block=g["row_block"], chunk_rows=g["chunk_rows"])
    assert [list(x) for x in lay.src_row] == g["src_row"]
    assert [list(x) for x in lay.dst_row] == g["dst_row"]
    assert list(lay.group_off) == g["group_off"]
    assert lay.m_pad == g["m_pad"]
    assert list(O.seeds(lay)) == g["seeds"]
    assert [list(x) for x in O.chunk_table(lay)] == g["chunk_table"]
    assert O.signal_counts(lay)["publishes"] == g["publishes"]


def test_ep_layout_equals_stable_sort_by_expert():
    ep = W.ep_inputs(5, n_shards=8, tokens=96, K=8, N=8)
    topk = ep.topk.numpy()
    lay = O.layout_topk(topk, ep.expert_base, ep.n_local)
    S, T, KK = topk.shape
    # independent construction: list local pairs in global token order, then a
    # stable argsort by expert id gives each expert's rows in token order.
    g_ids, e_ids, s_ids, t_ids = [], [], [], []
    flat = topk.reshape(S * T, KK)
    for gtok in range(S * T):
        for k in range(KK):
            e = flat[gtok, k] - ep.expert_base
            if 0 <= e < ep.n_local:
                g_ids.append(gtok); e_ids.append(e); s_ids.append(gtok // T); t_ids.append(gtok % T)
    e_ids = np.array(e_ids)
    order = np.argsort(e_ids, kind="stable")
    counts = np.bincount(e_ids, minlength=ep.n_local)
    off = np.concatenate([[0], np.cumsum(-(-counts // 128) * 128)])
    assert np.array_equal(lay.group_off, off)
    assert np.all(lay.group_off % 128 == 0)
    assert lay.m == len(e_ids) == counts.sum()
    expect_dst = np.empty(len(e_ids), np.int64)
    pos_in_e = np.zeros(ep.n_local, np.int64)
    for j in order:
        expect_dst[j] = off[e_ids[j]] + pos_in_e[e_ids[j]]
        pos_in_e[e_ids[j]] += 1
    # the oracle's streams, in (s, t, k) order, are the same pair list
    got_dst = np.concatenate(lay.dst_row)
    got_src = np.concatenate(lay.src_row)
    assert np.array_equal(got_dst, expect_dst)
    assert np.array_equal(got_src, np.array(t_ids))
    # no row block mixes experts
    grp = O.group_of_row(lay)
    assert np.all(grp.reshape(-1, 128).min(1) == grp.reshape(-1, 128).max(1))
    # every real block holds at least one real row, so seeds lie in [0, 127]
    sd = O.seeds(lay)
    assert sd.min() >= 0 and sd.max() <= 127


def test_ep_topk_choices_distinct_and_in_range():
    ep = W.ep_inputs(9, n_shards=2, tokens=64, K=8, N=8)
    t = ep.topk.numpy().reshape(-1, 8)
    assert t.min() >= 0 and t.max() < 64
    assert all(len(set(r)) == 8 for r in t)


# ------------------------------------------------------- protocol closed forms

def _layouts_small():
    rng = np.random.default_rng(17)
    yield O.layout_contiguous(3, 37, row_block=16, chunk_rows=8)
    yield O.layout_permutation(rng.permutation(4 * 24), 4, 24, row_block=16, chunk_rows=8)
    topk = np.stack([np.stack([rng.permutation(12)[:3] for _ in range(20)]) for _ in range(3)])
    yield O.layout_topk(topk, 2, 4, row_block=16, chunk_rows=8)


def _random_batches(lay, rng, max_batch):
    rows = [(s, i) for s in range(lay.n_shards) for i in range(int(lay.stream_len[s]))]
    rng.shuffle(rows)
    batches, j = [], 0
    while j < len(rows):
        n = int(rng.integers(1, max_batch + 1))
        batches.append(rows[j:j + n])
        j += n
    return batches


@pytest.mark.parametrize("lay_idx", [0, 1, 2])
def test_closed_forms_equal_event_simulation(lay_idx):
    lay = list(_layouts_small())[lay_idx]
    cap = int(max(-(-lay.stream_len // lay.chunk_rows)))
    rng = np.random.default_rng(100 + lay_idx)
    cf = O.signal_counts(lay)
    assert cf["seed_sum"] == int(O.seeds(lay).sum())
    state = O.state_after(lay, 0, cap)
    for t in range(1, 6):
        batches = _random_batches(lay, rng, 5)
        order = list(rng.permutation(len(batches)))
        r = O.simulate_iteration(lay, state, t, batches, order)
        assert r.publishes == cf["publishes"]
        assert r.arrivals == cf["arrivals"]
        assert r.gate_openings == cf["gate_openings"]
        assert r.early_gates == 0 and r.early_publishes == 0
        want = O.state_after(lay, t, cap)
        assert np.array_equal(r.state.slot, want.slot)
        assert np.array_equal(r.state.counter, want.counter)
        assert np.array_equal(r.state.elect, want.elect)
        assert np.array_equal(r.state.pub_count, want.pub_count)
        assert np.all(r.state.pub_count[r.state.slot > 0] == t)   # one publisher per slot per iteration


def test_planted_wrong_seed_is_caught():
    lay = O.layout_contiguous(3, 37, row_block=16, chunk_rows=8)
    cap = int(max(-(-lay.stream_len // lay.chunk_rows)))
    rng = np.random.default_rng(5)
    sd = O.seeds(lay)
    assert sd[-1] > 0
    # seed one too low: the counter stops one short and the gate never opens
    state = O.state_after(lay, 0, cap)
    state.counter[1] = sd - 1
    b = _random_batches(lay, rng, 4)
    r = O.simulate_iteration(lay, state, 1, b, list(range(len(b))))
    assert r.gate_openings == 0
    # seed one too high: the gate opens one row early, before all its rows landed
    early = 0
    for trial in range(5):
        state = O.state_after(lay, 0, cap)
        state.counter[1] = sd + 1
        b = _random_batches(lay, rng, 1)
        r = O.simulate_iteration(lay, state, 1, b, list(rng.permutation(len(b))))
        early += r.early_gates
    assert early == 5 * lay.n_rb


def test_election_brute_force_all_splits():
    for n in range(1, 7):
        for w in range(1, 4):
            for parts in _compositions(n, w):
                assert O.election_brute_force(parts) == 0


def _compositions(n, w):
    if w == 1:
        yield (n,)
        return
    for first in range(1, n - w + 2):
        for rest in _compositions(n - first, w - 1):
            yield (first,) + rest


def test_gate_model_check():
    good = [[('w', 'a0'), ('w', 'a1'), ('a', 2)], [('w', 'b0'), ('w', 'b1'), ('a', 2)]]
    assert O.model_check_gate(good, seed=0, target=4) == 0
    per_row = [[('w', 'a0'), ('a', 1), ('w', 'a1'), ('a', 1)], [('w', 'b0'), ('a', 1)]]
    assert O.model_check_gate(per_row, seed=1, target=4) == 0        # one padding row seeded
    add_first = [[('a', 2), ('w', 'a0'), ('w', 'a1')], [('w', 'b0'), ('w', 'b1'), ('a', 2)]]
    assert O.model_check_gate(add_first, seed=0, target=4) > 0        # signal before data: caught
    assert O.model_check_gate(per_row, seed=2, target=4) > 0          # wrong seed: caught


# -------------------------------------------------------------------- GEMM

def test_gemm_hand_example():
    g = _golden("gemm_hand.json")
    G = O.f64_to_bf16(np.array(g["G"], float))
    w = O.f64_to_bf16(np.array(g["w_store_NxK"], float))
    lay = O.layout_contiguous(1, 2, row_block=2)
    C = O.gemm(G, w, lay)
    assert np.array_equal(C, np.array(g["C"], float))
    assert np.array_equal(np.array(g["W_logical_KxN"]).T, np.array(g["w_store_NxK"]))


def test_gemm_identity_weight_returns_input():
    rng = np.random.default_rng(1)
    Gb = O.f64_to_bf16(rng.standard_normal((32, 16)))
    lay = O.layout_contiguous(1, 32, row_block=32)
    C = O.gemm(Gb, O.f64_to_bf16(np.eye(16)), lay)
    assert np.array_equal(C, O.bf16_to_f64(Gb))


def test_gemm_exact_rational_brute_force():
    rng = np.random.default_rng(2)
    M, K, N = 6, 9, 5
    Gb = O.f64_to_bf16(rng.standard_normal((M, K)))
    Wb = O.f64_to_bf16(0.02 * rng.standard_normal((N, K)))
    lay = O.layout_contiguous(1, M, row_block=M)
    C = O.gemm(Gb, Wb, lay)
    Gf = O.bf16_to_f64(Gb)
    Wf = O.bf16_to_f64(Wb)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(Gf[m, k]) * Fraction(Wf[n, k]) for k in range(K))
            assert abs(Fraction(C[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_gemm_grouped_uses_each_rows_group():
    # two groups, W_g = (g + 1) * I: row m of group g must come out (g+1) * G[m]
    lay = O.Layout([np.arange(3), np.arange(2)], [np.array([0, 1, 2]), np.array([4, 5])],
                   8, np.array([0, 4, 8]), row_block=4, chunk_rows=2)
    rng = np.random.default_rng(4)
    shards = [O.f64_to_bf16(rng.integers(-8, 8, (3, 4)).astype(float)),
              O.f64_to_bf16(rng.integers(-8, 8, (2, 4)).astype(float))]
    G = O.gather(shards, lay)
    Wb = np.stack([O.f64_to_bf16(np.eye(4)), O.f64_to_bf16(2 * np.eye(4))])
    C = O.gemm(G, Wb, lay)
    Gf = O.bf16_to_f64(G)
    assert np.array_equal(C[:3], Gf[:3]) and np.array_equal(C[4:6], 2 * Gf[4:6])
    assert np.all(C[3] == 0) and np.all(C[6:] == 0)


def test_gemm_check_has_teeth():
    rng = np.random.default_rng(6)
    C = rng.standard_normal((64, 32)) * 1.28
    out = O.f64_to_bf16(C)
    assert O.gemm_check(out, C, 4096, 1.0, 0.02)["ok"]
    bad = O.bf16_to_f64(out).copy()
    bad[3, 4] += 3 * O.gemm_tolerance(4096, 1.0, 0.02)
    assert not O.gemm_check(O.f64_to_bf16(bad), C, 4096, 1.0, 0.02)["ok"]
    mask = np.ones(64, bool)
    mask[60:] = False
    C2 = C.copy()
    C2[60:] = 0
    out2 = O.f64_to_bf16(C2)
    assert O.gemm_check(out2, C2, 4096, 1.0, 0.02, mask[:, None].repeat(32, 1))["ok"]
    out2[61, 0] = 0x3F80
    assert not O.gemm_check(out2, C2, 4096, 1.0, 0.02, mask[:, None].repeat(32, 1))["ok"]


def test_gemm_check_is_tight_at_exact_zeros():
    # where the fp64 result is exactly 0 (a real row whose products cancel)
    # the allowance is the stated tolerance plus half a subnormal step, so an
    # error a little above the tolerance fails there as it does elsewhere
    K = 256
    tol = O.gemm_tolerance(K, 1.0, 0.02)
    C = np.zeros((4, 8))
    C[0, 0] = 1.0
    ok = O.f64_to_bf16(C)
    assert O.gemm_check(ok, C, K, 1.0, 0.02)["ok"]
    bad = C.copy()
    bad[2, 3] = 1.25 * tol            # the result there is 0
    r = O.gemm_check(O.f64_to_bf16(bad), C, K, 1.0, 0.02)
    assert not r["ok"] and r["n_bad"] == 1


def test_gemm_tolerance_value():
    # 2 % of the output standard deviation sqrt(K) * 1 * 0.02 at K = 4096
    assert abs(O.gemm_tolerance(4096, 1.0, 0.02) - 0.0256) < 1e-15


# ------------------------------------------------------------------ stress

def test_stress_config_counts():
    st = W.stress_inputs(1004, iters=2)
    cr = st.chunk_rows.numpy()
    assert cr.shape == (64, 64, 4)
    exp = O.stress_expected(cr, 1)
    assert exp["signals"] == 10000
    assert int((cr > 0).sum()) == 10000 and cr.size == 16384
    assert cr.max() == 64 and cr[cr > 0].min() >= 1
    d = st.delays_ns.numpy()
    assert d.min() >= 0 and d.max() <= 20000


def test_stress_final_state_independent_of_delays():
    st = W.stress_inputs(21, producers=4, consumers=5, max_chunks=4, signals=48, iters=3)
    cr = st.chunk_rows.numpy()
    for t in range(1, 4):
        want = O.stress_expected(cr, t)
        got = O.stress_simulate(cr, t, st.delays_ns[t - 1].numpy())
        assert np.array_equal(got["slot"], want["slot"])
        assert np.array_equal(got["pubs"], (cr > 0).astype(int))
        assert got["stale"] == 0


def test_stress_payload_unique_per_iteration_and_row():
    seen = set()
    for seq in (1, 2):
        for p in range(3):
            for k in range(4):
                for r in range(64):
                    seen.add(O.stress_payload(seq, p, 1, k, r, 64, 4))
    assert len(seen) == 2 * 3 * 4 * 64


# ----------------------------------------------------------------- barrier

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_barrier_simulation_matches_closed_form(seed):
    for n in (2, 4, 8):
        assert np.array_equal(O.barrier_simulate(n, 5, seed), O.barrier_expected(n, 5))


# ----------------------------------------------------------- measurement

def test_overlap_formula():
    assert O.overlap_efficiency(100.0, 30.0, 100.0) == 1.0    # comm fully hidden
    assert O.overlap_efficiency(100.0, 30.0, 130.0) == 0.0    # serial
    assert abs(O.overlap_efficiency(100.0, 30.0, 106.0) - 0.8) < 1e-12
    assert O.compute_interference(110.0, 100.0) == 1.1


# ------------------------------------------------------------- workloads

def test_workload_distributions():
    d = W.dense_inputs(1001, 4, 256, 256, 512)
    x = torch.cat(d.shards).float()
    assert abs(x.mean().item()) < 0.02 and abs(x.std().item() - 1) < 0.02
    w = d.w.float()
    assert w.shape == (512, 256) and abs(w.std().item() - 0.02) < 0.001
    p = W.dense_inputs(3, 2, 64, 8, 8, gather="permutation").perm
    assert sorted(p.tolist()) == list(range(128))


# ----------------------------------------------------------------- combine

def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def test_combine_hand_worked_example():
    g = _golden("combine_tiny.json")
    topk = np.array(g["topk"])
    lay = O.layout_topk(topk, g["expert_base"], g["n_local"], row_block=g["row_block"])
    assert lay.m_pad == g["m_pad"]
    assert [list(map(int, d)) for d in lay.dst_row] == g["dst_row"]
    picks = O.combine_picks(topk, g["expert_base"], g["n_local"])
    assert [[list(p) for p in ps] for ps in picks] == g["picks"]
    out_bits = O.f64_to_bf16(np.array(g["out"], dtype=np.float64))
    y = O.combine(out_bits, np.array(g["weights"], dtype=np.float32), topk, g["expert_base"], g["n_local"], lay)
    assert np.array_equal(y, np.array(g["y"]))
    st = O.combine_staging(out_bits, lay)
    for s in range(2):
        assert np.array_equal(st[s], out_bits[np.array(g["dst_row"][s])])


def test_combine_after_identity_dispatch_is_identity():
    """Dispatch with every expert local, an identity expert (out row = its gathered
    row) and weights that sum to 1 over each token's picks: combine returns each
    token's own row exactly."""
    rng = np.random.default_rng(7)
    S, T, KK, E = 3, 40, 4, 8
    topk = np.stack([np.stack([rng.permutation(E)[:KK] for _ in range(T)]) for _ in range(S)])
    lay = O.layout_topk(topk, 0, E, row_block=16)
    x = [O.f64_to_bf16(rng.standard_normal((T, 24))) for _ in range(S)]
    G = O.gather(x, lay)
    w = np.array([0.5, 0.25, 0.125, 0.125], dtype=np.float32)[None, None, :].repeat(S, 0).repeat(T, 1)
    y = O.combine(G, w, topk, 0, E, lay)
    for s in range(S):
        assert np.array_equal(y[s], O.bf16_to_f64(x[s]))


def test_combine_partial_locality_and_tolerance_teeth():
    rng = np.random.default_rng(8)
    S, T, KK, E = 2, 30, 4, 16
    topk = np.stack([np.stack([rng.permutation(E)[:KK] for _ in range(T)]) for _ in range(S)])
    lay = O.layout_topk(topk, 4, 4, row_block=8)
    out = O.f64_to_bf16(rng.standard_normal((lay.m_pad, 16)))
    w = rng.random((S, T, KK)).astype(np.float32)
    y = O.combine(out, w, topk, 4, 4, lay)
    # brute force over the top-k lists directly
    gpos = {}
    for s in range(S):
        for i, d in enumerate(lay.dst_row[s]):
            gpos[(s, i)] = int(d)
    picks = O.combine_picks(topk, 4, 4)
    for s in range(S):
        for t in range(T):
            want = np.zeros(16)
            for i, (tt, k) in enumerate(picks[s]):
                if tt == t:
                    assert 4 <= topk[s, t, k] < 8
                    want += float(w[s, t, k]) * O.bf16_to_f64(out[gpos[(s, i)]])
            assert np.allclose(y[s, t], want, rtol=0, atol=1e-12)
            if not any(4 <= e < 8 for e in topk[s, t]):
                assert np.all(y[s, t] == 0)
    tol = O.combine_tolerance(out, w, topk, 4, 4, lay)
    assert np.all(tol > 0)
    yb = O.bf16_to_f64(O.f64_to_bf16(y))
    assert np.all(np.abs(yb - y) <= tol)
    bad = yb.copy()
    idx = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    bad[idx] += 3 * tol[idx]
    assert not np.all(np.abs(bad - y) <= tol)
    # a token with no local pick sums nothing: its row is exactly 0 and the
    # bound there admits no nonzero bf16 value (the smallest is 2^-133)
    empty = [(s, t) for s in range(S) for t in range(T) if not any(4 <= e < 8 for e in topk[s, t])]
    assert empty
    s0, t0 = empty[0]
    assert np.all(tol[s0, t0] < 2.0 ** -133)
    bad = yb.copy()
    bad[s0, t0, 5] = 2.0 ** -133
    assert not np.all(np.abs(bad - y) <= tol)


# ------------------------------------------------------------ two-stage dispatch

def _push_batches(lay, rng, self_shard, max_rows=3):
    """Random push batches of remote stream entries, each inside one chunk."""
    out = []
    for s in range(lay.n_shards):
        if s == self_shard:
            continue
        n = int(lay.stream_len[s])
        for c0 in range(0, n, lay.chunk_rows):
            i = c0
            end = min(n, c0 + lay.chunk_rows)
            while i < end:
                k = int(rng.integers(1, max_rows + 1))
                out.append([(s, j) for j in range(i, min(end, i + k))])
                i += k
    return out


def _scatter_batches(lay, rng, max_rows=5):
    rows = [int(d) for s in range(lay.n_shards) for d in lay.dst_row[s]]
    rows.sort()
    out, j = [], 0
    while j < len(rows):
        k = int(rng.integers(1, max_rows + 1))
        out.append(rows[j:j + k])
        j += k
    return out


def test_push_staging_special_cases():
    rng = np.random.default_rng(31)
    shards = [O.f64_to_bf16(rng.standard_normal((9, 4))) for _ in range(3)]
    lay = O.layout_contiguous(3, 9)
    st = O.push_staging(shards, lay)
    for s in range(3):
        assert np.array_equal(st[s], shards[s])          # contiguous: the stream is the shard itself
    st = O.push_staging(shards, lay, self_shard=1)
    assert st[1] is None and np.array_equal(st[2], shards[2])
    g = _golden("ep_route_tiny.json")
    lay = O.layout_topk(np.array(g["topk"]), g["expert_base"], g["n_local"], row_block=g["row_block"],
                        chunk_rows=g["chunk_rows"])
    sh = [O.f64_to_bf16(rng.standard_normal((3, 2))) for _ in range(2)]
    st = O.push_staging(sh, lay)
    for s in range(2):
        for i, t in enumerate(g["src_row"][s]):           # stream entry i carries token src_row[s][i]
            assert np.array_equal(st[s][i], sh[s][t])
    # the scatter of the staged rows rebuilds the one-stage gather
    G = O.gather(sh, lay)
    for s in range(2):
        for i, d in enumerate(g["dst_row"][s]):
            assert np.array_equal(G[d], st[s][i])


@pytest.mark.parametrize("self_shard", [-1, 0, 2])
def test_two_stage_simulation_matches_closed_form(self_shard):
    rng = np.random.default_rng(40 + self_shard)
    for lay in _layouts_small():
        if self_shard >= lay.n_shards:
            continue
        cap = int(max(-(-lay.stream_len // lay.chunk_rows)))
        state = O.state_after_two_stage(lay, 0, cap, self_shard)
        remote_chunks = sum(-(-int(lay.stream_len[s]) // lay.chunk_rows)
                            for s in range(lay.n_shards) if s != self_shard)
        for t in range(1, 4):
            pb = _push_batches(lay, rng, self_shard)
            sb = _scatter_batches(lay, rng)
            events = [("push", b) for b in range(len(pb))] + [("scatter", b) for b in range(len(sb))]
            events = [events[k] for k in rng.permutation(len(events))]
            r = O.simulate_two_stage(lay, state, t, pb, sb, events, self_shard)
            assert r.early_scatter == 0 and r.early_gates == 0
            assert r.publishes == remote_chunks
            want = O.state_after_two_stage(lay, t, cap, self_shard)
            assert np.array_equal(r.state.slot, want.slot)
            assert np.array_equal(r.state.counter, want.counter)
            assert np.array_equal(r.state.elect, want.elect)
            assert np.array_equal(r.state.pub_count, want.pub_count)
            for s in range(lay.n_shards):
                assert np.all(r.staged[s]) == (s != self_shard) or int(lay.stream_len[s]) == 0


def test_two_stage_missing_push_never_releases_the_scatter():
    lay = O.layout_contiguous(2, 40, row_block=16, chunk_rows=8)
    rng = np.random.default_rng(9)
    cap = int(max(-(-lay.stream_len // lay.chunk_rows)))
    pb = _push_batches(lay, rng, -1)
    sb = _scatter_batches(lay, rng)
    events = [("push", b) for b in range(1, len(pb))] + [("scatter", b) for b in range(len(sb))]
    with pytest.raises(RuntimeError):
        O.simulate_two_stage(lay, O.state_after_two_stage(lay, 0, cap), 1, pb, sb, events)
    # the self shard's rows need no push: dropping its batches changes nothing
    pb1 = _push_batches(lay, rng, 0)
    events = [("push", b) for b in range(len(pb1))] + [("scatter", b) for b in range(len(sb))]
    r = O.simulate_two_stage(lay, O.state_after_two_stage(lay, 0, cap, 0), 1, pb1, sb, events, self_shard=0)
    assert r.early_scatter == 0 and np.all(r.state.counter[1] == lay.row_block)


# ------------------------------------------------------------ streaming FIFO ring

@pytest.mark.parametrize("n_channels,ring_chunks,self_shard", [(1, 1, -1), (2, 1, 0), (3, 2, -1), (2, 3, 2)])
def test_ring_simulation_matches_closed_form(n_channels, ring_chunks, self_shard):
    rng = np.random.default_rng(60 + 7 * n_channels + ring_chunks)
    for lay in _layouts_small():
        if self_shard >= lay.n_shards:
            continue
        for trial in range(3):
            r = O.simulate_ring(lay, n_channels, ring_chunks, rng, self_shard)
            assert r.overwrites == 0 and r.early_reads == 0 and r.early_gates == 0
            assert r.max_occupancy <= ring_chunks
            assert np.array_equal(r.gathered_rows, O.real_rows(lay))
            assert np.all(r.counter == lay.row_block)
            tail, head = O.ring_state_after(lay, n_channels, 1, self_shard)
            assert np.array_equal(r.tail, tail[1]) and np.array_equal(r.head, head[1])
            assert not tail[0].any() and not head[0].any()
    # every chunk of a remote shard travels through exactly one ring, in order
    lay = list(_layouts_small())[2]
    ch = O.ring_chunks_of(lay, n_channels)
    for s in range(lay.n_shards):
        allc = sorted(c for k in range(n_channels) for c in ch[s][k])
        assert allc == list(range(-(-int(lay.stream_len[s]) // lay.chunk_rows)))
        for k in range(n_channels):
            assert ch[s][k] == sorted(ch[s][k]) and all(c % n_channels == k for c in ch[s][k])


def test_ring_planted_credit_mistake_overwrites():
    lay = O.layout_contiguous(2, 200, row_block=16, chunk_rows=8)
    rng = np.random.default_rng(71)
    over = sum(O.simulate_ring(lay, 2, 2, rng, credit_limit=3).overwrites for _ in range(10))
    assert over > 0, "one credit too many must let a producer overwrite an unconsumed slot"
    with pytest.raises(RuntimeError):
        O.simulate_ring(lay, 2, 0, rng)     # no slot: the producer never gets a credit


def test_ring_empty_rings_finish_at_once():
    lay = O.layout_contiguous(2, 10, row_block=16, chunk_rows=8)     # 2 chunks per shard, 4 rings per shard
    rng = np.random.default_rng(72)
    r = O.simulate_ring(lay, 4, 1, rng)
    tail, head = O.ring_state_after(lay, 4, 1)
    assert np.array_equal(r.tail, tail[1])
    assert sum(1 for x in tail[1] if x == O.RING_FINISH) == 4        # rings 2, 3 of each shard carry nothing
