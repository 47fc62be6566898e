"""Property-based pins of the oracle (CPU): invariants that the pages'
definitions fix, checked over many random small inputs."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O

SET = settings(max_examples=40, deadline=None)


@st.composite
def topk_case(draw):
    S = draw(st.integers(1, 3))
    T = draw(st.integers(1, 24))
    E_all = draw(st.integers(2, 12))
    KK = draw(st.integers(1, E_all))
    n_local = draw(st.integers(1, E_all))
    base = draw(st.integers(0, E_all - n_local))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    topk = np.stack([np.stack([rng.permutation(E_all)[:KK] for _ in range(T)]) for _ in range(S)])
    rb = draw(st.sampled_from([4, 8, 16]))
    return topk, base, n_local, rb


@SET
@given(topk_case())
def test_topk_layout_invariants(c):
    topk, base, n_local, rb = c
    lay = O.layout_topk(topk, base, n_local, row_block=rb, chunk_rows=4)
    S, T, KK = topk.shape
    dst = np.concatenate([np.asarray(lay.dst_row[s], dtype=np.int64) for s in range(S)]) if S else np.zeros(0)
    assert len(set(dst.tolist())) == len(dst), "every pick gets its own gathered row"
    assert np.all(lay.group_off % rb == 0) and lay.group_off[0] == 0 and lay.group_off[-1] == lay.m_pad
    for s in range(S):
        picks = [(t, k) for t in range(T) for k in range(KK) if 0 <= topk[s, t, k] - base < n_local]
        assert [int(x) for x in lay.src_row[s]] == [t for t, _ in picks], "stream in (token, k) order"
        for i, (t, k) in enumerate(picks):
            e = int(topk[s, t, k]) - base
            d = int(lay.dst_row[s][i])
            assert lay.group_off[e] <= d < lay.group_off[e + 1], "row inside its expert's group"
    # inside a group, rows follow the global token order
    for e in range(n_local):
        owners = sorted((int(lay.dst_row[s][i]), s * T + int(lay.src_row[s][i]))
                        for s in range(S) for i in range(len(lay.dst_row[s]))
                        if lay.group_off[e] <= int(lay.dst_row[s][i]) < lay.group_off[e + 1])
        assert [g for _, g in owners] == sorted(g for _, g in owners)
        assert [d for d, _ in owners] == list(range(lay.group_off[e], lay.group_off[e] + len(owners)))


@SET
@given(topk_case(), st.integers(0, 2**31 - 1))
def test_gather_and_combine_round_trip(c, seed):
    """Gather by the layout, take each gathered row as the expert output
    (an identity expert) and combine with every weight 1/4: the combine returns
    the token's own row times a quarter of its local pick count, exactly."""
    topk, base, n_local, rb = c
    lay = O.layout_topk(topk, base, n_local, row_block=rb, chunk_rows=4)
    S, T, KK = topk.shape
    rng = np.random.default_rng(seed)
    xs = [O.f64_to_bf16(rng.standard_normal((T, 8))) for _ in range(S)]
    G = O.gather(xs, lay)
    for s in range(S):
        for i, d in enumerate(lay.dst_row[s]):
            assert np.array_equal(G[int(d)], xs[s][int(lay.src_row[s][i])])
    w = np.full((S, T, KK), 0.25, dtype=np.float32)
    y = O.combine(G, w, topk, base, n_local, lay)
    for s in range(S):
        n_loc = np.sum((topk[s] - base >= 0) & (topk[s] - base < n_local), axis=1)
        assert np.array_equal(y[s], O.bf16_to_f64(xs[s]) * (0.25 * n_loc)[:, None])
    st_ = O.combine_staging(G, lay)
    for s in range(S):
        assert np.array_equal(st_[s], G[np.asarray(lay.dst_row[s], dtype=np.int64)])


@SET
@given(st.integers(1, 4), st.integers(1, 90), st.integers(1, 4), st.integers(1, 3), st.integers(-1, 3),
       st.integers(0, 2**31 - 1))
def test_ring_never_overwrites_or_stalls(n_shards, rows, n_channels, ring_chunks, self_shard, seed):
    if self_shard >= n_shards:
        self_shard = -1
    lay = O.layout_contiguous(n_shards, rows, row_block=8, chunk_rows=4)
    r = O.simulate_ring(lay, n_channels, ring_chunks, np.random.default_rng(seed), self_shard)
    assert r.overwrites == 0 and r.early_reads == 0 and r.early_gates == 0
    assert r.max_occupancy <= ring_chunks
    tail, head = O.ring_state_after(lay, n_channels, 1, self_shard)
    assert np.array_equal(r.tail, tail[1]) and np.array_equal(r.head, head[1])
    assert np.all(r.counter == lay.row_block)


@SET
@given(st.integers(1, 4), st.integers(1, 70), st.integers(-1, 3), st.integers(0, 2**31 - 1))
def test_two_stage_any_interleaving(n_shards, rows, self_shard, seed):
    if self_shard >= n_shards:
        self_shard = -1
    rng = np.random.default_rng(seed)
    lay = O.layout_permutation(rng.permutation(n_shards * rows), n_shards, rows, row_block=8, chunk_rows=4)
    cap = int(max(-(-lay.stream_len // lay.chunk_rows)))
    push = []
    for s in range(n_shards):
        if s == self_shard:
            continue
        for c0 in range(0, rows, 4):
            push.append([(s, i) for i in range(c0, min(rows, c0 + 4))])
    rows_g = sorted(int(d) for s in range(n_shards) for d in lay.dst_row[s])
    scat = [rows_g[j:j + 3] for j in range(0, len(rows_g), 3)]
    ev = [("push", b) for b in range(len(push))] + [("scatter", b) for b in range(len(scat))]
    ev = [ev[k] for k in rng.permutation(len(ev))]
    r = O.simulate_two_stage(lay, O.state_after_two_stage(lay, 0, cap, self_shard), 1, push, scat, ev, self_shard)
    assert r.early_scatter == 0 and r.early_gates == 0
    want = O.state_after_two_stage(lay, 1, cap, self_shard)
    assert np.array_equal(r.state.slot, want.slot) and np.array_equal(r.state.counter, want.counter)
