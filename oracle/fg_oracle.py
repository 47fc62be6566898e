"""Plain, slow CPU oracle of the fused gather-GEMM and of its signal protocol.

TEST INFRASTRUCTURE ONLY (see the package docstring). numpy, float64 for all
floating point, Python loops where the definition is a loop.

Pages cited (titles abbreviated):
  "PCIe sync protocols"  = Compute-comm fused operators (4): cross-card sync
                           protocols over PCIe -- single writer, election, watermark
  "Know your platform"   = Compute-comm fused operators (2): know your platform
  "NVLink atomic publish" = hardware atomic publish and monotonic counters over NVLink
  "DeepEP FIFO pipeline" = DeepEP v2 FIFO / streaming pipeline analysis

Where the pages leave a step open, the reading taken is stated in the docstring
of the function that takes it, under a label (R1, R2, ...) that later
docstrings use to refer back to it.

Every function here is pinned by tests against closed forms, invariants, hand
worked examples, library special cases or brute force, except the latency
figures, which are measurements only.
"""
from __future__ import annotations

import dataclasses
import itertools
import math

import numpy as np

CHUNK_ROWS = 64     # PCIe sync protocols §4: the watermark cuts each producer stream every 64 rows
ROW_BLOCK = 128     # PCIe sync protocols §5: the GEMM gate releases 128 gathered rows at a time

BF16_MAX = float.fromhex("0x1.fep127")


# ---------------------------------------------------------------------------
# bf16 <-> float64 (the contraction's inputs are bf16; the oracle computes in fp64)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Exact decode: a bf16 is the upper half of a float32."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 to bf16 bits, nearest with ties to even, in one step
    (no intermediate float32, so no double rounding). NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(ax)                       # ax = m * 2**e, m in [0.5, 1)
        e = np.maximum(e, -125)                    # below 2**-126 the grid is 2**-133
        q = np.ldexp(ax, (8 - e).astype(np.int32))  # bf16 grid points become integers
        y = np.ldexp(np.rint(q), (e - 8).astype(np.int32))  # rint = round half to even
        y = np.where(y > BF16_MAX, np.inf, y)
        y = np.where(np.isinf(ax), np.inf, y)
    bits = (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = bits | (np.signbit(x).astype(np.uint16) << np.uint16(15))
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of the bf16 grid at |x| (8 significant bits): 2**(e - 8) for
    |x| = m * 2**e with m in [0.5, 1); from 2**-126 down to zero the grid is the
    subnormal step 2**-133. frexp reports e = 0 for zero, so zero is mapped to
    the subnormal exponent explicitly."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)
    e = np.where(ax == 0.0, -125, np.maximum(e, -125))
    return np.ldexp(1.0, (e - 8).astype(np.int32))


# ---------------------------------------------------------------------------
# Layout / route (step a1): which source row lands on which gathered row
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Layout:
    """Per shard s a stream of (src_row, dst_row) pairs in stream order; the
    stream is what the producer emits and what the chunk watermark cuts
    (PCIe sync protocols §4)."""
    src_row: list           # n_shards arrays (int64)
    dst_row: list           # n_shards arrays (int64)
    m_pad: int              # gathered rows, a multiple of row_block
    group_off: np.ndarray   # [n_groups + 1] first gathered row of each group, multiples of row_block
    row_block: int = ROW_BLOCK
    chunk_rows: int = CHUNK_ROWS

    @property
    def n_shards(self) -> int:
        return len(self.src_row)

    @property
    def stream_len(self) -> np.ndarray:
        return np.array([len(d) for d in self.dst_row], dtype=np.int64)

    @property
    def m(self) -> int:
        return int(self.stream_len.sum())

    @property
    def n_rb(self) -> int:
        return self.m_pad // self.row_block

    @property
    def n_groups(self) -> int:
        return len(self.group_off) - 1


def _round_up(x: int, b: int) -> int:
    return -(-x // b) * b


def layout_contiguous(n_shards: int, rows: int, row_block: int = ROW_BLOCK,
                      chunk_rows: int = CHUNK_ROWS) -> Layout:
    """All-gather layout: shard s's row i lands on gathered row s*rows + i."""
    src = [np.arange(rows, dtype=np.int64) for _ in range(n_shards)]
    dst = [s * rows + np.arange(rows, dtype=np.int64) for s in range(n_shards)]
    m_pad = _round_up(n_shards * rows, row_block)
    return Layout(src, dst, m_pad, np.array([0, m_pad], dtype=np.int64), row_block, chunk_rows)


def layout_permutation(perm, n_shards: int, rows: int, row_block: int = ROW_BLOCK,
                       chunk_rows: int = CHUNK_ROWS) -> Layout:
    """Scattered all-gather: stream row (s, i) lands on gathered row perm[s*rows + i]."""
    perm = np.asarray(perm, dtype=np.int64)
    assert perm.shape == (n_shards * rows,)
    src = [np.arange(rows, dtype=np.int64) for _ in range(n_shards)]
    dst = [perm[s * rows:(s + 1) * rows].copy() for s in range(n_shards)]
    m_pad = _round_up(n_shards * rows, row_block)
    lay = Layout(src, dst, m_pad, np.array([0, m_pad], dtype=np.int64), row_block, chunk_rows)
    check_layout(lay)
    return lay


def layout_topk(topk, expert_base: int, n_local: int, row_block: int = ROW_BLOCK,
                chunk_rows: int = CHUNK_ROWS) -> Layout:
    """Expert-parallel dispatch layout (the "notify" counting stage of the DeepEP
    FIFO pipeline dispatch, with the padding rule of PCIe sync protocols §5).

    Reading R11: source shard s, token t, choice k routes to local expert
    e = topk[s][t][k] - expert_base when that lies in [0, n_local). Each shard's
    stream lists its pairs in (t, k) order. Inside expert e, rows are ordered by
    global token id g = s*T + t; expert e's rows start at off_e, where off_0 = 0 and
    off_{e+1} = off_e + ceil(n_e / row_block) * row_block, so no row block spans
    two experts and every padding row is at the end of its expert's segment.
    """
    topk = np.asarray(topk, dtype=np.int64)
    S, T, KK = topk.shape
    pairs = []                                   # (s, t, e) in (s, t, k) order = global token order
    for s in range(S):
        for t in range(T):
            for k in range(KK):
                e = int(topk[s, t, k]) - expert_base
                if 0 <= e < n_local:
                    pairs.append((s, t, e))
    n_e = [0] * n_local
    for (_, _, e) in pairs:
        n_e[e] += 1
    off = [0]
    for e in range(n_local):
        off.append(off[-1] + _round_up(n_e[e], row_block))
    cursor = off[:-1]
    src = [[] for _ in range(S)]
    dst = [[] for _ in range(S)]
    for (s, t, e) in pairs:
        src[s].append(t)
        dst[s].append(cursor[e])
        cursor[e] += 1
    lay = Layout([np.array(x, dtype=np.int64) for x in src],
                 [np.array(x, dtype=np.int64) for x in dst],
                 off[-1], np.array(off, dtype=np.int64), row_block, chunk_rows)
    check_layout(lay)
    return lay


def check_layout(lay: Layout) -> None:
    """dst rows are injective and in range; no group straddles a row block."""
    d = np.concatenate(lay.dst_row) if lay.n_shards else np.zeros(0, np.int64)
    assert d.size == 0 or (d.min() >= 0 and d.max() < lay.m_pad)
    assert np.unique(d).size == d.size, "two stream rows target one gathered row"
    assert np.all(lay.group_off % lay.row_block == 0)


def group_of_row(lay: Layout) -> np.ndarray:
    """Group (expert) index of every gathered row."""
    g = np.zeros(lay.m_pad, dtype=np.int64)
    for i in range(lay.n_groups):
        g[lay.group_off[i]:lay.group_off[i + 1]] = i
    return g


def real_rows(lay: Layout) -> np.ndarray:
    """Boolean [m_pad]: True where a stream row lands (False = padding row)."""
    r = np.zeros(lay.m_pad, dtype=bool)
    for d in lay.dst_row:
        r[d] = True
    return r


# ---------------------------------------------------------------------------
# Gather (step a3): a bitwise row copy
# ---------------------------------------------------------------------------

def gather(shards_bits, lay: Layout) -> np.ndarray:
    """G[dst_row[s][i]] = X_s[src_row[s][i]] bit for bit; padding rows stay +0.
    ``shards_bits``: n_shards uint16 arrays [rows, K] (bf16 bit patterns)."""
    K = shards_bits[0].shape[1]
    G = np.zeros((lay.m_pad, K), dtype=np.uint16)
    for s in range(lay.n_shards):
        for src, dst in zip(lay.src_row[s], lay.dst_row[s]):
            G[dst] = shards_bits[s][src]
    return G


# ---------------------------------------------------------------------------
# Closed forms of the protocol (PCIe sync protocols §2 point 2: writer counts and
# signal counts must have a closed form; §4 chunk watermark; §5 seeded counters)
# ---------------------------------------------------------------------------

def chunk_table(lay: Layout) -> list:
    """expected[s][c] = rows of stream s in chunk c = min(chunk, n_s - chunk*c)."""
    out = []
    for n in lay.stream_len:
        n = int(n)
        out.append(np.array([min(lay.chunk_rows, n - lay.chunk_rows * c)
                             for c in range(-(-n // lay.chunk_rows))], dtype=np.int64))
    return out


def seeds(lay: Layout) -> np.ndarray:
    """Padding seed per row block: row_block minus the real rows landing in it,
    so real arrivals lift the counter to exactly row_block (PCIe sync protocols §5)."""
    real = np.zeros(lay.n_rb, dtype=np.int64)
    for d in lay.dst_row:
        for r in d:
            real[r // lay.row_block] += 1
    return lay.row_block - real


def signal_counts(lay: Layout) -> dict:
    """Per-iteration closed forms."""
    n = lay.stream_len
    return dict(
        publishes=int(sum(-(-int(x) // lay.chunk_rows) for x in n)),
        arrivals=int(n.sum()),
        gate_openings=lay.n_rb,
        seed_sum=lay.m_pad - int(n.sum()),
        publishers_per_chunk=1,
    )


@dataclasses.dataclass
class ProtocolState:
    slot: np.ndarray        # [S, chunk_cap]   monotonic sequence numbers, never reset
    counter: np.ndarray     # [2, n_rb]        parity double-buffered arrival counters
    elect: np.ndarray       # [2, S, chunk_cap] parity double-buffered election counts
    pub_count: np.ndarray   # [S, chunk_cap]   publishes seen per slot


def state_after(lay: Layout, t: int, chunk_cap: int) -> ProtocolState:
    """Control-plane state after iterations 1..t over one fixed layout.

    PCIe sync protocols §2 point 1: the slot of iteration k holds k and is never
    cleared. Reading R4: counters and election counts are double-buffered by the
    parity of the iteration (the phase trick of the DeepEP FIFO pipeline barrier):
    iteration t consumes parity t&1 and re-arms parity (t+1)&1 (counters to the
    seed, election counts to 0); before iteration 1 both parities hold the seed.
    """
    S = lay.n_shards
    exp = chunk_table(lay)
    sd = seeds(lay)
    slot = np.zeros((S, chunk_cap), dtype=np.int64)
    elect = np.zeros((2, S, chunk_cap), dtype=np.int64)
    pub = np.zeros((S, chunk_cap), dtype=np.int64)
    counter = np.zeros((2, lay.n_rb), dtype=np.int64)
    counter[0] = sd
    counter[1] = sd
    if t >= 1:
        for s in range(S):
            nc = len(exp[s])
            slot[s, :nc] = t
            pub[s, :nc] = t
            elect[t & 1, s, :nc] = exp[s]
        counter[t & 1] = lay.row_block
        counter[(t + 1) & 1] = sd
    return ProtocolState(slot, counter, elect, pub)


# ---------------------------------------------------------------------------
# Step-by-step protocol simulation (the pages' steps in their order), used to pin
# the closed forms above; Python loops, small inputs only.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class SimResult:
    state: ProtocolState
    publishes: int
    arrivals: int
    gate_openings: int
    early_gates: int        # gate opened while a real row of its block was unwritten
    early_publishes: int    # chunk published while one of its rows was unwritten


def simulate_iteration(lay: Layout, state: ProtocolState, t: int, batches, order,
                       seed_vec=None) -> SimResult:
    """One iteration of the comm side, batch by batch.

    ``batches``: list of lists of (s, i) stream rows; each batch is what one wave
    moves before it signals. ``order``: the order in which batches complete.
    For each batch, in order (PCIe sync protocols §3 and §5):
      1. write its rows into the gathered buffer;
      2. per row block it touched, add its row count to the block's counter;
      3. per chunk it touched, add its row count to the chunk's election count;
         the add that brings the count to the chunk's expected size elects the
         batch, which stores t into the chunk's slot (single writer).
    A gate opens the first time its counter equals row_block. At the end, the
    other parity is re-armed (reading R4). ``seed_vec`` overrides the seed used to
    re-arm (to plant a mistake).
    """
    p = t & 1
    exp = chunk_table(lay)
    rb_of = lambda d: d // lay.row_block  # noqa: E731
    written = np.zeros(lay.m_pad, dtype=bool)
    real = real_rows(lay)
    chunk_rows_written = {}
    opened = np.zeros(lay.n_rb, dtype=bool)
    pubs = arr = gates = early_g = early_p = 0
    for b in order:
        rows = batches[b]
        for (s, i) in rows:
            written[lay.dst_row[s][i]] = True
        per_rb = {}
        per_chunk = {}
        for (s, i) in rows:
            r = int(rb_of(lay.dst_row[s][i]))
            per_rb[r] = per_rb.get(r, 0) + 1
            c = (s, i // lay.chunk_rows)
            per_chunk[c] = per_chunk.get(c, 0) + 1
        for r, n in per_rb.items():
            state.counter[p, r] += n
            arr += n
            if state.counter[p, r] == lay.row_block and not opened[r]:
                opened[r] = True
                gates += 1
                blk = slice(r * lay.row_block, (r + 1) * lay.row_block)
                if np.any(real[blk] & ~written[blk]):
                    early_g += 1
        for (s, c), n in per_chunk.items():
            chunk_rows_written[(s, c)] = chunk_rows_written.get((s, c), 0) + n
            old = state.elect[p, s, c]
            state.elect[p, s, c] = old + n
            if old + n == exp[s][c]:
                state.slot[s, c] = t
                state.pub_count[s, c] += 1
                pubs += 1
                lo = c * lay.chunk_rows
                d = lay.dst_row[s][lo:lo + exp[s][c]]
                if not np.all(written[d]):
                    early_p += 1
    q = (t + 1) & 1
    state.counter[q] = seeds(lay) if seed_vec is None else seed_vec
    state.elect[q] = 0
    return SimResult(state, pubs, arr, gates, early_g, early_p)


# ---------------------------------------------------------------------------
# Two-stage dispatch ("PCIe sync protocols" §4 chunk watermark: each producer
# stream is cut into 64-row chunks and the chunk's slot is the watermark the
# receiver waits on; §6 audit item 2: the receiver's scatter waits only on the
# remote watermarks and reads its own shard directly). Stage 1 pushes every
# stream row of a remote shard into that shard's staging buffer in stream
# order and publishes the chunk watermarks; stage 2 scatters rows into the
# gathered buffer, after the watermark of their chunk, and counts arrivals
# into the seeded 128-row counters of §5.
# ---------------------------------------------------------------------------

def push_staging(shards_bits, lay: Layout, self_shard: int = -1) -> list:
    """staging[s][i] = shard_s[src_row[s][i]] bitwise for every shard other
    than ``self_shard`` (reading R27); the self shard has no staging rows."""
    out = []
    for s in range(lay.n_shards):
        if s == self_shard:
            out.append(None)
            continue
        X = np.asarray(shards_bits[s])
        out.append(X[np.asarray(lay.src_row[s], dtype=np.int64)])
    return out


def state_after_two_stage(lay: Layout, t: int, chunk_cap: int, self_shard: int = -1) -> ProtocolState:
    """Control plane after t iterations of the two-stage dispatch (reading R27):
    the pushes publish the slot of every chunk of every remote shard, as the
    one-stage copy does, and the scatter brings every 128-row counter to 128;
    the self shard is never pushed, so its slots, election counts and
    publisher counts stay 0."""
    st = state_after(lay, t, chunk_cap)
    if 0 <= self_shard < lay.n_shards:
        st.slot[self_shard] = 0
        st.elect[:, self_shard] = 0
        st.pub_count[self_shard] = 0
    return st


@dataclasses.dataclass
class TwoStageResult:
    state: ProtocolState
    staged: list             # staging rows written, per shard (bool per stream entry)
    publishes: int
    early_scatter: int       # a row scattered from staging before the row was pushed
    early_gates: int         # a gate opened while one of its real rows was unscattered
    deferred: int            # scatter steps that found a watermark not yet published


def simulate_two_stage(lay: Layout, state: ProtocolState, t: int, push_batches, scatter_batches, events,
                       self_shard: int = -1) -> TwoStageResult:
    """One iteration, event by event. ``push_batches``: lists of (s, i) stream
    entries of remote shards, each inside one chunk; ``scatter_batches``: lists
    of gathered rows; ``events``: a sequence of ("push", b) and ("scatter", b).
      push b: write the batch's staging rows, add its row count to the chunk's
        election count; the add that completes the chunk stores t into its slot;
      scatter b: if a remote row of the batch has a chunk whose slot is not yet
        t, the step is deferred to the end of the sequence (the watermark wait);
        otherwise copy every row (remote rows from staging, self-shard rows from
        the shard) into the gathered buffer and add the rows per block to the
        counters; a gate opens when its counter reaches 128.
    At the end the other parity is re-armed (reading R4)."""
    p = t & 1
    exp = chunk_table(lay)
    inv = {}
    for s in range(lay.n_shards):
        for i, d in enumerate(lay.dst_row[s]):
            inv[int(d)] = (s, i)
    staged = [np.zeros(len(lay.src_row[s]), dtype=bool) for s in range(lay.n_shards)]
    written = np.zeros(lay.m_pad, dtype=bool)
    real = real_rows(lay)
    opened = np.zeros(lay.n_rb, dtype=bool)
    pubs = early_s = early_g = deferred = 0
    queue = list(events)
    k = 0
    stall = 0            # deferrals since the last step that ran
    while k < len(queue):
        kind, b = queue[k]
        k += 1
        if kind == "push":
            stall = 0
            rows = push_batches[b]
            for (s, i) in rows:
                staged[s][i] = True
            s, c = rows[0][0], rows[0][1] // lay.chunk_rows
            old = state.elect[p, s, c]
            state.elect[p, s, c] = old + len(rows)
            if old + len(rows) == exp[s][c]:
                state.slot[s, c] = t
                state.pub_count[s, c] += 1
                pubs += 1
            continue
        rows = scatter_batches[b]
        ready = True
        for g in rows:
            s, i = inv[g]
            if s != self_shard and state.slot[s, i // lay.chunk_rows] != t:
                ready = False
        if not ready:
            deferred += 1
            stall += 1
            queue.append((kind, b))
            if stall > len(queue) - k:      # a full pass over the pending steps ran nothing
                raise RuntimeError("scatter waits on a watermark no push publishes")
            continue
        stall = 0
        per_rb = {}
        for g in rows:
            s, i = inv[g]
            if s != self_shard and not staged[s][i]:
                early_s += 1
            written[g] = True
            r = g // lay.row_block
            per_rb[r] = per_rb.get(r, 0) + 1
        for r, n in per_rb.items():
            state.counter[p, r] += n
            if state.counter[p, r] == lay.row_block and not opened[r]:
                opened[r] = True
                blk = slice(r * lay.row_block, (r + 1) * lay.row_block)
                if np.any(real[blk] & ~written[blk]):
                    early_g += 1
    q = (t + 1) & 1
    state.counter[q] = seeds(lay)
    state.elect[q] = 0
    return TwoStageResult(state, staged, pubs, early_s, early_g, deferred)


# ---------------------------------------------------------------------------
# Streaming FIFO ring ("DeepEP FIFO pipeline": a bounded ring per channel, the
# sender waits until tail - head < capacity, writes slot tail mod capacity and
# advances tail; the receiver polls tail, consumes, and returns credit by
# advancing head; the sender's last tail carries a finish flag packed with it).
# Reading R28: each shard's stream of 64-row chunks is dealt to n_channels
# rings (chunk c to ring c mod n_channels, in increasing c); each ring has one
# producer and one consumer and ring_chunks chunk slots. The consumer scatters
# a consumed chunk into the gathered buffer and counts its rows into the
# seeded 128-row counters. A self shard is read straight from the shard.
# ---------------------------------------------------------------------------

RING_FINISH = 1 << 32


def ring_chunks_of(lay: Layout, n_channels: int) -> list:
    """chunks[s][k] = the chunk indices ring (s, k) carries, in order."""
    out = []
    for s in range(lay.n_shards):
        n = -(-int(lay.stream_len[s]) // lay.chunk_rows)
        out.append([list(range(k, n, n_channels)) for k in range(n_channels)])
    return out


def ring_state_after(lay: Layout, n_channels: int, t: int, self_shard: int = -1):
    """(tail, head) words after t iterations, [2][S * n_channels] each, parity
    double-buffered as in reading R4: iteration t leaves parity t & 1 with
    tail = finish | chunks and head = chunks for every ring of a remote shard
    (0 for the self shard's rings, which are never used) and re-arms the other
    parity to 0."""
    S = lay.n_shards
    tail = np.zeros((2, S * n_channels), dtype=np.int64)
    head = np.zeros((2, S * n_channels), dtype=np.int64)
    if t >= 1:
        ch = ring_chunks_of(lay, n_channels)
        for s in range(S):
            if s == self_shard:
                continue
            for k in range(n_channels):
                tail[t & 1, s * n_channels + k] = RING_FINISH | len(ch[s][k])
                head[t & 1, s * n_channels + k] = len(ch[s][k])
    return tail, head


@dataclasses.dataclass
class RingResult:
    gathered_rows: np.ndarray   # bool per gathered row: written by a consumer
    counter: np.ndarray         # [n_rb] arrival counters after the iteration
    tail: np.ndarray            # [S * n_channels]
    head: np.ndarray
    max_occupancy: int          # largest tail - head seen on any ring
    overwrites: int             # a slot rewritten before its chunk was consumed
    early_reads: int            # a consumer read a slot before its chunk was written
    early_gates: int
    steps: int


def simulate_ring(lay: Layout, n_channels: int, ring_chunks: int, rng, self_shard: int = -1,
                  credit_limit=None) -> RingResult:
    """One iteration, one ring step at a time in a random order. A producer step
    of ring r writes its next chunk j into slot j mod ring_chunks if
    tail - head < credit_limit (the capacity unless a mistake is planted), then
    sets tail = j + 1 (with the finish flag on the ring's last chunk, or at once
    for a ring with no chunk). A consumer step reads chunk j from its slot if
    tail > j, scatters its rows, counts them per 128-row block and sets
    head = j + 1. Self-shard rings have no producer: their consumer reads the
    shard directly. Raises if no step can run while work remains."""
    cap = ring_chunks if credit_limit is None else credit_limit
    S = lay.n_shards
    ch = ring_chunks_of(lay, n_channels)
    R = S * n_channels
    tail = np.zeros(R, dtype=np.int64)
    head = np.zeros(R, dtype=np.int64)
    slot = {}                                   # (ring, slot index) -> chunk index written there
    written_rows = np.zeros(lay.m_pad, dtype=bool)
    counter = seeds(lay).astype(np.int64).copy()
    real = real_rows(lay)
    opened = np.zeros(lay.n_rb, dtype=bool)
    occ = over = early = early_g = steps = 0
    cons = np.zeros(R, dtype=np.int64)          # chunks consumed per ring
    for s in range(S):
        for k in range(n_channels):
            r = s * n_channels + k
            if s != self_shard and not ch[s][k]:
                tail[r] = RING_FINISH
    while True:
        moves = []
        for r in range(R):
            s, k = divmod(r, n_channels)
            n = len(ch[s][k])
            if s != self_shard and (tail[r] & 0xFFFFFFFF) < n and (tail[r] & 0xFFFFFFFF) - head[r] < cap:
                moves.append(("p", r))
            if cons[r] < n and (s == self_shard or (tail[r] & 0xFFFFFFFF) > cons[r]):
                moves.append(("c", r))
        if not moves:
            break
        kind, r = moves[int(rng.integers(len(moves)))]
        s, k = divmod(r, n_channels)
        n = len(ch[s][k])
        steps += 1
        if kind == "p":
            j = int(tail[r] & 0xFFFFFFFF)
            key = (r, j % ring_chunks)
            if key in slot and slot[key] >= cons[r]:
                over += 1                        # that chunk was not consumed yet
            slot[key] = j
            tail[r] = (j + 1) | (RING_FINISH if j + 1 == n else 0)
            occ = max(occ, j + 1 - int(head[r]))
            continue
        j = int(cons[r])
        if s != self_shard and slot.get((r, j % ring_chunks)) != j:
            early += 1
        c = ch[s][k][j]
        lo, hi = c * lay.chunk_rows, min(int(lay.stream_len[s]), (c + 1) * lay.chunk_rows)
        per_rb = {}
        for i in range(lo, hi):
            d = int(lay.dst_row[s][i])
            written_rows[d] = True
            per_rb[d // lay.row_block] = per_rb.get(d // lay.row_block, 0) + 1
        for rb, m in per_rb.items():
            counter[rb] += m
            if counter[rb] == lay.row_block and not opened[rb]:
                opened[rb] = True
                blk = slice(rb * lay.row_block, (rb + 1) * lay.row_block)
                if np.any(real[blk] & ~written_rows[blk]):
                    early_g += 1
        cons[r] = j + 1
        if s != self_shard:
            head[r] = j + 1
    done = all(cons[s * n_channels + k] == len(ch[s][k]) for s in range(S) for k in range(n_channels))
    if not done:
        raise RuntimeError("the ring stalled with chunks left")
    return RingResult(written_rows, counter, tail, head, occ, over, early, early_g, steps)


def election_brute_force(parts) -> int:
    """A chunk of sum(parts) rows finished by len(parts) waves, wave w adding
    parts[w]: over every completion order, count the adds that see
    old + n == expected. The election is sound iff this is exactly 1 for every
    order (PCIe sync protocols §3). Returns the number of orders that break it."""
    expected = sum(parts)
    bad = 0
    for order in itertools.permutations(range(len(parts))):
        total = 0
        elected = 0
        for w in order:
            old = total
            total += parts[w]
            if old + parts[w] == expected:
                elected += 1
        bad += (elected != 1)
    return bad


def model_check_gate(programs, seed: int, target: int) -> int:
    """Exhaustive interleavings of a toy sequentially consistent protocol.

    ``programs``: one list of steps per producer; a step is ('w', row) to write a
    row or ('a', n) to add n to the gate counter. The counter starts at ``seed``;
    the consumer may check the gate between any two steps. Returns the number of
    interleavings in which the consumer sees counter == target while some row is
    unwritten (PCIe sync protocols §5: the gate must imply the data)."""
    rows = {st[1] for p in programs for st in p if st[0] == 'w'}
    lens = [len(p) for p in programs]
    bad = 0
    seqs = []
    for pi, n in enumerate(lens):
        seqs += [pi] * n
    for perm in set(itertools.permutations(seqs)):
        pos = [0] * len(programs)
        ctr = seed
        done = set()
        violated = False
        for pi in perm:
            op, v = programs[pi][pos[pi]]
            pos[pi] += 1
            if op == 'w':
                done.add(v)
            else:
                ctr += v
            if ctr == target and done != rows:
                violated = True
        bad += violated
    return bad


# ---------------------------------------------------------------------------
# The contraction (step a7)
# ---------------------------------------------------------------------------

def gemm(G_bits, W_bits, lay: Layout, rows=None) -> np.ndarray:
    """C[m, n] = sum_k G[m, k] * W_g(m)[k, n] in float64 (exact bf16 decode).

    ``W_bits``: uint16 [n_groups, N, K] holding W_g[k, n] at [g, n, k] (the
    logical K x N weight stored contraction-index contiguous).
    ``rows``: optional subset of gathered rows to compute (default: all).
    Padding rows yield 0 (their gathered row is 0)."""
    G = bf16_to_f64(G_bits if rows is None else G_bits[rows])
    grp = group_of_row(lay) if rows is None else group_of_row(lay)[rows]
    W = np.asarray(W_bits)
    if W.ndim == 2:
        W = W[None]
    N = W.shape[1]
    C = np.zeros((G.shape[0], N), dtype=np.float64)
    for g in range(W.shape[0]):
        sel = np.nonzero(grp == g)[0]
        if sel.size:
            C[sel] = G[sel] @ bf16_to_f64(W[g]).T
    if rows is None:
        C[~real_rows(lay)] = 0.0
    else:
        C[~real_rows(lay)[rows]] = 0.0
    return C


def gemm_tolerance(K: int, sigma_x: float, sigma_w: float) -> float:
    """Stated tolerance on the contraction: 2e-2 of the output's standard
    deviation sqrt(K) * sigma_x * sigma_w (reading R14)."""
    return 2e-2 * math.sqrt(K) * sigma_x * sigma_w


def gemm_check(out_bits, C64, K, sigma_x, sigma_w, real_mask=None) -> dict:
    """Compare bf16 GPU output with the float64 result. Pass iff every element
    satisfies |out - C| <= tol + ulp_bf16(C)/2, where tol is the stated
    contraction tolerance and the half ulp is the output's own round-to-nearest
    (reading R14); padding rows must be exactly 0 (either sign)."""
    out = bf16_to_f64(out_bits)
    tol = gemm_tolerance(K, sigma_x, sigma_w)
    diff = np.abs(out - C64)
    allow = tol + 0.5 * bf16_ulp(C64)
    ok_mask = diff <= allow
    if real_mask is not None:
        ok_mask[~real_mask] = (out[~real_mask] == 0.0)
    rms = float(np.sqrt(np.mean(C64 ** 2))) if C64.size else 0.0
    return dict(ok=bool(ok_mask.all()), n_bad=int((~ok_mask).sum()),
                max_abs=float(diff.max()) if diff.size else 0.0, tol=tol,
                max_over_scale=float(diff.max() / (tol / 2e-2)) if diff.size else 0.0,
                max_over_rms=float(diff.max() / rms) if rms else 0.0)


# ---------------------------------------------------------------------------
# Combine: the reverse of the expert dispatch ("PCIe sync protocols" §3: the
# producers' rows are pushed to the destination's staging buffer and the last
# writer of each 64-row chunk, elected by a local count, publishes its slot;
# the destination then sums each token's expert rows with its gate weights)
# ---------------------------------------------------------------------------

def combine_picks(topk, expert_base: int, n_local: int) -> list:
    """Per shard s, the stream of local picks in stream order (reading R11:
    tokens ascending, then their top-k choices in list order), as (t, k) pairs.
    Stream entry i of shard s is the i-th pair; it is the same stream as
    ``layout_topk``'s."""
    topk = np.asarray(topk, dtype=np.int64)
    S, T, KK = topk.shape
    out = []
    for s in range(S):
        pairs = []
        for t in range(T):
            for k in range(KK):
                if 0 <= int(topk[s, t, k]) - expert_base < n_local:
                    pairs.append((t, k))
        out.append(pairs)
    return out


def combine_staging(out_bits, lay: Layout) -> list:
    """Pushed rows, per shard in stream order: staging[s][i] = out[dst_row[s][i]]
    bitwise (reading R25: the staging buffer is the destination rank's receive
    buffer, indexed by the destination's stream entry)."""
    out_bits = np.asarray(out_bits)
    return [out_bits[np.asarray(lay.dst_row[s], dtype=np.int64)] for s in range(lay.n_shards)]


def combine(out_bits, weights, topk, expert_base: int, n_local: int, lay: Layout) -> np.ndarray:
    """y[s][t][n] = sum over the local picks (t, k) of shard s of
    weights[s][t][k] * out[g(s, t, k)][n], in float64 with bf16 outputs and fp32
    weights decoded exactly; tokens without a local pick give 0 (reading R25:
    on this GPU only the local experts' contributions are summed). g(s, t, k) is
    the gathered row the dispatch gave pick (t, k) of shard s."""
    out = bf16_to_f64(out_bits)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    picks = combine_picks(topk, expert_base, n_local)
    S, T, _ = np.asarray(topk).shape
    N = out.shape[1]
    y = np.zeros((S, T, N), dtype=np.float64)
    for s in range(S):
        for i, (t, k) in enumerate(picks[s]):
            g = int(lay.dst_row[s][i])
            y[s, t] += w[s, t, k] * out[g]
    return y


def combine_tolerance(out_bits, weights, topk, expert_base: int, n_local: int, lay: Layout) -> np.ndarray:
    """Per element bound for a float32 weighted sum of at most KK terms rounded
    once to bf16 (reading R26): half a bf16 ulp of the exact sum plus
    KK * 2^-23 times the sum of the terms' magnitudes (float32 products and adds)."""
    out = np.abs(bf16_to_f64(out_bits))
    w = np.abs(np.asarray(weights, dtype=np.float32).astype(np.float64))
    picks = combine_picks(topk, expert_base, n_local)
    S, T, KK = np.asarray(topk).shape
    mag = np.zeros((S, T, out.shape[1]), dtype=np.float64)
    for s in range(S):
        for i, (t, k) in enumerate(picks[s]):
            mag[s, t] += w[s, t, k] * out[int(lay.dst_row[s][i])]
    y = combine(out_bits, weights, topk, expert_base, n_local, lay)
    return 0.5 * bf16_ulp(y) + KK * 2.0 ** -23 * mag


# ---------------------------------------------------------------------------
# Protocol stress workload (PCIe sync protocols §3: tens of thousands of
# signals per round over dozens of rounds; §4 chunked slots)
# ---------------------------------------------------------------------------

def stress_payload(seq: int, p: int, c: int, k: int, r: int, C: int, KC: int) -> int:
    """The 4-byte word a producer writes for row r of chunk (p, c, k) at
    iteration ``seq`` (reading R13): the iteration in the top bits, the row's
    unique index below, so a stale row is visible."""
    idx = ((p * C + c) * KC + k) * CHUNK_ROWS + r
    return ((seq << 20) ^ idx) & 0xFFFFFFFF


def stress_expected(chunk_rows, t: int) -> dict:
    """After iterations 1..t: slot = t and pub_count = t where a chunk is active,
    0 elsewhere; every written payload row holds iteration t's word. Independent
    of the producers' delays."""
    cr = np.asarray(chunk_rows, dtype=np.int64)
    P, C, KC = cr.shape
    active = cr > 0
    slot = np.where(active, t, 0)
    payload = np.zeros((C, P, KC, CHUNK_ROWS), dtype=np.uint32)
    valid = np.zeros((C, P, KC, CHUNK_ROWS), dtype=bool)
    if t >= 1:
        for p in range(P):
            for c in range(C):
                for k in range(KC):
                    for r in range(int(cr[p, c, k])):
                        payload[c, p, k, r] = stress_payload(t, p, c, k, r, C, KC)
                        valid[c, p, k, r] = True
    return dict(slot=slot, pub_count=slot.copy(), payload=payload, valid=valid,
                signals=int(active.sum()))


def stress_simulate(chunk_rows, t: int, delays, waves: int = 4) -> dict:
    """Event-order simulation of one stress iteration: producers' chunks complete
    in the order of their delays (ties by index); each chunk is written by
    ``waves`` waves that elect one publisher; consumers check each chunk's rows
    after seeing its slot. Returns slots, publisher counts and stale rows."""
    cr = np.asarray(chunk_rows, dtype=np.int64)
    P, C, KC = cr.shape
    d = np.asarray(delays, dtype=np.int64)
    slot = np.zeros((P, C, KC), dtype=np.int64)
    pubs = np.zeros((P, C, KC), dtype=np.int64)
    mem = {}
    events = sorted(((int(d[p, c, k]), p, c, k) for p in range(P) for c in range(C)
                     for k in range(KC) if cr[p, c, k] > 0))
    for (_, p, c, k) in events:
        n = int(cr[p, c, k])
        per = [len(range(w, n, waves)) for w in range(waves)]
        total = 0
        for w in range(waves):
            for r in range(w, n, waves):
                mem[(c, p, k, r)] = stress_payload(t, p, c, k, r, C, KC)
            if per[w] == 0:
                continue
            old = total
            total += per[w]
            if old + per[w] == n:
                slot[p, c, k] = t
                pubs[p, c, k] += 1
    stale = 0
    for p in range(P):
        for c in range(C):
            for k in range(KC):
                if slot[p, c, k] >= t:
                    for r in range(int(cr[p, c, k])):
                        stale += mem.get((c, p, k, r)) != stress_payload(t, p, c, k, r, C, KC)
    return dict(slot=slot, pubs=pubs, stale=stale)


# ---------------------------------------------------------------------------
# Slot barrier (PCIe sync protocols §2: every rank owns one slot on every rank)
# ---------------------------------------------------------------------------

def barrier_expected(n_ranks: int, rounds: int) -> np.ndarray:
    """After ``rounds`` barriers: bslot[j][i] = rounds for every rank pair."""
    return np.full((n_ranks, n_ranks), rounds, dtype=np.int64)


def barrier_simulate(n_ranks: int, rounds: int, order_seed: int = 0) -> np.ndarray:
    """Ranks run rounds with a random interleaving of their slot stores; rank i
    leaves round b only when every bslot[i][j] >= b. Returns the final slots."""
    rng = np.random.default_rng(order_seed)
    bslot = np.zeros((n_ranks, n_ranks), dtype=np.int64)
    rnd = [1] * n_ranks          # round each rank is in
    stored = [False] * n_ranks
    while min(rnd) <= rounds:
        i = int(rng.integers(n_ranks))
        b = rnd[i]
        if b > rounds:
            continue
        if not stored[i]:
            for j in range(n_ranks):     # signal: my slot on every rank
                bslot[j][i] = b
            stored[i] = True
        elif all(bslot[i][j] >= b for j in range(n_ranks)):
            rnd[i] = b + 1
            stored[i] = False
    return bslot


# ---------------------------------------------------------------------------
# Measurement formulas (Know your platform §5)
# ---------------------------------------------------------------------------

def overlap_efficiency(t_comp: float, t_comm: float, t_total: float) -> float:
    """(T_comp + T_comm - T_total) / min(T_comp, T_comm); target >= 0.8."""
    return (t_comp + t_comm - t_total) / min(t_comp, t_comm)


def compute_interference(t_comp_fused: float, t_comp_alone: float) -> float:
    """T_comp measured inside the fused run over T_comp alone; target <= 1.1."""
    return t_comp_fused / t_comp_alone
