/*
 * fg.h -- C ABI of the fused producer/consumer gather-GEMM for AMD MI355X (gfx950).
 *
 * One persistent HIP kernel: communication workgroups move rows from N source
 * shards (separate HBM regions standing in for peer ranks) into a gathered
 * buffer, optionally scattered by a routing index, and signal completion;
 * compute workgroups spin-gate on the signals and run the bf16 contraction with
 * fp32 accumulation.
 *
 * Pages this interface follows (titles abbreviated):
 *   "PCIe sync protocols" -- compute-comm fused operators (4): cross-card sync
 *       protocols over PCIe: single writer, election, watermark.
 *       §1 the problem (how A tells B its data is written), §2 slot + monotonic
 *       seq and the all-rank barrier, §3 local election + single-writer
 *       publish, §4 64-row chunk watermark, §5 seeded 128-row arrival counters
 *       gating the GEMM, §6 residency/deadlock audit, §7 isolated debug entries
 *       and host-recomputed expectation tables.
 *   "NVLink atomic publish" -- §3.1 control plane separate from data and
 *       aligned, §5.2 one publish wrapper, §7 a hidden observation counter and
 *       packaging as a small primitive library.
 *   "Know your platform" -- §5 the three timings and overlap efficiency.
 *   "DeepEP FIFO pipeline" -- dispatch "notify" stage (per-expert counts fix
 *       offsets), bounded spins with timeouts.
 *
 * Conventions for every entry point:
 *   - Pointers documented "device" are HIP device pointers owned by the caller
 *     unless stated otherwise; "host" pointers are ordinary host memory.
 *   - bf16 data are 16-bit bit patterns (uint16), rows contiguous (row-major).
 *   - Every call returns an fg_status; nothing is thrown and nothing aborts.
 *   - Launches are asynchronous on the given stream. A device-side failure
 *     (a wait that timed out, a counter that overshot) is recorded in the
 *     context and reported by the next call on it; the context then answers
 *     FG_ESTATE to everything but fg_stats and fg_destroy.
 *   - A context is bound to the first stream it is used with; work on a
 *     different stream returns FG_EINVAL (the parity re-arming of the control
 *     plane relies on stream order between consecutive calls).
 *   - The gather-GEMM and combine kernels are persistent grids sized to be
 *     resident all at once, whose workgroups wait for one another ("PCIe sync
 *     protocols" §6 audit). Two such kernels must not run at the same time on
 *     one GPU: contexts used on different streams, or other long kernels
 *     running concurrently, can keep part of a grid from starting. The waits
 *     then end at the context's watchdog (timeout_ns) with FG_ETIMEOUT rather
 *     than hanging. Contexts that share one stream run one after another and
 *     are safe.
 */
#ifndef FG_H
#define FG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FG_CHUNK_ROWS 64    /* "PCIe sync protocols" §4: one signal per 64 rows of a producer stream */
#define FG_ROW_BLOCK 128    /* "PCIe sync protocols" §5: the GEMM gate releases 128 gathered rows */
#define FG_COUNTER_STRIDE 64  /* int32 per arrival counter: each counter has a 256-byte line of its own */
#define FG_MAX_SHARDS 64
#define FG_MAX_GROUPS 64

typedef enum {
  FG_OK = 0,
  FG_EINVAL = -1,      /* bad argument, shape or stream */
  FG_ENOMEM = -2,      /* device or pinned allocation failed (fg_init only) */
  FG_EHIP = -3,        /* a HIP runtime call failed */
  FG_ERESIDENCY = -4,  /* the persistent grid would not be co-resident (deadlock risk) */
  FG_ETIMEOUT = -5,    /* a device-side wait hit its watchdog */
  FG_EPROTOCOL = -6,   /* a counter overshot its target / duplicate route row */
  FG_ESTATE = -7       /* context carries an earlier device-side error */
} fg_status;

/* Per-call flags of fg_gather_gemm. */
enum {
  FG_CALL_COMM_ONLY = 1u << 0,  /* communication role only (T_comm alone) */
  FG_CALL_GEMM_ONLY = 1u << 1,  /* compute role only, gates pre-opened, gathered pre-filled (T_comp alone) */
  FG_CALL_VERIFY = 1u << 2,     /* count publishes per slot, polls and waits (observation counters) */
  FG_CALL_STRICT = 1u << 3,     /* formal agent-scope release fences on every signal (slow reference mode) */
  FG_CALL_SAME_ROUTE = 1u << 4, /* EXPLICIT/TOPK: route identical to the previous call, skip the layout step */
  FG_CALL_TRACE = 1u << 5,      /* record per compute item and per row block timestamps (fg_views trace) */
  FG_CALL_LAYOUT_TWO_PASS = 1u << 6, /* TOPK: run the layout as two kernels (count + scan, then place) even
                                        when its grid fits on the device at once (the one-kernel layout waits
                                        for the scan inside the kernel) */
  FG_CALL_GATE_WATERMARK = 1u << 7,  /* CONTIG routes of fg_gather_gemm only ("PCIe sync protocols" §4): the
                                        compute role gates each tile on the slots (chunk watermarks) of the
                                        64-row chunks its rows come from instead of the 128-row counters
                                        (which are still counted, so the control plane is the same) */
  /* Fault injection (tests). Each makes a bounded wait or a check fail so that
   * the error path is exercised; every kernel still runs to completion. */
  FG_FAULT_SEED_LOW = 1u << 8,      /* seed of row block 0 one too low: its gate never opens -> FG_ETIMEOUT */
  FG_FAULT_SEED_HIGH = 1u << 9,     /* seed of row block 0 one too high: counter overshoots -> FG_EPROTOCOL */
  FG_FAULT_DROP_PUBLISH = 1u << 10  /* elected publisher of chunk (0,0) skips its slot store */
};

typedef struct {
  int32_t n_shards;            /* source shards = virtual ranks, 1..FG_MAX_SHARDS */
  int32_t max_rows_per_shard;  /* capacity of one shard's stream (rows) */
  int32_t K;                   /* row width in bf16 elements; multiple of 128 */
  int32_t N;                   /* GEMM output width; multiple of 128 */
  int32_t n_groups;            /* 1 = one dense weight; >1 = one weight per group (expert) */
  int32_t n_comm_wg;           /* communication workgroups (0 = three quarters of the compute units, 192 on
                                  MI355X); they join the compute role
                                  once their rows are copied */
  int32_t n_gemm_wg;           /* dedicated compute workgroups (0 = CUs - n_comm_wg) */
  int32_t tile_n;              /* GEMM tile width 128 or 256 (0 = default) */
  int64_t timeout_ns;          /* watchdog of every device-side wait (0 = 2 s) */
  int32_t stress_producers;    /* protocol-stress plane (0 = none): producers x consumers x chunks slots */
  int32_t stress_consumers;
  int32_t stress_max_chunks;
  int32_t split_parts;         /* split-K tail: at most this many k-ranges per split tile, 1..8 (0 = 8,
                                  1 = no split). By default every tile list keeps a whole number of rounds
                                  of whole tiles and its leftover tiles are split into
                                  P = min(split_parts, K / 128, grid / leftover tiles) ranges */
  int32_t split_tiles;         /* 0 = the default above; > 0: split this many tiles (taken evenly from the
                                  end of the tile lists) into split_parts ranges, even when the tiles fill
                                  whole rounds. Partial workspace: max(grid, split_tiles * split_parts) blocks
                                  of 256 * tile_n fp32, allocated by fg_init */
  int32_t tile_order;          /* 0 = tiles grouped per XCD when the grid is a multiple of 8 (default);
                                  1 = one row-block-major list */
  int32_t copy_rows;           /* rows per copy batch of one wave: 1, 2, 4, 8 or 16, capped so that at most
                                  32 16-byte vectors per lane are in flight (0 = the cap) */
  int32_t combine_wg;          /* workgroups of the combine kernel (0 = 2 per compute unit); the grid must
                                  be co-resident (checked by fg_init: FG_ERESIDENCY) */
  int32_t copy_mode;           /* who moves the rows of fg_gather_gemm ("PCIe sync protocols" §3-§5):
                                  0 = copy workgroups (default): n_comm_wg workgroups copy every row first
                                      and then join the compute role;
                                  1 = in tiles where the shape allows: every workgroup copies the lead rows
                                      that the first round of tiles reads, then each tile copies rows of a
                                      later round's slabs inside its K loop, in the shadow of its MFMAs,
                                      and counts and publishes them (one-group CONTIG or EXPLICIT routes,
                                      K a multiple of 512 and >= 1536, per-XCD tile lists, no forced split,
                                      no watermark gating); otherwise as 0 */
} fg_config;

typedef enum {
  FG_ROUTE_CONTIG = 0,   /* all-gather: shard s row i -> gathered row s*rows_per_shard + i */
  FG_ROUTE_EXPLICIT = 1, /* caller-given stream (src_row, dst_row) per shard */
  FG_ROUTE_TOPK = 2      /* expert dispatch: layout computed on the device from top-k choices */
} fg_route_mode;

typedef struct {
  int32_t mode;               /* fg_route_mode */
  int32_t rows_per_shard;     /* CONTIG: rows of every shard; TOPK: tokens of every shard */
  /* EXPLICIT */
  const int32_t* stream_len;  /* host  [n_shards] stream length of each shard */
  const int32_t* src_row;     /* device [n_shards][max_rows_per_shard]: source row of stream entry i */
  const int32_t* dst_row;     /* device [n_shards][max_rows_per_shard]: gathered row of stream entry i */
  int32_t m_pad;              /* gathered rows, a multiple of FG_ROW_BLOCK */
  const int32_t* group_off;   /* host [n_groups+1] first gathered row of each group (NULL: one group) */
  /* TOPK */
  const int32_t* topk;        /* device [n_shards][rows_per_shard][topk_k] chosen experts, distinct per token;
                                 rows_per_shard <= max_rows_per_shard */
  int32_t topk_k;
  int32_t expert_base;        /* this GPU owns experts [expert_base, expert_base + n_groups) */
} fg_route;

typedef struct fg_ctx fg_ctx;

/* Observation counters of the library ("NVLink atomic publish" §7: a hidden
 * observation counter beside the protocol, read by the host, and the package
 * as a small primitive library; "PCIe sync protocols" §7: the host compares
 * what the device did with a table it recomputes, here expected_publishes
 * against publishes). Cumulative fields count from fg_init; "last" fields
 * describe the last fused kernel. */
typedef struct {
  int32_t seq, bseq, stress_seq;  /* last sequence numbers issued (monotonic, never reset) */
  int32_t m_pad;                  /* gathered rows of the last gather-GEMM (device-computed for TOPK) */
  int32_t error_code, error_id;   /* first device-side error and the wait/slot it concerns */
  int64_t publishes;              /* VERIFY: slot stores by elected publishers, cumulative */
  int64_t gate_polls, slot_polls; /* VERIFY: relaxed polls issued by waiters, cumulative */
  int64_t gate_passes;            /* VERIFY: gates passed by compute workgroups, cumulative */
  int64_t stale;                  /* stress: rows read with a value other than the expected one */
  double t_kernel_us;             /* last fused kernel: first start to last end (device clock) */
  double t_comm_span_us;          /* last fused kernel: communication role span */
  double t_gemm_span_us;          /* last fused kernel: compute role span */
  double t_gemm_busy_us;          /* compute-role time net of waits (gates, split-K part waits), summed
                                     over workgroups, per whole-tile equivalent (a part counts 1/P) */
  double t_gate_wait_us;          /* mean over workgroups that ran compute items of their wait time */
  double t_barrier_us;            /* last fg_barrier: device time per barrier */
  double t_rtt_us;                /* last fg_pingpong: device round trip */
  int32_t n_comm_wg, n_gemm_wg, cu_count, m_pad_cap;
  int32_t tiles_whole, tiles_split; /* last fused kernel: whole tiles, tiles computed as split-K parts */
  int32_t split_parts;            /* k-ranges per split tile (1 when none is split) */
  int32_t combine_seq;            /* last combine sequence number issued (monotonic, never reset) */
  double clock_mhz;               /* last fused kernel: shader-clock cycles / wall time, over all workgroups */
  int64_t litmus_stale;           /* fg_litmus: words read with a value other than the round's, cumulative */
  int64_t litmus_words;           /* fg_litmus: words checked, cumulative */
  int64_t expected_publishes;     /* VERIFY: publishes the calls should have made, one per active 64-row chunk of
                                     every stream they publish (device-computed from the route in use), cumulative;
                                     equal to publishes when every chunk had exactly one publisher */
  int64_t timeouts;               /* device-side waits that hit their watchdog, cumulative (any entry point) */
  int64_t max_wait_ns;            /* last fused kernel: longest single wait of a compute workgroup (a gate, or a
                                     split-K part waiting for its siblings) */
  int32_t first_timeout_id;       /* id of the first wait that timed out (-1: none); error_id names the first
                                     error of any kind */
  int32_t copy_in_tiles;          /* last fused kernel: 1 if its rows were copied in tiles (copy_mode 1) */
  int32_t lead_rows;              /* last fused kernel: rows every workgroup copied first (in-tile copy) */
  int32_t reserved4;
} fg_stats_t;

/* Read-only device views of the library-owned control plane (for tests that
 * compare it element by element with the host-recomputed table). */
typedef struct {
  const int32_t* slot;        /* [n_shards][chunk_cap] */
  const int32_t* counter;     /* [2][rb_cap][FG_COUNTER_STRIDE] parity double-buffered; value at [..][..][0] */
  const int32_t* elect;       /* [2][n_shards][chunk_cap] */
  const int32_t* pub_count;   /* [n_shards][chunk_cap] (VERIFY) */
  const int32_t* seed;        /* [rb_cap] */
  const uint64_t* inv_row;    /* [m_pad_cap] versioned inverse map: (route_ver << 32) | (shard << 24 | stream
                                 index); an entry with another version is a padding row */
  const int32_t* group_of_rb; /* [rb_cap] */
  const int32_t* src_row;     /* [n_shards][max_rows_per_shard] route in use */
  const int32_t* dst_row;     /* [n_shards][max_rows_per_shard] */
  const int32_t* stream_len;  /* [n_shards] */
  const int32_t* group_off;   /* [n_groups + 1] */
  const int32_t* bslot;       /* [n_shards][n_shards] barrier slots */
  const int32_t* stress_slot; /* [P][C][KC] */
  const int32_t* stress_pub;  /* [P][C][KC] */
  int32_t chunk_cap, rb_cap, m_pad_cap;
  uint32_t route_ver;         /* version of the route in use */
  /* Timing observation (device wall clock, wall_khz ticks per ms), written by
   * the last fused kernel: */
  const int64_t* wg_time;     /* [grid][12]: start, end, wait ticks, whole tiles, end of the copy role,
                                 split parts, start of the compute role, parts per split tile, shader-clock
                                 counter at start and at end, 2 unused */
  const int64_t* trace;       /* FG_CALL_TRACE: [trace_cap][8] per compute item (whole tile t at row t,
                                 split-K part q at row n_tiles + q): workgroup, ticket taken, gate open, item
                                 done; parts also: k loop done, partial stored, all parts counted; 1 unused */
  const int64_t* rb_time;     /* FG_CALL_TRACE: [rb_cap] issue time of the add that brought the row block's
                                 counter to 128 (its publish) */
  int32_t grid, trace_cap;
  int64_t wall_khz;
  const int32_t* desc;        /* [3]: gathered rows m_pad, row slabs n_slabs and groups of the route in use */
  const int32_t* slab;        /* [n_slabs] compute row slabs: first row | 1 for a 128-row slab (else 256 rows);
                                 every group is cut into 256-row slabs plus one 128-row slab if its size is an
                                 odd number of 128-row blocks */
  const int32_t* group_slab;  /* [groups + 1] first slab of each group (the last entry is n_slabs) */
  /* Combine plane (fg_combine) and the per-entry tables of the TOPK route: */
  const int32_t* combine_slot;  /* [n_shards][chunk_cap][FG_COUNTER_STRIDE], value at [..][..][0] */
  const int32_t* combine_elect; /* [2][n_shards][chunk_cap][FG_COUNTER_STRIDE] parity double-buffered */
  const int32_t* combine_pub;   /* [n_shards][chunk_cap] (VERIFY) */
  const int32_t* src_k;         /* [n_shards][max_rows_per_shard] top-k position of each stream entry */
  const int32_t* tok_first;     /* [n_shards][max_rows_per_shard + 1] first stream entry of each token;
                                   entry [tokens] = the stream length */
  /* FIFO rings (fg_gather_gemm_ring), parity double-buffered: */
  const uint64_t* ring_tail;    /* [2][ring_cap][32], value at [..][r][0] = finish << 32 | tail */
  const int32_t* ring_head;     /* [2][ring_cap][FG_COUNTER_STRIDE], value at [..][r][0] */
  int32_t ring_cap, reserved2;  /* ring_cap: rings the copy workgroups can serve (n_comm_wg / 2) */
  const int32_t* src_of;        /* [m_pad_cap] source row of each gathered row of the route in use (valid where
                                   the inverse map has a current entry) */
} fg_views_t;

/* Create a context on `hip_device`: validates the configuration, allocates and
 * zeroes the control plane (slots, counters x2, election counts x2, publisher
 * counts, route tables, barrier slots, host-visible status word) and checks
 * that the persistent grid is co-resident and that fewer workgroups spin than
 * there are compute units ("PCIe sync protocols" §6 audit items 1 and 2).
 * Returns FG_EINVAL, FG_ENOMEM, FG_EHIP or FG_ERESIDENCY on failure (*out = NULL). */
fg_status fg_init(const fg_config* cfg, int hip_device, fg_ctx** out);

/* One iteration of the hot path ("PCIe sync protocols" §3-§5): seq = ++seq;
 * layout step (TOPK/EXPLICIT, unless FG_CALL_SAME_ROUTE); then one persistent
 * kernel in which communication workgroups copy every stream row
 * shards[s][src_row] -> gathered[dst_row] bitwise (device-coherent 16-byte
 * stores), add arrivals to the 128-row counters (seeded with the padding
 * count), elect the last writer of each 64-row chunk, which stores seq into the
 * chunk's single-writer slot; compute workgroups (and communication
 * workgroups once their rows are copied) take tiles from a ticket counter,
 * wait for each 128-row block's counter to equal 128 and compute
 * out[m][n] = sum_k gathered[m][k] * W_g(m)[k][n] (fp32 accumulation, bf16
 * round-to-nearest-even output; padding rows = 0). The last tiles are split
 * into k-ranges whose fp32 partials are summed in a fixed order, so results
 * are deterministic.
 *   shards:   host array of n_shards device pointers, bf16 [rows, K]
 *   route:    NULL = CONTIG with rows_per_shard = max_rows_per_shard
 *   W:        device bf16 [n_groups][N][K]: W_g[k][n] stored at W[g][n][k]
 *   gathered: device bf16 [m_pad_cap][K] (written; padding rows never written)
 *   out:      device bf16 [m_pad_cap][N]
 *   flags:    FG_CALL_* / FG_FAULT_*
 * Every device row buffer (shards, W, gathered, out, and the staging and ring
 * buffers of the variants below) starts on a 16-byte boundary: rows move in
 * 16-byte vectors.
 * Errors: FG_EINVAL (shapes, NULLs, misaligned buffers, stream; the context is
 * unchanged), FG_ESTATE, FG_ETIMEOUT / FG_EPROTOCOL from an earlier call,
 * FG_EHIP. */
fg_status fg_gather_gemm(fg_ctx* ctx, const void* const* shards, const fg_route* route,
                         const void* W, void* gathered, void* out, uint32_t flags,
                         hipStream_t stream);

/* The same iteration as fg_gather_gemm with the dispatch in two stages
 * ("PCIe sync protocols" §4 chunk watermark; §6 audit item 2: the receiver's
 * scatter waits only on remote watermarks and reads its own shard directly).
 * Stage 1, push: every stream entry i of every shard s other than self_shard
 * is copied shards[s][src_row[s][i]] -> staging[s][i] bitwise (write-through
 * stores); the wave that completes a 64-entry chunk, elected by a local count,
 * stores seq into the chunk's slot (the watermark). Stage 2, scatter: gathered
 * rows, in gathered-row order, are copied from staging (remote shards, after
 * their chunk's slot carries seq) or from the shard (self_shard, no wait) and
 * counted into the seeded 128-row counters; the compute role gates on those
 * counters as in fg_gather_gemm. The slots, election counts and publisher
 * counts of self_shard are not touched.
 *   staging:    host array of n_shards device pointers, bf16 [max_rows_per_shard][K]
 *               (written; the entry of self_shard may be NULL)
 *   self_shard: -1 (every shard is remote) or 0..n_shards-1
 * Other arguments, flags and errors as fg_gather_gemm. */
fg_status fg_gather_gemm_staged(fg_ctx* ctx, const void* const* shards, const fg_route* route,
                                const void* W, void* const* staging, int32_t self_shard, void* gathered,
                                void* out, uint32_t flags, hipStream_t stream);

/* The same iteration as fg_gather_gemm_staged with bounded staging memory: a
 * streaming FIFO ring per (shard, channel) ("DeepEP FIFO pipeline": head/tail
 * credits, slot = index mod capacity, a finish flag packed beside the tail).
 * Shard s's stream of 64-row chunks is dealt to n_channels rings, chunk c to
 * ring c mod n_channels. Copy workgroup r produces ring r: it writes the ring's
 * j-th chunk shards[s][src_row] rows into slot j mod ring_chunks once the
 * consumer's head shows chunk j - ring_chunks drained, then stores the tail
 * (j + 1, with the finish bit on the last chunk). Copy workgroup rings + r
 * consumes it: it waits for the tail, scatters the chunk into the gathered
 * buffer, counts the rows into the seeded 128-row counters and advances the
 * head. Rings of self_shard have no producer; their consumer reads the shard.
 * The compute role gates on the counters as in fg_gather_gemm.
 *   ring:        device bf16 [n_shards][n_channels][ring_chunks][64][K]
 *                (fg_ring_bytes gives its size)
 *   n_channels:  rings per shard, n_shards * n_channels <= n_comm_wg / 2
 *   ring_chunks: 64-row slots per ring, >= 1
 *   self_shard:  -1 (every shard is remote) or 0..n_shards-1
 * Other arguments, flags and errors as fg_gather_gemm; FG_EINVAL when the
 * rings need more copy workgroups than the context has. */
fg_status fg_gather_gemm_ring(fg_ctx* ctx, const void* const* shards, const fg_route* route, const void* W,
                              void* ring, int32_t n_channels, int32_t ring_chunks, int32_t self_shard,
                              void* gathered, void* out, uint32_t flags, hipStream_t stream);

/* Bytes of the ring buffer fg_gather_gemm_ring needs for this configuration. */
fg_status fg_ring_bytes(const fg_config* cfg, int32_t n_channels, int32_t ring_chunks, int64_t* bytes);

/* `rounds` consecutive all-rank barriers over n_shards virtual ranks in one
 * kernel ("PCIe sync protocols" §2): rank i's lane j stores bseq into
 * bslot[j][i] (its own slot on every rank), then waits until
 * bslot[i][0..n) >= bseq. bseq advances by `rounds` (1..1e6). */
fg_status fg_barrier(fg_ctx* ctx, int32_t rounds, hipStream_t stream);

/* Slot ping-pong between two workgroups on different XCDs, `round_trips`
 * round trips in one kernel; the mean round trip lands in fg_stats.t_rtt_us.
 * sys_scope != 0 uses system-scope slot stores and polls. */
fg_status fg_pingpong(fg_ctx* ctx, int32_t round_trips, int32_t sys_scope, hipStream_t stream);

/* One iteration of the protocol-stress workload ("PCIe sync protocols" §3-§4
 * at the scale of §3's validation): producer workgroup p, after waiting
 * delays_ns[p][c][k], writes chunk_rows[p][c][k] 4-byte rows of payload
 * ((seq << 20) ^ (((p*C + c)*KC + k)*64 + r)) into payload[c][p][k][r]; its waves
 * elect one publisher per chunk, which stores seq into slot (p,c,k); consumer
 * workgroup c waits for every active slot addressed to it and checks every
 * row, counting mismatches in fg_stats.stale.
 *   chunk_rows: device int32 [P][C][KC] (0 = inactive, else 1..64)
 *   delays_ns:  device int32 [P][C][KC]
 *   payload:    device int32 [C][P][KC][64]
 *   flags:      FG_CALL_STRICT / FG_FAULT_DROP_PUBLISH */
fg_status fg_stress(fg_ctx* ctx, const int32_t* chunk_rows, const int32_t* delays_ns,
                    int32_t* payload, uint32_t flags, hipStream_t stream);

/* Combine, the reverse of the expert dispatch ("PCIe sync protocols" §3 the
 * pushed rows, the local count and the last writer's slot store; §4 one slot
 * per 64 entries of a stream). Runs on the TOPK route of the last
 * fg_gather_gemm call (FG_EINVAL for any other route). cseq = ++cseq; one
 * kernel whose workgroups first push every stream entry i of every shard s,
 * staging[s][i] = out[dst_row[s][i]] bitwise (device-coherent 16-byte stores),
 * and count the rows of each 64-entry chunk; the add that completes a chunk
 * elects its single publisher, which stores cseq into the chunk's combine
 * slot. Then, per token t of shard s, after the slots of the chunks holding
 * its entries carry cseq:
 *   y[s][t][n] = bf16_rne( sum over the token's local picks k, in k order, of
 *                          weights[s][t][k] * staging[s][i(t,k)][n] )
 * in fp32; a token with no local pick gets a zero row. Only this GPU's experts
 * are summed.
 *   out:     device bf16 [m_pad][N] expert outputs in gathered-row order (as
 *            written by fg_gather_gemm)
 *   weights: device fp32 [n_shards][tokens][topk_k] gate weights
 *   staging: host array of n_shards device pointers, bf16 [max_rows_per_shard][N]
 *            (each shard's receive buffer, indexed by stream entry; written)
 *   y:       host array of n_shards device pointers, bf16 [tokens][N] (written)
 *   flags:   FG_CALL_COMM_ONLY (push only), FG_CALL_GEMM_ONLY (weighted sums
 *            only, from a staging buffer an earlier call filled; no slot
 *            waits), FG_CALL_VERIFY (publisher counts, polls), FG_CALL_STRICT,
 *            FG_FAULT_DROP_PUBLISH (publisher of chunk (0,0) skips its slot
 *            store: the waits on it time out -> FG_ETIMEOUT)
 * out, staging and y start on 16-byte boundaries, weights on a 4-byte one.
 * Errors: FG_EINVAL (route, NULLs, misaligned buffers, stream), FG_ESTATE,
 * FG_ETIMEOUT / FG_EPROTOCOL from an earlier call, FG_EHIP. */
fg_status fg_combine(fg_ctx* ctx, const void* out, const float* weights, void* const* staging,
                     void* const* y, uint32_t flags, hipStream_t stream);

/* Message-passing litmus test of how signalled data is read (an isolated
 * debug entry, "PCIe sync protocols" §7, for the data-then-signal chain of
 * §3): `rounds` rounds (1..1e6) in one kernel of two workgroups on different
 * XCDs. Each round the writer stores a 16 KB block with device-scope
 * write-through stores, waits for their acknowledgement and stores the round
 * number into a flag; the reader, whose caches hold the block's previous
 * contents, polls the flag and reads the block again:
 *   mode 0: device-scope loads, as the library reads signalled data;
 *   mode 1: plain loads (expected to see stale words: shows the test's reach);
 *   mode 2: plain loads after the formal agent-scope acquire fence.
 * Words that differ from the round number accumulate in
 * fg_stats.litmus_stale (out of fg_stats.litmus_words). Every wait has the
 * context's watchdog. */
fg_status fg_litmus(fg_ctx* ctx, int32_t rounds, int32_t mode, hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * iteration as fg_gather_gemm with no context: the call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the control plane
 * lives in a file-scope device array of the library, 4 MiB per GPU, held until
 * the process ends (8 shards x 4096 rows at K = N = 8192 fit; a configuration
 * whose control plane does not fit returns FG_EINVAL). The split-K tail is not
 * used (leftover tiles run whole) and nothing is traced.
 *   cfg, hip_device: configuration and device of this call; shapes may change
 *                    from call to call
 *   shards, route, W, gathered, out: as fg_gather_gemm (CONTIG, EXPLICIT or
 *                    TOPK routes)
 *   status:          device int32, set to 0 at the start of the call; a device-side
 *                    error (a wait that timed out, a counter that overshot) stores
 *                    its fg_status code there; read it after the stream's work ends
 *   flags:           0, FG_CALL_STRICT or FG_CALL_GATE_WATERMARK (others: FG_EINVAL)
 * Every call on one GPU uses that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller. The slots keep their monotonic
 * sequence numbers across calls; everything else is cleared by the call.
 * Errors: FG_EINVAL (shapes, NULLs, flags, control plane too large), FG_EHIP,
 * FG_ERESIDENCY. */
fg_status fg_gather_gemm_noalloc(const fg_config* cfg, int hip_device, const void* const* shards,
                                 const fg_route* route, const void* W, void* gathered, void* out, int32_t* status,
                                 uint32_t flags, hipStream_t stream);

/* Copy the observation counters to *out ("NVLink atomic publish" §7: the
 * observation counter and the small library around the protocol; fields as
 * documented in fg_stats_t). wait != 0 first synchronises the bound stream,
 * which the device-computed fields and timings need; wait == 0 returns only
 * the host-side sequence numbers and sizes. Callable on a context in the
 * error state. Errors: FG_EINVAL (NULL), FG_EHIP, FG_ENOMEM. */
fg_status fg_stats(fg_ctx* ctx, fg_stats_t* out, int wait);

/* Read-only device pointers of the control plane, valid until fg_destroy
 * ("PCIe sync protocols" §7: the host recomputes the expected table and
 * compares it with the device state element by element; "NVLink atomic
 * publish" §3.1: the control plane lives apart from the data). The caller
 * must not write through them. Errors: FG_EINVAL (NULL). */
fg_status fg_views(fg_ctx* ctx, fg_views_t* out);

/* Minimum number of gathered / output rows the caller must allocate for a
 * configuration: the real rows plus the padding of every group to a multiple
 * of FG_ROW_BLOCK ("PCIe sync protocols" §5: padding rows are pre-counted by
 * the seed, so the gathered buffer holds whole 128-row blocks). Errors:
 * FG_EINVAL (invalid configuration or NULL). */
fg_status fg_capacity(const fg_config* cfg, int32_t* m_pad_cap);

/* Synchronise the bound stream and free the context's control plane, split-K
 * workspace and status word; the caller's buffers are not touched. The
 * counterpart of fg_init ("NVLink atomic publish" §7: the protocol packaged
 * as a small library that owns only its control plane). Errors: FG_EINVAL
 * (NULL). */
fg_status fg_destroy(fg_ctx* ctx);

/* Static text of a status code (never NULL; "unknown" for other values).
 * The codes are the error conventions of every entry point: a device-side
 * wait that hit its watchdog ("DeepEP FIFO pipeline": every spin bounded by a
 * timeout), a counter past its target ("PCIe sync protocols" §5: the gate
 * compares for equality with the row block), or a context left in the error
 * state. */
const char* fg_strerror(fg_status s);

#ifdef __cplusplus
}
#endif

#endif /* FG_H */
