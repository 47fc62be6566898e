// Kernels of the fused producer/consumer gather-GEMM and of its protocol
// entry points (layout, fused persistent kernel, slot barrier, ping-pong,
// protocol stress). Included once, by fg.hip.
#pragma once

#include "fg_gemm.hpp"
#include "fg_plan.hpp"
#include "fg.h"

namespace fg {

constexpr int kChunk = FG_CHUNK_ROWS;
constexpr int kRB = FG_ROW_BLOCK;
constexpr int kCtr = FG_COUNTER_STRIDE;  // arrival counters sit 256 bytes apart: a gate's pollers and
                                         // the copy role's adds then spread over memory channels
constexpr int kThreads = 64 * kWaves;   // workgroup size of the fused kernel
constexpr int kXcds = 8;                // XCDs of the part; workgroup i runs on XCD i % 8
constexpr int kTickInts = 1024;         // ticket block per parity: global ticket + one per XCD, 256 B apart
constexpr int kTraceFields = 8;

// per-call flag bits as seen by the device
constexpr uint32_t kCommOnly = FG_CALL_COMM_ONLY;
constexpr uint32_t kGemmOnly = FG_CALL_GEMM_ONLY;
constexpr uint32_t kVerify = FG_CALL_VERIFY;
constexpr uint32_t kStrict = FG_CALL_STRICT;
constexpr uint32_t kDropPublish = FG_FAULT_DROP_PUBLISH;
constexpr uint32_t kTrace = FG_CALL_TRACE;
constexpr uint32_t kGateWatermark = FG_CALL_GATE_WATERMARK;

// Device statistics block (int64 counters, cumulative).
// ST_EXPECTED: the publishes a VERIFY call should make (one per active chunk of
// the streams it copies), added by the call itself so that the host can
// compare it with ST_PUBLISHES whatever route the device computed.
enum { ST_PUBLISHES = 0, ST_GATE_POLLS, ST_SLOT_POLLS, ST_GATE_PASSES, ST_STALE, ST_EXPECTED, ST_COUNT };

// Versioned inverse map: entry = (route version << 32) | (shard << 24 | stream index).
__device__ __forceinline__ unsigned long long inv_pack(uint32_t ver, int v) {
  return ((unsigned long long)ver << 32) | (uint32_t)v;
}
__device__ __forceinline__ int inv_read(const unsigned long long* inv, int g, uint32_t ver) {
  const unsigned long long e = inv[g];
  return (uint32_t)(e >> 32) == ver ? (int)(uint32_t)e : -1;
}

struct FusedArgs {
  const uint16_t* shards[FG_MAX_SHARDS];
  const uint16_t* W;
  uint16_t* gathered;
  uint16_t* out;
  int K, N, n_shards, chunk_cap, rs_cap, rb_cap, m_pad_cap;
  int shard_rows;            // rows of every source shard (bounds of the row loads)
  int* slot;
  int* counter_cur;          // [rb_cap][kCtr]
  int* counter_nxt;
  int* elect_cur;
  int* elect_nxt;
  int* pub_count;
  const int* seed;
  const unsigned long long* inv;   // versioned inverse map
  const int* src_of;         // [m_pad_cap] source row of each gathered row (with the inverse map)
  uint32_t route_ver;
  // in-tile copy: every workgroup copies the rows [0, lead_rows) first, the
  // compute items copy the other rows inside their K loops (fg_plan.hpp)
  int tcopy;
  int lead_rows;
  const int* group_of_rb;
  const int* src_row;
  const int* dst_row;        // [S][rs_cap] gathered row of each stream entry
  const int* stream_len;
  const int* desc;           // [0] = m_pad of this iteration, [1] = number of row slabs, [2] = groups
  const int* slab;           // [n_slabs] row slab: first row | 1 if the slab has 128 rows (else 256)
  const int* gslab;          // [groups + 1] first slab of each group
  unsigned long long* stats;
  long long* wgtime;         // [grid][kWgTimeFields], see WgTime
  ErrorSink err;
  int seq;
  int n_comm, n_gemm;
  int rows_per_batch;
  uint32_t flags;
  uint64_t timeout_ticks;
  // compute schedule: tickets and the split-K tail
  int* tick_cur;             // [kTickInts]: [0] next split-K part, [64 (1 + x)] next entry of list x
  int* tick_nxt;             // the other parity, zeroed here for the next call
  int tile_order;            // 0: XCD-grouped lists when the grid is a multiple of 8; 1: one list
  int* skc_cur;              // [split_slots] parts finished per split tile (zero at kernel start)
  int* skc_nxt;
  float* skws;               // partial blocks of 256 x BN floats, P consecutive blocks per split tile
  uint32_t skws_bytes;
  int split_tiles;           // given split tile count (split_forced), else 0
  int split_slots;           // capacity of the part counters
  int split_parts;           // into this many k-ranges (1 = no split)
  int split_forced;          // split a tail even when the tiles fill whole rounds (split_tiles given)
  long long* trace;          // TRACE: [trace_cap][kTraceFields] per item: workgroup, taken, gate open,
                             // done; parts also: k loop done, partial stored, all parts counted
  long long* rb_time;        // TRACE: [rb_cap] time a row block's counter reached 128
  int trace_cap;
  // two-stage dispatch: pushes into per-shard staging buffers, then a
  // watermark-gated scatter into the gathered buffer
  int two_stage;
  int self_shard;            // shard read directly by the scatter (-1 = none)
  uint16_t* staging[FG_MAX_SHARDS];   // [rs_cap][K] per shard, stream order
  // streaming FIFO ring: n_channels rings per shard of ring_chunks 64-row slots
  int ring_mode;
  int n_channels, ring_chunks, ring_cap;
  uint16_t* ring;            // [S][n_channels][ring_chunks][64][K]
  unsigned long long* rtail_cur;   // [ring_cap][kRingTailStride]: finish << 32 | tail
  unsigned long long* rtail_nxt;
  int* rhead_cur;            // [ring_cap][kCtr]
  int* rhead_nxt;
};

constexpr int kRingTailStride = 32;                    // u64 words per tail (one 256-byte line)
constexpr unsigned long long kRingFinish = 1ull << 32;

// Per-workgroup timing record (device clock ticks).
// WT_CLK0 / WT_CLK1: shader-clock counter (s_memtime) at start and end, for the
// effective clock = cycles / wall time.
// WT_MAXWAIT: the longest single wait of the compute role (a gate, or the wait
// of a split-K part for its siblings).
enum { WT_START = 0, WT_END, WT_GATE, WT_TILES, WT_COMM_END, WT_PARTS, WT_GEMM_START, WT_P, WT_CLK0, WT_CLK1,
       WT_MAXWAIT, kWgTimeFields = 12 };

// ---------------------------------------------------------------------------
// Communication role ("PCIe sync protocols" §3 election + publish, §4 chunk
// watermark, §5 arrival counters). Rows are walked in gathered-row order, the
// order in which the compute role consumes row blocks (§6 audit item 3); a
// communication workgroup never waits on anything (§6 audit item 2).
// ---------------------------------------------------------------------------
// Re-arm the other parity for the next iteration: nothing else touches it
// during this kernel, and stream order publishes it to the next one.
__device__ __forceinline__ void arm_next(const FusedArgs& a) {
  const int cw = blockIdx.x;
  for (int i = cw * kThreads + threadIdx.x; i < a.rb_cap; i += a.n_comm * kThreads)
    a.counter_nxt[(size_t)i * kCtr] = a.seed[i];
  for (int i = cw * kThreads + threadIdx.x; i < a.n_shards * a.chunk_cap; i += a.n_comm * kThreads)
    a.elect_nxt[i] = 0;
  for (int i = cw * kThreads + threadIdx.x; i < a.split_slots; i += a.n_comm * kThreads) a.skc_nxt[i] = 0;
  if (cw == 0 && threadIdx.x <= kXcds) a.tick_nxt[threadIdx.x * 64] = 0;
  for (int i = cw * kThreads + threadIdx.x; i < a.ring_cap; i += a.n_comm * kThreads) {
    a.rtail_nxt[(size_t)i * kRingTailStride] = 0;
    a.rhead_nxt[(size_t)i * kCtr] = 0;
  }
}

// Lane r < RB of a batch describes gathered row b * RB + r. Its inverse-map
// word is loaded a batch ahead of its use, by every lane and from an index
// kept in range, so that the load sits on no branch: a value that reaches a
// join on one path only makes the compiler wait for it there.
__device__ __forceinline__ unsigned long long batch_inv_word(const FusedArgs& a, int b, int RB, int n_batches,
                                                             int lane) {
  return a.inv[min(b, n_batches - 1) * RB + min(lane, RB - 1)];
}
// The word's inverse entry (-1: padding, a lane past the batch, or no batch).
__device__ __forceinline__ int batch_info(const FusedArgs& a, unsigned long long w, int b, int RB, int n_batches,
                                          int lane) {
  return lane < RB && b < n_batches && (uint32_t)(w >> 32) == a.route_ver ? (int)(uint32_t)w : -1;
}
// Source row of an inverse entry (any value for -1), loaded on no branch.
__device__ __forceinline__ int batch_srow(const FusedArgs& a, int info) {
  return a.src_row[info >= 0 ? (info >> 24) * a.rs_cap + (info & 0xFFFFFF) : 0];
}

// The batches b, b + nw, ... of RB gathered rows (each at most 64 * UPR
// 16-byte vectors, RB * UPR <= 32 vectors per lane in flight) of one wave,
// software-pipelined so that a batch costs two dependent memory round trips
// instead of six: the next batch's loads leave as soon as this batch's stores
// are acknowledged and its signals are issued, and the signals' return values
// (needed only for the election and the overshoot check) are examined once
// those loads are in flight; the inverse-map words of the batch after next
// are fetched alongside.
// Per batch: stores, release (every store acknowledged), one add to the row
// block's arrival counter, one add per chunk touched (from the first lane of
// the chunk, all chunks in one instruction), and the publish of each chunk
// whose add completed it. A padding row (or the part of a row beyond K) gets
// zero-sized descriptors, so its loads read 0 and its stores are dropped by the
// buffer unit; so do the register rows RB .. RM-1 when a batch is shorter than
// the register set (lanes >= RB describe no row).
// The atomics' results are left undefined on the lanes that do not issue them
// (and read only on the lanes that do), so no join copies them before the next
// batch's loads are out.
template <int UPR, bool strict>
__device__ __forceinline__ void comm_batches(const FusedArgs& a, const uint16_t* const* sh_shard, int RB, int b,
                                             int nw, int n_batches, uint32_t row_bytes, int lane) {
  constexpr int RM = 32 / UPR < 16 ? 32 / UPR : 16;   // rows of the register set
  v4i v[RM][UPR];
  auto load = [&](int binfo, int bsrow) {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const int rinfo = readlane(binfo, r);
      const bool valid = rinfo >= 0;
      const int s = valid ? (rinfo >> 24) : 0;
      const int sr = readlane(bsrow, r);
      const uint64_t base = (uint64_t)sh_shard[s];
      const uint16_t* shard =
          (const uint16_t*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base));
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(shard + (size_t)sr * a.K, valid ? row_bytes : 0u);
#pragma unroll
      for (int u = 0; u < UPR; ++u)
        v[r][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(u * 64 + lane) * 16, 0, 0);
    }
  };
  // lane s holds shard s's stream length (which fixes the size of its last
  // chunk), so that the election check reads it with a lane shuffle rather
  // than a dependent load
  const int slen = lane < a.n_shards ? a.stream_len[lane] : 0;
  int info = batch_info(a, batch_inv_word(a, b, RB, n_batches, lane), b, RB, n_batches, lane);
  load(info, batch_srow(a, info));
  int nb = b + nw;                                     // the batch to load next
  unsigned long long nword = batch_inv_word(a, nb, RB, n_batches, lane);
  while (true) {
    // the call flags, re-read each pass through an opaque copy: as loop
    // invariants they invite the compiler to clone the loop once per flag
    const uint32_t fl = opaque_u32(a.flags);
    const int ninfo = batch_info(a, nword, nb, RB, n_batches, lane);
    const int nsrow = batch_srow(a, ninfo);
    const int g0 = b * RB;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const bool valid = readlane(info, r) >= 0;
      const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(a.gathered + (size_t)(g0 + r) * a.K, valid ? row_bytes : 0u);
#pragma unroll
      for (int u = 0; u < UPR; ++u) store16_coherent(rd, (uint32_t)(u * 64 + lane) * 16, v[r][u]);
    }
    release_coherent(strict);
    // signals of batch b
    const int n_real = __popcll(ballot(lane < RB && info >= 0));
    int old_c, old_e, cnt = 0;
    // TRACE: the publish time of the block is the issue of the add that
    // completes it (its result, which says so, is examined a round trip later)
    const long long t_pub = (fl & kTrace) ? (long long)now_ticks() : 0;
    // (an opaque zero in the address keeps the compiler from rewriting this
    // one-lane add as a wave-wide one whose result it needs at once)
    if (lane == 0 && n_real > 0)
      old_c = fetch_add_relaxed(a.counter_cur + (size_t)(g0 / kRB) * kCtr + opaque_zero(), n_real);
    const int src_s = info >= 0 ? info >> 24 : 0, src_c = (info & 0xFFFFFF) / kChunk;
    const int chunk = (lane < RB && info >= 0) ? src_s * a.chunk_cap + src_c : -1;
    const int expect = min(kChunk, __shfl(slen, src_s) - kChunk * src_c);
    bool leader = false;
    uint64_t pending = ballot(chunk >= 0);
    while (pending) {
      const int l = __ffsll((long long)pending) - 1;
      const int ch = readlane(chunk, l);
      const uint64_t mask = ballot(chunk == ch) & pending;
      if (lane == l) { leader = true; cnt = __popcll(mask); }
      pending &= ~mask;
    }
    if (leader)
      old_e = strict ? fetch_add_acq_rel(a.elect_cur + chunk, cnt) : fetch_add_relaxed(a.elect_cur + chunk, cnt);
    // the next batch goes out before those values are examined
    const bool more = nb < n_batches;
    if (more) load(ninfo, nsrow);
    const unsigned long long nnword = batch_inv_word(a, nb + nw, RB, n_batches, lane);
    if (lane == 0 && n_real > 0) {
      const int blk = g0 / kRB;
      if (old_c + n_real > kRB) raise_error(a.err, kErrProtocol, blk);
      if ((fl & kTrace) && old_c + n_real == kRB) a.rb_time[blk] = t_pub;
    }
    if (leader) {
      if (old_e + cnt == expect) {
        if (!((fl & kDropPublish) && chunk == 0)) slot_publish(a.slot + chunk, a.seq, strict);
        if (fl & kVerify) {
          atomicAdd(a.pub_count + chunk, 1);
          atomicAdd(a.stats + ST_PUBLISHES, 1ull);
        }
      } else if (old_e + cnt > expect) {
        raise_error(a.err, kErrProtocol, 0x10000000 | chunk);
      }
    }
    if (!more) break;
    b = nb; info = ninfo; nb += nw; nword = nnword;
  }
}

template <int UPR>
__device__ __forceinline__ void comm_batches_any(bool strict, const FusedArgs& a, const uint16_t* const* sh_shard,
                                                 int RB, int b, int nw, int n_batches, uint32_t row_bytes, int lane) {
  if (strict) comm_batches<UPR, true>(a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
  else comm_batches<UPR, false>(a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
}

__device__ __forceinline__ void comm_role(const FusedArgs& a, const uint16_t* const* sh_shard) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = blockIdx.x;
  const bool strict = a.flags & kStrict;
  if (a.flags & kGemmOnly) return;

  const int m_pad = __builtin_amdgcn_readfirstlane(a.desc[0]);
  const int RB = a.rows_per_batch;
  // in-tile copy: the copy role takes only the lead rows, which the first
  // round of compute items reads; the items copy the rest
  const int m_copy = (a.tcopy && !(a.flags & kCommOnly)) ? min(m_pad, a.lead_rows) : m_pad;
  const int n_batches = m_copy / RB;
  const int upr = (a.K / 8 + 63) / 64;       // 64-lane units of 16 bytes per row
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const int nw = a.n_comm * kWaves;
  const int b = cw * kWaves + wave;
  if (b >= n_batches) return;
  // bitwise row copy: 16-byte loads (default cache policy: the non-temporal hint made the
  // copy 20 % slower), device-coherent 16-byte stores
  if (upr <= 1)       comm_batches_any<1>(strict, a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
  else if (upr <= 2)  comm_batches_any<2>(strict, a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
  else if (upr <= 4)  comm_batches_any<4>(strict, a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
  else if (upr <= 8)  comm_batches_any<8>(strict, a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
  else if (upr <= 16) comm_batches_any<16>(strict, a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
  else                comm_batches_any<32>(strict, a, sh_shard, RB, b, nw, n_batches, row_bytes, lane);
}

// ---------------------------------------------------------------------------
// Two-stage dispatch ("PCIe sync protocols" §4 chunk watermark, §6 audit item
// 2). Copy rows between per-row addresses: lane r < RB holds row r's source
// and destination address (valid = false: a zero-sized descriptor, so loads
// read 0 and stores are dropped).
// ---------------------------------------------------------------------------
template <int UPR, int RB>
__device__ __forceinline__ void copy_batch_addr(uint64_t src, uint64_t dst, bool valid, uint32_t row_bytes, int lane) {
  __amdgpu_buffer_rsrc_t rs[RB], rd[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const bool v = readlane((int)valid, r) != 0;
    const uint64_t sp = ((uint64_t)(uint32_t)readlane((int)(src >> 32), r) << 32) | (uint32_t)readlane((int)src, r);
    const uint64_t dp = ((uint64_t)(uint32_t)readlane((int)(dst >> 32), r) << 32) | (uint32_t)readlane((int)dst, r);
    rs[r] = buffer_rsrc((const void*)sp, v ? row_bytes : 0u);
    rd[r] = buffer_rsrc((const void*)dp, v ? row_bytes : 0u);
  }
  v4i v[RB][UPR];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int u = 0; u < UPR; ++u)
      v[r][u] = __builtin_amdgcn_raw_buffer_load_b128(rs[r], (uint32_t)(u * 64 + lane) * 16, 0, kPolSC1);
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int u = 0; u < UPR; ++u) store16_coherent(rd[r], (uint32_t)(u * 64 + lane) * 16, v[r][u]);
}

template <int UPR>
__device__ __forceinline__ void copy_rows_addr(int RB, uint64_t src, uint64_t dst, bool valid, uint32_t row_bytes,
                                               int lane) {
  if (RB == 1) copy_batch_addr<UPR, 1>(src, dst, valid, row_bytes, lane);
  else if (RB == 2) { if constexpr (UPR * 2 <= 32) copy_batch_addr<UPR, 2>(src, dst, valid, row_bytes, lane); }
  else if (RB == 4) { if constexpr (UPR * 4 <= 32) copy_batch_addr<UPR, 4>(src, dst, valid, row_bytes, lane); }
  else if (RB == 8) { if constexpr (UPR * 8 <= 32) copy_batch_addr<UPR, 8>(src, dst, valid, row_bytes, lane); }
  else { if constexpr (UPR * 16 <= 32) copy_batch_addr<UPR, 16>(src, dst, valid, row_bytes, lane); }
}

__device__ __forceinline__ void copy_addr(int upr, int RB, uint64_t src, uint64_t dst, bool valid,
                                          uint32_t row_bytes, int lane) {
  if (upr <= 1)       copy_rows_addr<1>(RB, src, dst, valid, row_bytes, lane);
  else if (upr <= 2)  copy_rows_addr<2>(RB, src, dst, valid, row_bytes, lane);
  else if (upr <= 4)  copy_rows_addr<4>(RB, src, dst, valid, row_bytes, lane);
  else if (upr <= 8)  copy_rows_addr<8>(RB, src, dst, valid, row_bytes, lane);
  else if (upr <= 16) copy_rows_addr<16>(RB, src, dst, valid, row_bytes, lane);
  else                copy_rows_addr<32>(RB, src, dst, valid, row_bytes, lane);
}

// Stage 1, push: every wave takes batches i, i + waves, ... of RB consecutive
// stream entries of one remote shard (RB divides 64, so a batch lies inside
// one chunk), copies shard_s[src_row] -> staging[s][entry] with write-through
// stores, releases, and adds its rows to the chunk's election count; the add
// that completes the chunk stores seq into the chunk's slot (the watermark).
// Stage 2, scatter: the batches of gathered rows in gathered-row order, as the
// one-stage copy walks them; a remote row is read from staging after its
// chunk's slot carries seq (one poll per distinct chunk of the batch), a row
// of the self shard straight from the shard; then the rows are counted into
// their 128-row block's counter. A wave scatters only after all its pushes,
// so every watermark wait has a supplier that never waits.
__device__ __forceinline__ void comm_two_stage(const FusedArgs& a, const uint16_t* const* sh_shard, uint16_t* const* sh_stage,
                               const int* sh_pbase) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool strict = a.flags & kStrict;
  const bool verify = a.flags & kVerify;
  const int RB = a.rows_per_batch;
  const int upr = (a.K / 8 + 63) / 64;
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const int nw = a.n_comm * kWaves, wid = blockIdx.x * kWaves + wave;
  const int n_push = sh_pbase[a.n_shards];
  for (int it = wid; it < n_push; it += nw) {
    int s = 0;
    while (s + 1 < a.n_shards && sh_pbase[s + 1] <= it) ++s;
    s = __builtin_amdgcn_readfirstlane(s);
    const int n_s = __builtin_amdgcn_readfirstlane(a.stream_len[s]);
    const int e0 = (it - sh_pbase[s]) * RB;
    const bool valid = lane < RB && e0 + lane < n_s;
    int srow = 0;
    if (valid) srow = min(max(a.src_row[s * a.rs_cap + e0 + lane], 0), a.shard_rows - 1);
    const uint64_t src = (uint64_t)(sh_shard[s] + (size_t)srow * a.K);
    const uint64_t dst = (uint64_t)(sh_stage[s] + (size_t)(e0 + lane) * a.K);
    copy_addr(upr, RB, src, dst, valid, row_bytes, lane);
    release_coherent(strict);
    const int n_done = __popcll(ballot(valid));
    if (lane == 0 && n_done > 0) {
      const int c = e0 / kChunk, ch = s * a.chunk_cap + c;
      const int old = strict ? fetch_add_acq_rel(a.elect_cur + ch, n_done) : fetch_add_relaxed(a.elect_cur + ch, n_done);
      const int expect = min(kChunk, n_s - kChunk * c);
      if (old + n_done == expect) {
        if (!((a.flags & kDropPublish) && ch == 0)) slot_publish(a.slot + ch, a.seq, strict);
        if (verify) {
          atomicAdd(a.pub_count + ch, 1);
          atomicAdd(a.stats + ST_PUBLISHES, 1ull);
        }
      } else if (old + n_done > expect) {
        raise_error(a.err, kErrProtocol, 0x10000000 | ch);
      }
    }
  }
  const int m_pad = __builtin_amdgcn_readfirstlane(a.desc[0]);
  const int n_batches = m_pad / RB;
  for (int b = wid; b < n_batches; b += nw) {
    const int g0 = b * RB;
    int info = -1, s = 0, i = 0;
    if (lane < RB) {
      info = inv_read(a.inv, g0 + lane, a.route_ver);
      if (info >= 0) { s = info >> 24; i = info & 0xFFFFFF; }
    }
    // watermark waits: one poll per distinct remote chunk of the batch
    const int chunk = (info >= 0 && s != a.self_shard) ? s * a.chunk_cap + i / kChunk : -1;
    uint64_t pending = ballot(chunk >= 0);
    int ok = 1;
    while (pending) {
      const int leader = __ffsll((long long)pending) - 1;
      const int ch = readlane(chunk, leader);
      if (lane == 0) {
        uint32_t polls = 0;
        ok = wait_ge(a.slot + ch, a.seq, now_ticks() + a.timeout_ticks, a.err, 0x30000000 | ch, &polls);
        if (verify) atomicAdd(a.stats + ST_SLOT_POLLS, (unsigned long long)polls);
      }
      if (!readlane(ok, 0)) break;
      pending &= ~ballot(chunk == ch);
    }
    if (!readlane(ok, 0)) break;
    if (strict) acquire_agent();
    uint64_t src = 0;
    if (info >= 0) {
      if (s == a.self_shard) {
        const int srow = min(max(a.src_row[s * a.rs_cap + i], 0), a.shard_rows - 1);
        src = (uint64_t)(sh_shard[s] + (size_t)srow * a.K);
      } else {
        src = (uint64_t)(sh_stage[s] + (size_t)i * a.K);
      }
    }
    const uint64_t dst = (uint64_t)(a.gathered + (size_t)(g0 + lane) * a.K);
    copy_addr(upr, RB, src, dst, info >= 0, row_bytes, lane);
    release_coherent(strict);
    const int n_real = __popcll(ballot(lane < RB && info >= 0));
    if (lane == 0 && n_real > 0) {
      const int rb = g0 / kRB;
      const long long t_pub = (long long)now_ticks();   // issue of the add (publish time under TRACE)
      const int old = fetch_add_relaxed(a.counter_cur + (size_t)rb * kCtr, n_real);
      if (old + n_real > kRB) raise_error(a.err, kErrProtocol, rb);
      if ((a.flags & kTrace) && old + n_real == kRB) a.rb_time[rb] = t_pub;
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming FIFO ring ("DeepEP FIFO pipeline": head/tail credits, slot = index
// mod capacity, finish flag packed beside the tail). Ring r = (shard s =
// r / n_channels, channel k = r % n_channels) carries the 64-row chunks
// c = k, k + n_channels, ... of shard s's stream. Copy workgroup r is its
// producer, copy workgroup rings + r its consumer; both walk the ring's chunks
// in order, so the producer of chunk j waits only on the consumer of chunk
// j - ring_chunks and the consumer of chunk j only on the producer of chunk j.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ring_chunk_count(const FusedArgs& a, int s, int k) {
  const int n_chunks = (a.stream_len[s] + kChunk - 1) / kChunk;
  return n_chunks > k ? (n_chunks - k + a.n_channels - 1) / a.n_channels : 0;
}

__device__ __forceinline__ void ring_producer(const FusedArgs& a, const uint16_t* const* sh_shard, int r, int* sh) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool strict = a.flags & kStrict;
  const int s = r / a.n_channels, k = r - s * a.n_channels;
  if (s == a.self_shard) return;
  const int n_s = __builtin_amdgcn_readfirstlane(a.stream_len[s]);
  const int n_j = __builtin_amdgcn_readfirstlane(ring_chunk_count(a, s, k));
  unsigned long long* tail = a.rtail_cur + (size_t)r * kRingTailStride;
  if (n_j == 0) {
    if (threadIdx.x == 0) __hip_atomic_store(tail, kRingFinish, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int RB = a.rows_per_batch;
  const int upr = (a.K / 8 + 63) / 64;
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const uint16_t* ring = a.ring + (size_t)r * a.ring_chunks * kChunk * a.K;
  constexpr int kRowsPerWave = kChunk / kWaves;
  for (int j = 0; j < n_j; ++j) {
    if (j >= a.ring_chunks) {
      // credit: the consumer has drained chunk j - ring_chunks from this slot
      if (threadIdx.x == 0) {
        uint32_t polls = 0;
        sh[0] = wait_ge(a.rhead_cur + (size_t)r * kCtr, j - a.ring_chunks + 1, now_ticks() + a.timeout_ticks, a.err,
                        0x72000000 | r, &polls);
      }
      __syncthreads();
      const int ok = sh[0];
      __syncthreads();
      if (!ok) return;
    }
    const int c = k + j * a.n_channels;
    const uint16_t* slot = ring + (size_t)(j % a.ring_chunks) * kChunk * a.K;
    for (int b0 = 0; b0 < kRowsPerWave; b0 += RB) {
      const int row = wave * kRowsPerWave + b0 + lane;      // row of the chunk, lane < RB
      const int e = c * kChunk + row;
      const bool valid = lane < RB && b0 + lane < kRowsPerWave && e < n_s;
      int srow = 0;
      if (valid) srow = min(max(a.src_row[s * a.rs_cap + e], 0), a.shard_rows - 1);
      const uint64_t src = (uint64_t)(sh_shard[s] + (size_t)srow * a.K);
      const uint64_t dst = (uint64_t)(slot + (size_t)min(row, kChunk - 1) * a.K);
      copy_addr(upr, RB, src, dst, valid, row_bytes, lane);
    }
    release_coherent(strict);
    __syncthreads();      // every wave's rows of the chunk are acknowledged
    if (threadIdx.x == 0) {
      const unsigned long long w = (unsigned long long)(j + 1) | (j + 1 == n_j ? kRingFinish : 0ull);
      if (strict) __hip_atomic_store(tail, w, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      else __hip_atomic_store(tail, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Bounded wait on a ring tail: returns 1 once tail > j, 2 once the finish flag
// is set with tail == j (the ring is drained), 0 on timeout / error elsewhere.
__device__ __forceinline__ int wait_tail(const unsigned long long* p, int j, uint64_t deadline, const ErrorSink& e,
                                         int id) {
  int lvl = 0;
  uint32_t n = 0;
  while (true) {
    const unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ++n;
    if ((int)(v & 0xFFFFFFFFull) > j) return 1;
    if ((v & kRingFinish) && (int)(v & 0xFFFFFFFFull) == j) return 2;
    if ((n & 15) == 0) {
      if (now_ticks() > deadline) { raise_error(e, kErrTimeout, id); return 0; }
      if (error_raised(e)) return 0;
    }
    backoff(lvl, kBackoffShort);
  }
}

__device__ __forceinline__ void ring_consumer(const FusedArgs& a, const uint16_t* const* sh_shard, int r, int* sh) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool strict = a.flags & kStrict;
  const int s = r / a.n_channels, k = r - s * a.n_channels;
  const bool self = s == a.self_shard;
  const int n_s = __builtin_amdgcn_readfirstlane(a.stream_len[s]);
  const int n_j = __builtin_amdgcn_readfirstlane(ring_chunk_count(a, s, k));
  const unsigned long long* tail = a.rtail_cur + (size_t)r * kRingTailStride;
  const int RB = a.rows_per_batch;
  const int upr = (a.K / 8 + 63) / 64;
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const uint16_t* ring = a.ring + (size_t)r * a.ring_chunks * kChunk * a.K;
  constexpr int kRowsPerWave = kChunk / kWaves;
  for (int j = 0;; ++j) {
    if (self) {
      if (j >= n_j) return;
    } else {
      if (threadIdx.x == 0) sh[0] = wait_tail(tail, j, now_ticks() + a.timeout_ticks, a.err, 0x73000000 | r);
      __syncthreads();
      const int st = sh[0];
      __syncthreads();
      if (st != 1) return;                 // drained (2) or failed (0)
      if (j >= n_j) {                      // more chunks than the stream has
        if (threadIdx.x == 0) raise_error(a.err, kErrProtocol, 0x74000000 | r);
        return;
      }
      if (strict) acquire_agent();
    }
    const int c = k + j * a.n_channels;
    const uint16_t* slot = ring + (size_t)(j % a.ring_chunks) * kChunk * a.K;
    for (int b0 = 0; b0 < kRowsPerWave; b0 += RB) {
      const int row = wave * kRowsPerWave + b0 + lane;
      const int e = c * kChunk + row;
      const bool valid = lane < RB && b0 + lane < kRowsPerWave && e < n_s;
      int d = -1;
      uint64_t src = 0;
      if (valid) {
        d = a.dst_row[s * a.rs_cap + e];
        if (d < 0 || d >= a.m_pad_cap) d = -1;
        if (self) src = (uint64_t)(sh_shard[s] + (size_t)min(max(a.src_row[s * a.rs_cap + e], 0), a.shard_rows - 1) * a.K);
        else src = (uint64_t)(slot + (size_t)row * a.K);
      }
      const uint64_t dst = (uint64_t)(a.gathered + (size_t)max(d, 0) * a.K);
      copy_addr(upr, RB, src, dst, d >= 0, row_bytes, lane);
      release_coherent(strict);
      // arrivals: one add per distinct row block of the batch
      const int rb = d >= 0 ? d / kRB : -1;
      uint64_t pending = ballot(rb >= 0);
      while (pending) {
        const int leader = __ffsll((long long)pending) - 1;
        const int blk = readlane(rb, leader);
        const uint64_t mask = ballot(rb == blk) & pending;
        if (lane == leader) {
          const int cnt = __popcll(mask);
          const long long t_pub = (long long)now_ticks();   // issue of the add (publish time under TRACE)
          const int old = fetch_add_relaxed(a.counter_cur + (size_t)blk * kCtr, cnt);
          if (old + cnt > kRB) raise_error(a.err, kErrProtocol, blk);
          if ((a.flags & kTrace) && old + cnt == kRB) a.rb_time[blk] = t_pub;
        }
        pending &= ~mask;
      }
    }
    __syncthreads();      // every wave has read its rows of the slot
    if (!self && threadIdx.x == 0)
      __hip_atomic_store(a.rhead_cur + (size_t)r * kCtr, j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// In-tile copy ("PCIe sync protocols" §3-§5 carried out inside a compute
// item): a wave of a compute workgroup copies its share of the rows of a later
// round's slabs (fg_plan.hpp), one 1 KB segment (64 lanes x 16 bytes) per K
// loop stage, in the shadow of the stage's MFMAs: the segment loaded in stage
// k is stored in stage k + 1 (device-coherent write-through stores). Once the
// wave's last store has been acknowledged (the wait for the stage loads that
// follows it), each of its rows adds 1 to its 128-row block's arrival counter
// ("PCIe sync protocols" §5, one add per row as on the pages), at a boundary
// between stage pairs; after the K loop each row adds 1 to its chunk's
// election count and the add that completes a chunk publishes seq into the
// chunk's slot (§3).
// Lane l describes row l of the wave (at most 64 rows).
// ---------------------------------------------------------------------------
struct TileCopy {
  const FusedArgs& a;
  CopyPlan plan;
  int x, rho0, n_rows;     // list, first non-lead row and row count of this wave
  int upr;                 // segments per row (K * 2 / 1024)
  int n_seg, seg, r, u;    // segments to load, the next one, its row and segment in the row
  int pend0, pr0, pu0;     // the segment loaded in the last stage waits for its store: row, segment
  int k_mid;               // stage in which the rows are counted
  int counted;             // the counting adds are issued
  long long t_cnt;         // issue time of the counting adds (the TRACE stamp of the blocks they complete)
  uint32_t row_bytes;
  uint32_t g_lo, g_hi;     // the gathered buffer, held in registers (no argument load in the loop)
  bool strict;
  // the wave's rows, entry i for row i: (shard << 24 | stream index, -1 for a
  // padding row), gathered row, source row address (low, high); kept in LDS
  // rather than in lane registers, which the K loop needs for its fragments
  v4i* rows;
  uint32_t voff;           // per lane: byte offset of the lane's 16 bytes in a segment
  v4i data0;               // the segment loaded in the last stage

  __device__ __forceinline__ TileCopy(const FusedArgs& a_, const CopyPlan& p, v4i* wave_rows)
      : a(a_), plan(p), x(0), rho0(0), n_rows(0), upr(1), n_seg(0), seg(0), r(0), u(0), pend0(0), pr0(0), pu0(0),
        k_mid(-1), counted(1), t_cnt(0), row_bytes((uint32_t)a_.K * 2), g_lo((uint32_t)(uintptr_t)a_.gathered),
        g_hi((uint32_t)((uintptr_t)a_.gathered >> 32)),
        strict((a_.flags & kStrict) != 0), rows(wave_rows), voff(0) {}

  // Rows [c0, c1) of list x's non-lead rows for the item; this wave's share.
  __device__ __forceinline__ void begin(int x_, int c0, int c1, int wave, int lane) {
    x = x_;
    // opaque, so that the compiler keeps them instead of reloading the argument inside the loop
    asm volatile("" : "+s"(g_lo), "+s"(g_hi));
    const int n = c1 - c0;
    const int w0 = c0 + n * wave / kWaves, w1 = c0 + n * (wave + 1) / kWaves;
    rho0 = w0;
    n_rows = min(w1 - w0, 64);
    // a lane describes one row: a share above 64 rows would leave rows
    // uncounted, and their gates closed (the schedule never gives one)
    if (w1 - w0 > 64 && lane == 0) raise_error(a.err, kErrProtocol, 0x40000000 | rho0);
    upr = a.K / 512;
    n_seg = n_rows * upr;
    seg = 0; r = 0; u = 0; pend0 = 0;
    counted = n_rows > 0 ? 0 : 1;
    // the last segment is loaded in phase B of stage n_seg - 1 and stored in
    // phase B of stage n_seg + 1; the wait in phase A of stage n_seg + 2
    // acknowledges the store
    k_mid = n_rows > 0 ? n_seg + 1 : -1;
    int info = -1, grow = 0;
    uint32_t src_lo = 0, src_hi = 0;
    // computed by an opaque instruction, so that the compiler keeps it in one
    // register instead of recomputing it into registers the stages reuse
    asm volatile("v_lshlrev_b32 %0, 4, %1" : "=v"(voff) : "v"(lane));
    if (lane < n_rows) {
      grow = plan_row(plan, x, rho0 + lane);
      info = inv_read(a.inv, grow, a.route_ver);
      if (info >= 0) {
        // the source row's address, read here once so that the loop needs no
        // scalar load (whose wait would also cover the stage's LDS reads)
        const uint64_t p = (uint64_t)(a.shards[info >> 24] + (size_t)a.src_of[grow] * a.K);
        src_lo = (uint32_t)p;
        src_hi = (uint32_t)(p >> 32);
      }
    }
    // only this wave reads its entries, and a wave's LDS operations complete in order
    rows[lane] = v4i{info, grow, (int)src_lo, (int)src_hi};
  }

  // Entry i of the wave's rows, the same in every lane (i wave-uniform, < 64).
  __device__ __forceinline__ v4i row_entry(int i) const { return rows[i]; }

  // The copy in the K loop: early in phase B of stage k the wave stores the
  // segment it loaded in stage k - 1 and loads the next one into the same
  // registers; the load's latency hides behind the rest of phase B and phase
  // A of stage k + 1, which ends with the wait for the wave's loads (P, the
  // stage's parity, is not needed: one register set serves every stage).
  // Each is a uniform branch, taken only while there is a segment to move
  // (the branch costs a few scalar instructions; the descriptors and the
  // instructions, issued empty in every stage, cost 4-8 % of the tile).
  // Between a load and its store lies a stage barrier, before which the
  // compiler waits for every memory operation of the wave, so the store does
  // not wait for its data; the store reads its data registers when it issues,
  // so the next load into them need not wait for it; the register set stays
  // allocated through the loop (finish() reads it), so no other value lands
  // in registers a store still reads; the per-lane offset is a register set
  // once per item. With any of these missing, the compiler put a wait for all
  // loads in flight at the top of the stage.
  template <int P>
  __device__ __forceinline__ void store(int) {
    const v4i e = row_entry(pr0);
    if (pend0 && __builtin_amdgcn_readfirstlane(e[0]) >= 0) {
      const int g = __builtin_amdgcn_readfirstlane(e[1]);
      const uint16_t* gbase = (const uint16_t*)(((uint64_t)g_hi << 32) | g_lo);
      const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(gbase + (size_t)g * (row_bytes / 2) + pu0 * 512, 1024u);
      store16_coherent(rd, voff, data0);
    }
    pend0 = 0;
  }

  template <int P>
  __device__ __forceinline__ void load(int) {
    const bool ld = seg < n_seg;
    const v4i e = row_entry(min(r, 63));
    if (ld && __builtin_amdgcn_readfirstlane(e[0]) >= 0) {
      const uint64_t row = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(e[3]) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane(e[2]);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc((const uint16_t*)row + u * 512, 1024u);
      // the registers stay reserved until this load (the store just issued reads them)
      asm volatile("" : "+v"(data0));
      data0 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
    }
    pend0 = ld; pr0 = r; pu0 = u;
    seg += ld;
    const int nu = u + ld;
    const bool wrap = nu == upr;
    u = wrap ? 0 : nu;
    r += wrap;
  }

  // In phase A of stage k, after the wait for the wave's loads (which
  // acknowledged the wave's last store when k > that store's stage): the
  // wave's rows are added to their 128-row blocks' arrival counters, one add
  // per block (reading R5: wave-aggregated adds). Each add is issued by one lane with the
  // counter's address in the buffer descriptor and returns nothing; the
  // stage's barrier waits for it. A block that overshoots is reported by its
  // gate's waiter, which checks for a count above 128.
  __device__ __forceinline__ void mid(int k) {
    if (k == k_mid) count();
  }

  __device__ __forceinline__ void count() {
    const int lane = threadIdx.x & 63;
    if (strict) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    t_cnt = (long long)now_ticks();
    const v4i e = rows[lane];
    const int blk = (lane < n_rows && e[0] >= 0) ? e[1] / kRB : -1;
    uint64_t pending = ballot(blk >= 0);
    while (pending) {
      const int l = __ffsll((long long)pending) - 1;
      const int b = readlane(blk, l);
      const uint64_t m = ballot(blk == b) & pending;
      pending &= ~m;
      if (lane == 0)
        __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(__popcll(m), buffer_rsrc(a.counter_cur + (size_t)b * kCtr, 4),
                                                       0, 0, 0);
    }
    counted = 1;
  }

  // After the K loop: finish the copy if the loop was too short for it, count
  // if not yet done, then elect ("PCIe sync protocols" §3): every row adds 1
  // to its 64-row chunk's election count, and the add that completes a chunk
  // publishes seq into the chunk's slot; an add past the chunk's size is a
  // protocol error.
  __device__ __forceinline__ void finish() {
    // keeps the copy's register set allocated through the K loop
    asm volatile("" ::"v"(data0));
    if (n_rows == 0) return;
    if (!counted) {
      while (pend0 || seg < n_seg) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        store<0>(0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        load<0>(0);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      count();
    }
    const int lane = threadIdx.x & 63;
    const v4i e = rows[lane];
    const int info = e[0], grow = e[1];
    // TRACE: each block's stamp rises to the issue time of this wave's add;
    // the last add to a block completes it, so its stamp is the block's publish
    if ((a.flags & kTrace) && lane < n_rows && info >= 0)
      atomicMax((unsigned long long*)a.rb_time + grow / kRB, (unsigned long long)t_cnt);
    if (lane < n_rows && info >= 0) {
      const int s = info >> 24, c = (info & 0xFFFFFF) / kChunk, ch = s * a.chunk_cap + c;
      const int expect = min(kChunk, a.stream_len[s] - kChunk * c);
      const int old = strict ? fetch_add_acq_rel(a.elect_cur + ch, 1) : fetch_add_relaxed(a.elect_cur + ch, 1);
      if (old + 1 == expect) {
        if (!((a.flags & kDropPublish) && ch == 0)) slot_publish(a.slot + ch, a.seq, strict);
        if (a.flags & kVerify) {
          atomicAdd(a.pub_count + ch, 1);
          atomicAdd(a.stats + ST_PUBLISHES, 1ull);
        }
      } else if (old + 1 > expect) {
        raise_error(a.err, kErrProtocol, 0x10000000 | ch);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Compute role ("PCIe sync protocols" §5 gate).
//
// Work lists. With a grid that is a multiple of the 8 XCDs (workgroup i runs
// on XCD i % 8), XCD x owns the row slabs s = x, x + 8, x + 16, ... (with
// exactly 8 groups, e.g. 8 local experts: the slabs of group x, so that one
// XCD streams one expert's weights) and hands out their tiles from its own
// ticket counter, in groups of GS slabs x GN column tiles, GS * GN =
// workgroups per XCD: the tiles that run at the same time on one XCD share A
// and W lines in that XCD's L2. Slabs are walked in increasing order, the
// order in which the copy role delivers row blocks. (Other grids use one
// list, x = 0, in row-block-major order.)
//
// Split-K tail. When the tiles leave the grid's last round partial, or the
// XCD lists differ in length, the last r tiles of every XCD list are split
// into P k-ranges ("parts"); all parts sit in one global ticket queue, tile by
// tile, taken by any workgroup whose own list is empty. A part stores all
// its fragments to the partial workspace, counts itself in the tile's part
// counter, waits until all P parts have done so, then sums the P partials of
// the fragments it owns, in part order (so deterministic), and stores them.
//
// Every item first waits until each row block it reads has counter == 128,
// acquires, and runs the MFMA tile. Communication workgroups enter this role
// once their rows are copied.
//
// Deadlock freedom: parts of a tile are consecutive tickets of the one part
// queue, so at most one tile at a time has parts not yet taken; its waiting
// holders are at most P-1 workgroups, and every other workgroup either
// computes (and finishes), waits at a gate (whose supplier never waits), or
// waits on a tile whose parts are all taken. With P <= grid some workgroup is
// always free to take the remaining parts.
// ---------------------------------------------------------------------------
struct TileLists {
  int nx;        // lists (8 or 1)
  int n_tn;      // column tiles
  int n_slabs;   // row slabs (256 rows, or 128 at the end of a group)
  bool by_group; // list x = the slabs of group x (8 groups on 8 XCDs), else slabs x, x + nx, ...
  const int* gslab;
  int GN, GS;    // group shape: GS slabs x GN column tiles
  int per_list;  // workgroups per list
  int forced_r;  // split tiles per list when given (>= 0), else -1: leftover of each list
  bool split;    // the tail is split
  bool lead_order;  // in-tile copy: the lead slabs first, then groups (fg_plan.hpp)
  CopyPlan plan;
  __device__ int slabs_of(int x) const { return by_group ? gslab[x + 1] - gslab[x] : (n_slabs - x + nx - 1) / nx; }
  __device__ int slab_at(int x, int i) const { return by_group ? gslab[x] + i : x + nx * i; }
  __device__ int len(int x) const { return slabs_of(x) * n_tn; }
  // split tiles taken from the end of list x
  __device__ int r(int x) const { return !split ? 0 : forced_r >= 0 ? forced_r : len(x) % per_list; }
  // tile of split slot `slot` (slots of list 0 first, then list 1, ...)
  __device__ int split_tile(int slot) const {
    int x = 0, base = 0;
    while (x + 1 < nx && slot >= base + r(x)) { base += r(x); ++x; }
    return tile(x, len(x) - r(x) + (slot - base));
  }
  // tile index (slab * n_tn + column tile) of entry j of list x
  __device__ int tile(int x, int j) const { return tile_in(x, slabs_of(x), by_group ? gslab[x] : 0, j); }
  // the same, given list x's slab count and (grouped lists) first slab, so that
  // a workgroup's own list needs no table load per item
  __device__ int tile_in(int x, int ns, int base, int j) const {
    if (lead_order) return plan_tile(plan, x, j);
    const int g = j / (GS * n_tn);
    const int gs = min(GS, ns - g * GS);
    const int rr = j - g * GS * n_tn;
    const int ng = rr / (gs * GN), r2 = rr - ng * gs * GN;
    const int si = r2 / GN, nn = r2 - si * GN;
    const int si2 = g * GS + si;
    return (by_group ? base + si2 : x + nx * si2) * n_tn + ng * GN + nn;
  }
};

// One work item on a BM-row slab: the tile (whole) or one k-range of it
// (part q of P, split slot `slot`). Returns false if a wait failed.
template <int BM, int BN, class Hook>
__device__ __forceinline__ bool run_item(const FusedArgs& a, char* const* lds, int* sh, int m0, int n0,
                                         int g, int q, int P, int nk2, bool strict, long long& gate,
                                         __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rO,
                                         __amdgpu_buffer_rsrc_t rW, long long* tr, int* pf_tick, int& pf_j,
                                         Hook& cp) {
  using T = Tile<BM, BN>;
  const bool whole = q < 0;
  const int part = whole ? 0 : q % P;
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(a.W + (size_t)g * a.N * a.K, (uint32_t)a.N * row_bytes);
  const int k0 = whole ? 0 : 2 * (nk2 * part / P);
  const int k1 = whole ? 2 * nk2 : 2 * (nk2 * (part + 1) / P);
  Acc<BM, BN> acc;
  acc_zero<BM, BN>(acc);
  uint32_t ver_w[T::VW];
  if (whole) tile_row_versions<BM, BN>(a.inv, m0, ver_w);
  uint32_t padmask = 0;
  // k0, k1 count k-iterations of 64 (128 bytes of a row)
  tile_mainloop<BM, BN>(rA, (uint32_t)m0 * row_bytes + (uint32_t)k0 * 128u, rB,
                        (uint32_t)n0 * row_bytes + (uint32_t)k0 * 128u, row_bytes, k1 - k0, lds[0], lds[1], lds[2],
                        lds[3], acc, cp, whole, ver_w, a.route_ver, padmask);
  cp.finish();
  if (whole) {
    // thread 0 (when pf_tick is given): the next ticket goes out before the
    // stores; the opaque zero keeps the atomic optimizer from rewriting the add
    // into a wave-wide one whose result it needs at once
    if (pf_tick) pf_j = fetch_add_relaxed(pf_tick + opaque_zero(), 1);
    tile_store<BM, BN>(rO, a.N, m0, n0, acc, padmask, lds[0], lds[1]);
    return true;
  }
  // split-K part: blocks of one split tile are 256 x BN floats apart (the
  // largest slab), so one workspace layout serves both slab heights
  const int slot = q / P;
  const uint32_t stride = (uint32_t)(256 * BN * 4);
  const uint32_t base = (uint32_t)slot * (uint32_t)P * stride;
  if (tr && threadIdx.x == 0) tr[4] = now_ticks();
  partial_store<BM, BN>(rW, base + (uint32_t)part * stride, acc);
  release_coherent(strict);
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long t0 = (long long)now_ticks();
    if (tr) tr[5] = t0;
    const int old = fetch_add_relaxed(a.skc_cur + slot, 1);
    int ok = old < P;
    if (!ok) raise_error(a.err, kErrProtocol, 0x20000000 | slot);
    uint32_t polls = 0;
    if (ok) ok = wait_eq(a.skc_cur + slot, P, now_ticks() + a.timeout_ticks, a.err, 0x20000000 | slot, &polls);
    gate += (long long)now_ticks() - t0;
    if (tr) tr[6] = now_ticks();
    sh[2] = ok;
  }
  __syncthreads();
  if (!sh[2]) return false;
  partial_sum_store<BM, BN>(rW, base, stride, part, P, rO, a.N, m0, n0, a.inv, a.route_ver);
  return true;
}

template <int BN>
__device__ __forceinline__ void gemm_role(const FusedArgs& a, char* const* lds, int* sh, long long* wt) {
  if (a.flags & kCommOnly) return;
  const int m_pad = __builtin_amdgcn_readfirstlane(a.desc[0]);
  const int grid = gridDim.x;
  const int nk2 = a.K / 128;                             // pairs of 64-wide k-iterations
  TileLists L;
  L.n_tn = a.N / BN;
  L.n_slabs = __builtin_amdgcn_readfirstlane(a.desc[1]);
  L.nx = (a.tile_order == 0 && grid % kXcds == 0) ? kXcds : 1;
  // the group slab offsets (nine words) are read from LDS: the split tail
  // walks them once per list for every part it hands out
  __shared__ int sh_gslab[kXcds + 1];
  __shared__ v4i sh_copy_rows[kWaves * 64];   // in-tile copy: each wave's row table (TileCopy)
  if (threadIdx.x <= kXcds) sh_gslab[threadIdx.x] = a.gslab[threadIdx.x];
  __syncthreads();
  L.gslab = sh_gslab;
  const int n_groups = __builtin_amdgcn_readfirstlane(a.desc[2]);
  L.by_group = L.nx == kXcds && n_groups == kXcds;
  // one group (the dense routes): the slab table holds 256-row slabs in order,
  // the last one of 128 rows when m_pad is an odd multiple of 128, and every row
  // block is in group 0, so an item's slab entry and group are computed here
  // instead of loaded (one round trip less before each item)
  const bool one_group = n_groups == 1;
  const int per_list = grid / L.nx;                      // workgroups per list
  {
    int gn = 1;
    while (gn * 2 <= min(8, per_list) && L.n_tn % (gn * 2) == 0) gn *= 2;
    L.GN = L.nx == 1 ? L.n_tn : gn;
    L.GS = L.nx == 1 ? 1 : max(1, per_list / gn);
  }
  // in-tile copy (fg_plan.hpp): the lead slabs first in every list; the
  // items copy the other rows unless the gates are pre-opened
  L.lead_order = a.tcopy && L.nx == kXcds && !L.by_group;
  L.plan.n_slabs = L.n_slabs;
  L.plan.half_last = (m_pad % 256) != 0;
  L.plan.nx = kXcds;
  L.plan.per_list = per_list;
  L.plan.n_tn = L.n_tn;
  L.plan.GS = L.GS;
  L.plan.GN = L.GN;
  L.plan.lead = plan_lead_slabs(per_list, L.n_tn);
  const bool copy_in_items = L.lead_order && !(a.flags & kGemmOnly);
  const int n_tiles = L.n_slabs * L.n_tn;
  // Split-K tail. Default: every list keeps a whole number of rounds of whole
  // tiles (a multiple of its workgroups); its leftover tiles are split into
  // P = min(parts cap, k pairs, grid / leftover) k-ranges, so that the parts
  // fill about one round of the grid. With split_tiles given (split_forced),
  // split_tiles / lists tiles are taken from the end of every list, P = cap.
  int R = 0, P = 1;
  {
    int min_len = L.len(0);                            // the shortest list
    for (int xx = 1; xx < L.nx; ++xx) min_len = min(min_len, L.len(xx));
    L.per_list = per_list;
    L.forced_r = a.split_forced ? min(a.split_tiles / L.nx, min_len) : -1;
    L.split = true;
    int rsum = 0;
    for (int xx = 0; xx < L.nx; ++xx) rsum += L.r(xx);
    if (rsum > 0 && n_tiles > grid) {
      P = min(min(a.split_parts, nk2), a.split_forced ? grid : grid / rsum);   // P <= grid: deadlock note
      R = P > 1 ? rsum : 0;
    }
    if (R == 0) { P = 1; L.split = false; }
  }
  const int x = blockIdx.x % L.nx;
  const int my_whole = L.len(x) - L.r(x);
  const int my_ns = L.slabs_of(x), my_base = L.by_group ? L.gslab[x] : 0;
  const bool verify = a.flags & kVerify;
  const bool strict = a.flags & kStrict;
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(a.gathered, (uint32_t)m_pad * row_bytes);
  const __amdgpu_buffer_rsrc_t rO = buffer_rsrc(a.out, (uint32_t)m_pad * (uint32_t)a.N * 2);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(a.skws, a.skws_bytes);
  int* const my_tick = a.tick_cur + (L.nx == 1 ? 64 : 64 * (1 + x));
  int* const part_tick = a.tick_cur;
  long long gate = 0, max_wait = 0;
  int tiles = 0, parts = 0;
  bool own_done = false;                                 // thread 0 only
  // thread 0: the ticket of the next whole tile, taken when the current tile's
  // K loop ends, so that its round trip overlaps the tile's store instead of
  // following it; taken any earlier, a busy workgroup would hold tiles that
  // others, joining later, could run sooner (valid while pf_valid; other lanes
  // leave it undefined, so that no copy of the pending value forces a wait)
  bool pf_valid = false;
  int pf_j;
  const long long t_begin = (long long)now_ticks();
  for (;;) {
    if (threadIdx.x == 0) {
      const long long t_take = (long long)now_ticks();
      int tile = -1, q = -1, entry = 0, jitem = -1;
      // the error flag is read with the item's first loads and examined once
      // they are out (an item taken after an error is dropped)
      const int err_word = poll_relaxed(a.err.dev + opaque_zero());   // stays a per-lane value until used
      if (!own_done) {
        const int j = pf_valid ? pf_j : fetch_add_relaxed(my_tick, 1);
        pf_valid = false;
        if (j < my_whole) { tile = L.tile_in(x, my_ns, my_base, j); jitem = j; }
        else own_done = true;
      }
      if (tile < 0 && R > 0) {
        q = fetch_add_relaxed(part_tick, 1);
        if (q < R * P) {
          tile = L.split_tile(q / P);
        } else {
          q = -1;
        }
      }
      int ok = tile >= 0;
      int grp = 0;
      if (ok) {
        const int si = tile / L.n_tn;
        entry = one_group ? ((si << 8) | (si == (m_pad >> 8) ? 1 : 0)) : a.slab[si];
        const int m0 = entry & ~1, bm = (entry & 1) ? 128 : 256;
        const long long t0 = (long long)now_ticks();
        uint32_t polls = 0;
        // the item's weight group and the first poll of each of its row
        // blocks' counters go out together: one round trip when the gates are
        // open, instead of one per load
        grp = one_group ? 0 : a.group_of_rb[m0 / kRB];
        const bool counters = !(a.flags & kGateWatermark);
        int c0 = kRB, c1 = kRB;
        if (counters) {
          c0 = poll_relaxed(a.counter_cur + (size_t)(m0 / kRB) * kCtr);
          if (bm == 256) c1 = poll_relaxed(a.counter_cur + (size_t)(m0 / kRB + 1) * kCtr);
          polls += bm / kRB;
        }
        if (err_word != 0) ok = 0;
        if ((a.flags & kGateWatermark) && !(a.flags & kGemmOnly)) {   // compute only: nothing to wait for
          // contiguous layout: gathered row g is row g % R of shard g / R, so
          // the tile's rows are covered by whole 64-row chunks of the shard
          // streams; wait for each chunk's slot (its watermark) to carry seq
          const int R = a.shard_rows, M = a.n_shards * R;
          for (int g = m0; g < min(m0 + bm, M) && ok;) {
            const int s = g / R, c = (g - s * R) / kChunk;
            ok = wait_ge(a.slot + s * a.chunk_cap + c, a.seq, now_ticks() + a.timeout_ticks, a.err,
                         0x31000000 | (s * a.chunk_cap + c), &polls);
            g = s * R + min(R, (c + 1) * kChunk);
          }
        } else if (counters) {
          // a block not yet complete (or overshot) goes to the bounded wait,
          // which also reports an overshoot
          if (ok && c0 != kRB)
            ok = wait_eq(a.counter_cur + (size_t)(m0 / kRB) * kCtr, kRB, now_ticks() + a.timeout_ticks, a.err,
                         m0 / kRB, &polls, kBackoffLong);
          if (ok && c1 != kRB)
            ok = wait_eq(a.counter_cur + (size_t)(m0 / kRB + 1) * kCtr, kRB, now_ticks() + a.timeout_ticks, a.err,
                         m0 / kRB + 1, &polls, kBackoffLong);
        }
        const long long t_open = (long long)now_ticks();
        gate += t_open - t0;
        max_wait = max(max_wait, t_open - t0);
        if (verify) {
          atomicAdd(a.stats + ST_GATE_POLLS, (unsigned long long)polls);
          if (ok) atomicAdd(a.stats + ST_GATE_PASSES, 1ull);
        }
        const int tr_id = q < 0 ? tile : n_tiles + q;
        if ((a.flags & kTrace) && tr_id < a.trace_cap) {
          long long* tr = a.trace + (size_t)tr_id * kTraceFields;
          tr[0] = blockIdx.x; tr[1] = t_take; tr[2] = t_open; tr[3] = 0; tr[4] = 0; tr[5] = 0; tr[6] = 0;
        }
      }
      sh[0] = tile;
      sh[1] = ok;
      sh[3] = q;
      sh[4] = entry;
      sh[5] = grp;
      sh[6] = jitem;
    }
    __syncthreads();
    const int tile = __builtin_amdgcn_readfirstlane(sh[0]);
    const int q = __builtin_amdgcn_readfirstlane(sh[3]);
    const int entry = __builtin_amdgcn_readfirstlane(sh[4]);
    const int g = __builtin_amdgcn_readfirstlane(sh[5]);
    const int jitem = __builtin_amdgcn_readfirstlane(sh[6]);
    if (!sh[1]) break;
    // the tile reads the gathered rows with device-scope loads issued after the
    // gate poll returned 128; the formal acquire fence is the strict variant
    if (strict) acquire_agent();
    const int m0 = entry & ~1, n0 = (tile - (tile / L.n_tn) * L.n_tn) * BN;
    const int tr_id = q < 0 ? tile : n_tiles + q;
    long long* tr = ((a.flags & kTrace) && q >= 0 && tr_id < a.trace_cap) ? a.trace + (size_t)tr_id * kTraceFields
                                                                            : nullptr;
    int* const pf_tick = (threadIdx.x == 0 && q < 0 && !own_done) ? my_tick : nullptr;
    const long long gate_before = gate;
    // an item with rows to copy runs the loop with the copy; every other item without it
    int c0 = 0, c1 = 0;
    if (copy_in_items && q < 0 && jitem >= 0) plan_item_rows(L.plan, x, jitem, &c0, &c1);
    bool ok;
    if (c1 > c0) {
      TileCopy cp(a, L.plan, sh_copy_rows + 64 * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
      cp.begin(x, c0, c1, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63);
      ok = (entry & 1) ? run_item<128, BN>(a, lds, sh, m0, n0, g, q, P, nk2, strict, gate, rA, rO, rW, tr, pf_tick,
                                           pf_j, cp)
                       : run_item<256, BN>(a, lds, sh, m0, n0, g, q, P, nk2, strict, gate, rA, rO, rW, tr, pf_tick,
                                           pf_j, cp);
    } else {
      NoHook nh;
      ok = (entry & 1) ? run_item<128, BN>(a, lds, sh, m0, n0, g, q, P, nk2, strict, gate, rA, rO, rW, tr, pf_tick,
                                           pf_j, nh)
                       : run_item<256, BN>(a, lds, sh, m0, n0, g, q, P, nk2, strict, gate, rA, rO, rW, tr, pf_tick,
                                           pf_j, nh);
    }
    if (pf_tick) pf_valid = true;
    max_wait = max(max_wait, gate - gate_before);   // a split-K part's wait for its siblings
    if (!ok) break;
    if (q < 0) ++tiles; else ++parts;
    if ((a.flags & kTrace) && threadIdx.x == 0 && tr_id < a.trace_cap) a.trace[(size_t)tr_id * kTraceFields + 3] = now_ticks();
  }
  if (threadIdx.x == 0) {
    wt[WT_GATE] = gate;
    wt[WT_MAXWAIT] = max_wait;
    wt[WT_TILES] = tiles;
    wt[WT_PARTS] = parts;
    wt[WT_GEMM_START] = t_begin;
    wt[WT_P] = R > 0 ? P : 1;
  }
}

template <int BN>
__global__ __launch_bounds__(kThreads, 1) void fused_kernel(FusedArgs) {
  const FusedArgs& a = kernel_arg<FusedArgs>();
  // one array per LDS stage (distinct objects for the compiler's wait placement)
  constexpr int kS23 = kStages == 4 ? Tile<256, BN>::STAGE : 16;
  __shared__ __attribute__((aligned(16))) char lds0[Tile<256, BN>::STAGE];
  __shared__ __attribute__((aligned(16))) char lds1[Tile<256, BN>::STAGE];
  __shared__ __attribute__((aligned(16))) char lds2[kS23];
  __shared__ __attribute__((aligned(16))) char lds3[kS23];
  char* const lds[4] = {lds0, lds1, lds2, lds3};
  __shared__ const uint16_t* sh_shard[FG_MAX_SHARDS];
  __shared__ int sh[8];   // item broadcast: tile, ok, part ok, part, slab entry, group, list item
  long long* wt = a.wgtime + (size_t)blockIdx.x * kWgTimeFields;
  const long long t_start = (long long)now_ticks();
  const long long c_start = (long long)__builtin_amdgcn_s_memtime();
  long long t_comm = 0;
  if (threadIdx.x == 0) {
    wt[WT_GATE] = 0; wt[WT_TILES] = 0; wt[WT_PARTS] = 0; wt[WT_GEMM_START] = 0; wt[WT_P] = 1;
  }
  if (blockIdx.x < a.n_comm) {
    __shared__ uint16_t* sh_stage[FG_MAX_SHARDS];
    __shared__ int sh_pbase[FG_MAX_SHARDS + 1];   // push batches before shard s (two-stage)
    if (threadIdx.x < a.n_shards) {
      sh_shard[threadIdx.x] = a.shards[threadIdx.x];
      sh_stage[threadIdx.x] = a.staging[threadIdx.x];
    }
    if (a.two_stage && threadIdx.x == 0) {
      int n = 0;
      for (int s = 0; s < a.n_shards; ++s) {
        sh_pbase[s] = n;
        if (s != a.self_shard) n += (a.stream_len[s] + a.rows_per_batch - 1) / a.rows_per_batch;
      }
      sh_pbase[a.n_shards] = n;
    }
    __syncthreads();
    arm_next(a);
    // VERIFY: the publishes this call should make, one per active 64-row chunk
    // of every stream whose slots it publishes (all shards in the one-stage
    // copy, the remote ones in the two-stage push; the ring publishes none)
    if (blockIdx.x == 0 && threadIdx.x == 0 && (a.flags & kVerify) && !(a.flags & kGemmOnly) && !a.ring_mode) {
      unsigned long long want = 0;
      for (int s2 = 0; s2 < a.n_shards; ++s2)
        if (!(a.two_stage && s2 == a.self_shard)) want += (a.stream_len[s2] + kChunk - 1) / kChunk;
      atomicAdd(a.stats + ST_EXPECTED, want);
    }
    const int rings = a.n_shards * a.n_channels;
    if (a.ring_mode) {
      __shared__ int sh_ring[2];
      if (!(a.flags & kGemmOnly)) {
        if ((int)blockIdx.x < rings) ring_producer(a, sh_shard, blockIdx.x, sh_ring);
        else if ((int)blockIdx.x < 2 * rings) ring_consumer(a, sh_shard, blockIdx.x - rings, sh_ring);
      }
    } else if (a.two_stage) {
      if (!(a.flags & kGemmOnly)) comm_two_stage(a, sh_shard, sh_stage, sh_pbase);
    } else {
      comm_role(a, sh_shard);
    }
    t_comm = (long long)now_ticks();
  }
  gemm_role<BN>(a, lds, sh, wt);
  if (threadIdx.x == 0) {
    wt[WT_CLK1] = (long long)__builtin_amdgcn_s_memtime();
    wt[WT_START] = t_start;
    wt[WT_END] = (long long)now_ticks();
    wt[WT_COMM_END] = t_comm;
    wt[WT_CLK0] = c_start;
  }
}

// ---------------------------------------------------------------------------
// Layout step (step a1): the route tables, the inverse map gathered row ->
// (shard, stream index), the padding seed of every row block, and the arming
// of the current parity (counters = seed, election counts = 0).
//
// The inverse map is versioned: entry = (route version << 32) | value, and an
// entry whose version is not the current one reads as a padding row, so no
// pass clears it between routes. Work that needs every workgroup's result is
// done by the last workgroup to finish (agent-scope release by each, acquire
// by the last), which also resets the shared scratch for the next call.
// ---------------------------------------------------------------------------
struct RouteArgs {
  int mode;                  // FG_ROUTE_*
  int n_shards, rs_cap, chunk_cap, rb_cap, m_pad_cap;
  int rows_per_shard;        // CONTIG / EXPLICIT: rows of every shard; TOPK: tokens of every shard
  int m_pad;                 // CONTIG / EXPLICIT
  int n_groups;
  int group_off[FG_MAX_GROUPS + 1];   // EXPLICIT (host-given)
  int stream_len_in[FG_MAX_SHARDS];   // EXPLICIT (host-given)
  const int* src_in;         // EXPLICIT device
  const int* dst_in;
  const int* topk;           // TOPK device [S][T][KK]
  int topk_k, expert_base;
  int wpb;                   // TOPK: workgroups per shard
  int n_wg;                  // TOPK: workgroups of the layout grid
  uint64_t timeout_ticks;    // TOPK in one kernel: watchdog of the wait for the scan
  uint32_t ver;              // route version stamped into the inverse map
  int* src_row;
  int* dst_row;
  int* stream_len;
  int* group_off_out;
  unsigned long long* inv;
  int* src_of;               // [m_pad_cap] source row of each gathered row (read with the inverse map)
  int* seed;
  int* group_of_rb;
  int* rbcount;              // EXPLICIT: [rb_cap][kRbSlots] real rows per row block, in slots (zero between calls)
  int* counter_cur;          // [rb_cap][kCtr]
  int* elect_cur;
  int* desc;
  int* slab;                 // row slab table (see FusedArgs)
  int* gslab;                // first slab of each group
  int* wgcount;              // TOPK: [n_wg][E + 1] per-workgroup expert counts, picks
  int* wgbase;               // TOPK: [n_wg][E + 1] expert row bases, stream base
  int* src_k;                // TOPK: [S][rs_cap] top-k position of each stream entry
  int* tok_first;            // TOPK: [S][rs_cap + 1] first stream entry of each token; [T] = stream length
  int* ticket;               // [0] last-workgroup ticket, [1] failure flag (zero between calls),
                             // [2] failure of the last layout, [3] route version whose scan is done
  ErrorSink err;
};

constexpr int kRouteThreads = 256;
// EXPLICIT: each row block's real-row count is spread over kRbSlots words
// (workgroup w adds to slot w % kRbSlots), which the last workgroup sums. With
// one word per block, a block's 128 adds arrive at the same address from 128
// threads: measured 22.5 us per Large layout (a permutation of 32768 rows),
// 13.0 us with 8 slots, 14.9 us with 32 (the sums and clears then cost more).
constexpr int kRbSlots = 8;
static_assert((kRbSlots & (kRbSlots - 1)) == 0, "slot of workgroup w = w & (kRbSlots - 1)");


// True in every thread of the workgroup that finishes last.
__device__ bool last_workgroup(int* ticket, int* sh) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int t = atomicAdd(ticket, 1);
    *sh = (t == (int)gridDim.x - 1);
  }
  __syncthreads();
  const bool last = *sh;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// Row slabs of the compute role (one workgroup): every group [goff[g],
// goff[g+1]) (multiples of 128 rows) is cut into 256-row slabs and, when its
// size is an odd number of row blocks, one last 128-row slab, so that no slab
// straddles two groups. Entry = first row | (128-row slab ? 1 : 0).
__device__ void build_slabs(const int* goff, int n_groups, int* slab, int* gslab, int* desc) {
  __shared__ int sh_base[FG_MAX_GROUPS + 1];
  if (threadIdx.x == 0) {
    int n = 0;
    for (int g = 0; g < n_groups; ++g) {
      sh_base[g] = n;
      const int S = goff[g + 1] - goff[g];
      n += S / 256 + (S % 256 ? 1 : 0);
    }
    sh_base[n_groups] = n;
    desc[1] = n;
    desc[2] = n_groups;
  }
  __syncthreads();
  for (int g = 0; g < n_groups; ++g) {
    const int S = goff[g + 1] - goff[g], n256 = S / 256, ns = n256 + (S % 256 ? 1 : 0);
    for (int j = threadIdx.x; j < ns; j += blockDim.x) slab[sh_base[g] + j] = (goff[g] + 256 * j) | (j == n256 ? 1 : 0);
  }
  if ((int)threadIdx.x <= n_groups) gslab[threadIdx.x] = sh_base[threadIdx.x];
}

// Seeds, group of each row block, arming, row slabs; real(rb) gives the real rows of rb.
// failed: the route was rejected (m_pad is then 0 and goff may be invalid, so no
// slab is built and the descriptor reports no groups); an empty valid route
// keeps its groups, all of them empty.
template <class Real>
__device__ void route_finish(const RouteArgs& a, int m_pad, const int* goff, int n_groups, bool failed, Real real) {
  const int n_rb = m_pad / kRB;
  for (int rb = threadIdx.x; rb < a.rb_cap; rb += blockDim.x) {
    int sd = 0, g = 0;
    if (rb < n_rb) {
      sd = kRB - real(rb);
      for (int j = 0; j < n_groups; ++j)
        if (rb * kRB >= goff[j] && rb * kRB < goff[j + 1]) g = j;
    }
    a.seed[rb] = sd;
    a.group_of_rb[rb] = g;
    a.counter_cur[(size_t)rb * kCtr] = sd;
  }
  for (int i = threadIdx.x; i < a.n_shards * a.chunk_cap; i += blockDim.x) a.elect_cur[i] = 0;
  if ((int)threadIdx.x <= n_groups) a.group_off_out[threadIdx.x] = goff[threadIdx.x];
  if (threadIdx.x == 0) a.desc[0] = m_pad;
  build_slabs(goff, failed ? 0 : n_groups, a.slab, a.gslab, a.desc);
}

// CONTIG: shard s row i -> gathered row s*R + i; everything is arithmetic, so
// every thread works independently.
__global__ __launch_bounds__(kRouteThreads) void route_contig_kernel(RouteArgs a) {
  const int R = a.rows_per_shard, M = a.n_shards * R, m_pad = a.m_pad;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x, nth = gridDim.x * blockDim.x;
  for (int g = tid; g < M; g += nth) {
    const int s = g / R, i = g - s * R;
    a.inv[g] = inv_pack(a.ver, (s << 24) | i);
    a.src_of[g] = i;
    a.src_row[s * a.rs_cap + i] = i;
    a.dst_row[s * a.rs_cap + i] = g;
  }
  const int n_rb = m_pad / kRB;
  for (int rb = tid; rb < a.rb_cap; rb += nth) {
    const int real = rb < n_rb ? min(kRB, max(0, M - rb * kRB)) : kRB;
    const int sd = kRB - real;
    a.seed[rb] = sd;
    a.group_of_rb[rb] = 0;
    a.counter_cur[(size_t)rb * kCtr] = sd;
  }
  for (int i = tid; i < a.n_shards * a.chunk_cap; i += nth) a.elect_cur[i] = 0;
  const int n256 = m_pad / 256, n_slabs = n256 + (m_pad % 256 ? 1 : 0);
  for (int j = tid; j < n_slabs; j += nth) a.slab[j] = (256 * j) | (j == n256 ? 1 : 0);
  if (tid < a.n_shards) a.stream_len[tid] = R;
  if (tid == 0) {
    a.group_off_out[0] = 0; a.group_off_out[1] = m_pad;
    a.desc[0] = m_pad; a.desc[1] = n_slabs; a.desc[2] = 1;
    a.gslab[0] = 0; a.gslab[1] = n_slabs;
  }
}

// EXPLICIT: one thread per stream entry; the last workgroup computes the seeds.
__global__ __launch_bounds__(kRouteThreads) void route_explicit_kernel(RouteArgs a) {
  __shared__ int sh_last;
  __shared__ int sh_goff[FG_MAX_GROUPS + 1];
  const int tid = blockIdx.x * blockDim.x + threadIdx.x, nth = gridDim.x * blockDim.x;
  for (int f = tid; f < a.n_shards * a.rs_cap; f += nth) {
    const int s = f / a.rs_cap, i = f - s * a.rs_cap;
    if (i >= a.stream_len_in[s]) continue;
    const int src = a.src_in[f], dst = a.dst_in[f];
    if (dst < 0 || dst >= a.m_pad || src < 0 || src >= a.rows_per_shard) {
      raise_error(a.err, kErrProtocol, 0x20000000 | s);
      atomicOr(a.ticket + 1, 1);
      continue;
    }
    a.src_row[f] = src;
    a.dst_row[f] = dst;
    a.src_of[dst] = src;
    const unsigned long long old = atomicExch(a.inv + dst, inv_pack(a.ver, (s << 24) | i));
    if ((uint32_t)(old >> 32) == a.ver) {
      raise_error(a.err, kErrProtocol, 0x30000000 | dst);
      atomicOr(a.ticket + 1, 1);
    }
    atomicAdd(a.rbcount + (dst / kRB) * kRbSlots + (blockIdx.x & (kRbSlots - 1)), 1);
  }
  if (!last_workgroup(a.ticket, &sh_last)) return;
  if ((int)threadIdx.x <= a.n_groups) sh_goff[threadIdx.x] = a.group_off[threadIdx.x];
  if ((int)threadIdx.x < a.n_shards) a.stream_len[threadIdx.x] = a.stream_len_in[threadIdx.x];
  __syncthreads();
  const int fail = __hip_atomic_load(a.ticket + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  route_finish(a, fail ? 0 : a.m_pad, sh_goff, a.n_groups, fail != 0, [&](int rb) {
    int n = 0;
    for (int j = 0; j < kRbSlots; ++j)
      n += __hip_atomic_load(a.rbcount + rb * kRbSlots + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return n;
  });
  __syncthreads();
  for (int i = threadIdx.x; i < a.rb_cap * kRbSlots; i += blockDim.x) a.rbcount[i] = 0;
  if (threadIdx.x == 0) { a.ticket[0] = 0; a.ticket[1] = 0; }
}

// TOPK layout, both passes: each workgroup takes 256 consecutive tokens of one
// shard and first copies their top-k lists into LDS, one byte per choice: the
// local expert index, or 0xFF for an expert this GPU does not own.

__device__ __forceinline__ int stage_topk(const RouteArgs& a, uint8_t* sh_tk, int s, int t0) {
  const int E = a.n_groups, KK = a.topk_k, T = a.rows_per_shard;
  const int ntok = min(kRouteThreads, T - t0);
  const int* src = a.topk + ((size_t)s * T + t0) * KK;
  for (int i = threadIdx.x; i < ntok * KK; i += blockDim.x) {
    const int e = src[i] - a.expert_base;
    sh_tk[i] = (e >= 0 && e < E) ? (uint8_t)e : (uint8_t)0xFF;
  }
  return ntok;
}

// TOPK, counting: per workgroup the number of its tokens choosing each local
// expert and its number of local pairs (one wave ballot and one LDS add per
// wave and expert); top-k lists already staged in sh_tk.
__device__ void topk_count(const RouteArgs& a, const uint8_t* sh_tk, int* sh_cnt, int w, int s, int t0) {
  const int E = a.n_groups, KK = a.topk_k, T = a.rows_per_shard, t = t0 + threadIdx.x;
  unsigned long long mask = 0;
  if (t < T) {
    const uint8_t* tk = sh_tk + threadIdx.x * KK;
    for (int k = 0; k < KK; ++k) {
      const int e = tk[k];
      if (e == 0xFF) continue;
      if ((mask >> e) & 1ull) {   // one token routed twice to one expert: not a valid top-k
        raise_error(a.err, kErrProtocol, 0x48000000 | s);
        atomicOr(a.ticket + 1, 1);
        continue;
      }
      mask |= 1ull << e;
    }
  }
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int e = 0; e < E; ++e) {
    const int n = __popcll(ballot((mask >> e) & 1ull));
    total += n;
    if (lane == 0 && n) atomicAdd(sh_cnt + e, n);
  }
  if (lane == 0 && total) atomicAdd(sh_cnt + E, total);
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) a.wgcount[w * (E + 1) + e] = sh_cnt[e];
}

// TOPK, the last workgroup: scans the counts in global token order (workgroup
// order) into relative expert row bases and per-shard stream bases ("DeepEP
// FIFO pipeline" dispatch notify stage: counts fix the offsets), then the group
// offsets (each expert padded to a multiple of 128 rows), seeds, arming and the
// slab table; resets the last-workgroup ticket and records failure in ticket[2].
// Column e < E is an exclusive scan over the workgroups, 64 at a time, one
// wave per column; column E one thread per shard over its workgroups.
__device__ void topk_scan_finish(const RouteArgs& a, int* sh_goff, int* sh_ne) {
  const int E = a.n_groups, T = a.rows_per_shard;
  const int n_wg = a.n_wg;
  {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    for (int e = wave; e < E; e += nwaves) {
      int carry = 0;
      for (int v0 = 0; v0 < n_wg; v0 += 64) {
        const int v = v0 + lane;
        const int x = v < n_wg ? a.wgcount[v * (E + 1) + e] : 0;
        int incl = x;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(incl, d, 64);
          if (lane >= d) incl += y;
        }
        if (v < n_wg) a.wgbase[v * (E + 1) + e] = carry + incl - x;
        carry += __shfl(incl, 63, 64);
      }
      if (lane == 0) sh_ne[e] = carry;
    }
    if ((int)threadIdx.x < a.n_shards) {
      const int sp = threadIdx.x;
      int run = 0;
      for (int v = sp * a.wpb; v < (sp + 1) * a.wpb; ++v) {
        a.wgbase[v * (E + 1) + E] = run;
        run += a.wgcount[v * (E + 1) + E];
      }
      a.stream_len[sp] = run;
      a.tok_first[(size_t)sp * (a.rs_cap + 1) + T] = run;
      if (run > a.rs_cap) { raise_error(a.err, kErrProtocol, 0x40000000 | sp); atomicOr(a.ticket + 1, 1); }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int off = 0;
    sh_goff[0] = 0;
    for (int e = 0; e < E; ++e) {
      off += ((sh_ne[e] + kRB - 1) / kRB) * kRB;
      sh_goff[e + 1] = off;
    }
    if (off > a.m_pad_cap) { raise_error(a.err, kErrProtocol, 0x50000000); atomicOr(a.ticket + 1, 1); }
  }
  __syncthreads();
  const int fail = __hip_atomic_load(a.ticket + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  route_finish(a, fail ? 0 : sh_goff[E], sh_goff, E, fail != 0, [&](int rb) {
    int real = 0;
    for (int j = 0; j < E; ++j)
      if (rb * kRB >= sh_goff[j] && rb * kRB < sh_goff[j + 1]) real = min(kRB, max(0, sh_ne[j] - (rb * kRB - sh_goff[j])));
    return real;
  });
  __syncthreads();
  if (threadIdx.x == 0) { a.ticket[0] = 0; a.ticket[2] = fail; a.ticket[1] = 0; }
}

// TOPK, placing every local pair of this workgroup's tokens (lists in sh_tk,
// sh_base = absolute expert row bases, [E] = stream base). The rank of a token
// among those choosing expert e comes from wave ballots (tokens are in thread
// order, i.e. global token order); the stream index from a scan of the local
// pick counts.
__device__ void topk_place(const RouteArgs& a, const uint8_t* sh_tk, const int* sh_base, int (*sh_wave)[kRouteThreads / 64],
                           int* sh_pick, uint8_t* sh_kpos, int s, int t0) {
  const int E = a.n_groups, KK = a.topk_k, T = a.rows_per_shard, t = t0 + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* tk = sh_tk + threadIdx.x * KK;
  // one pass over the list: the experts chosen, the list positions holding a
  // local expert, and each local expert's position (sh_kpos[e][thread])
  unsigned long long mask = 0, lpos = 0;
  if (t < T)
    for (int k = 0; k < KK; ++k) {
      const int e = tk[k];
      if (e != 0xFF) {
        mask |= 1ull << e;
        lpos |= 1ull << k;
        sh_kpos[e * kRouteThreads + threadIdx.x] = (uint8_t)k;
      }
    }
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int e = 0; e < E; ++e) {
    const unsigned long long b = ballot((mask >> e) & 1ull);
    if (lane == 0) sh_wave[e][wave] = __popcll(b);
  }
  const int picks = __popcll(mask);
  int x = picks;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh_pick[wave] = x;
  __syncthreads();
  int pick_base = x - picks;
  for (int v = 0; v < wave; ++v) pick_base += sh_pick[v];
  const int stream0 = sh_base[E] + pick_base;
  if (t < T) a.tok_first[(size_t)s * (a.rs_cap + 1) + t] = stream0;
  for (int e = 0; e < E; ++e) {
    const bool f = (mask >> e) & 1ull;
    const unsigned long long b = ballot(f);
    if (!f) continue;
    int rank = sh_base[e] + __popcll(b & lt);
    for (int v = 0; v < wave; ++v) rank += sh_wave[e][v];
    const int kk = sh_kpos[e * kRouteThreads + threadIdx.x];        // e's position in the token's list
    const int i = stream0 + __popcll(lpos & ((1ull << kk) - 1ull));  // after the local picks ahead of it
    a.src_row[s * a.rs_cap + i] = t;
    a.src_k[s * a.rs_cap + i] = kk;
    a.dst_row[s * a.rs_cap + i] = rank;
    a.src_of[rank] = t;
    a.inv[rank] = inv_pack(a.ver, (s << 24) | i);
  }
}

// Absolute bases of workgroup w into sh_base (the group offsets are final).
__device__ __forceinline__ int topk_base_load(const RouteArgs& a, int w) {
  const int E = a.n_groups;
  int base = 0;
  if ((int)threadIdx.x <= E)
    base = a.wgbase[w * (E + 1) + threadIdx.x] + ((int)threadIdx.x < E ? a.group_off_out[threadIdx.x] : 0);
  return base;
}

// TOPK in one kernel (the grid is co-resident, checked by the host): count,
// the last workgroup scans and publishes the route version in ticket[3], the
// others wait for it (a bounded wait on a supplier that never waits) and
// place their pairs from the lists still in LDS.
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(RouteArgs a) {
  __shared__ uint8_t sh_tk[kRouteThreads * 64];
  __shared__ int sh_cnt[FG_MAX_GROUPS + 1];
  __shared__ int sh_last;
  __shared__ int sh_goff[FG_MAX_GROUPS + 1];
  __shared__ int sh_ne[FG_MAX_GROUPS];
  __shared__ int sh_wave[FG_MAX_GROUPS + 1][kRouteThreads / 64];
  __shared__ int sh_pick[kRouteThreads / 64];
  __shared__ int sh_base[FG_MAX_GROUPS + 1];
  __shared__ uint8_t sh_kpos[FG_MAX_GROUPS * kRouteThreads];
  __shared__ int sh_ok;
  const int E = a.n_groups;
  const int w = blockIdx.x, s = w / a.wpb, t0 = (w - s * a.wpb) * kRouteThreads;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) sh_cnt[e] = 0;
  stage_topk(a, sh_tk, s, t0);
  __syncthreads();
  topk_count(a, sh_tk, sh_cnt, w, s, t0);
  if (last_workgroup(a.ticket, &sh_last)) {
    topk_scan_finish(a, sh_goff, sh_ne);
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(a.ticket + 3, (int)a.ver, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh_ok = 1;
    }
  } else if (threadIdx.x == 0) {
    uint32_t polls = 0;
    sh_ok = wait_ge(a.ticket + 3, (int)a.ver, now_ticks() + a.timeout_ticks, a.err, 0x75000000, &polls);
  }
  __syncthreads();
  if (!sh_ok) return;
  acquire_agent();
  if (__hip_atomic_load(a.ticket + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;   // layout failed
  const int base = topk_base_load(a, w);
  if ((int)threadIdx.x <= E) sh_base[threadIdx.x] = base;
  __syncthreads();
  topk_place(a, sh_tk, sh_base, sh_wave, sh_pick, sh_kpos, s, t0);
}

// TOPK in two kernels, for grids that are not co-resident: pass 1 counts and
// the last workgroup scans; pass 2 places.
__global__ __launch_bounds__(kRouteThreads) void route_topk_count_kernel(RouteArgs a) {
  __shared__ uint8_t sh_tk[kRouteThreads * 64];
  __shared__ int sh_cnt[FG_MAX_GROUPS + 1];
  __shared__ int sh_last;
  __shared__ int sh_goff[FG_MAX_GROUPS + 1];
  __shared__ int sh_ne[FG_MAX_GROUPS];
  const int E = a.n_groups;
  const int w = blockIdx.x, s = w / a.wpb, t0 = (w - s * a.wpb) * kRouteThreads;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) sh_cnt[e] = 0;
  stage_topk(a, sh_tk, s, t0);
  __syncthreads();
  topk_count(a, sh_tk, sh_cnt, w, s, t0);
  if (!last_workgroup(a.ticket, &sh_last)) return;
  topk_scan_finish(a, sh_goff, sh_ne);
}

__global__ __launch_bounds__(kRouteThreads) void route_topk_place_kernel(RouteArgs a) {
  __shared__ uint8_t sh_tk[kRouteThreads * 64];
  __shared__ int sh_wave[FG_MAX_GROUPS + 1][kRouteThreads / 64];
  __shared__ int sh_pick[kRouteThreads / 64];
  __shared__ int sh_base[FG_MAX_GROUPS + 1];
  __shared__ uint8_t sh_kpos[FG_MAX_GROUPS * kRouteThreads];
  const int E = a.n_groups;
  const int w = blockIdx.x, s = w / a.wpb, t0 = (w - s * a.wpb) * kRouteThreads;
  // the failure flag, this workgroup's bases and its top-k lists are loaded
  // together (one memory round trip); nothing is written before the flag is seen
  const int failed = __hip_atomic_load(a.ticket + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int base = topk_base_load(a, w);
  stage_topk(a, sh_tk, s, t0);
  if ((int)threadIdx.x <= E) sh_base[threadIdx.x] = base;
  __syncthreads();
  if (failed) return;   // layout failed: the tables stay as they are
  topk_place(a, sh_tk, sh_base, sh_wave, sh_pick, sh_kpos, s, t0);
}

// Small helpers: fill, poke (fault injection on a counter).
// p[i * stride] = v for i < n
__global__ void fill_kernel(int* p, int n, int v, int stride) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[(size_t)i * stride] = v;
}
__global__ void poke_kernel(int* p, int delta) {
  if (threadIdx.x == 0 && blockIdx.x == 0) p[0] += delta;
}

// ---------------------------------------------------------------------------
// All-rank slot barrier ("PCIe sync protocols" §2): one workgroup per virtual
// rank, lane j < n stores bseq into bslot[j][me] (my slot on rank j) and waits
// on bslot[me][j] (the local slot rank j writes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64, 1) void barrier_kernel(int* bslot, int n, int bseq0, int rounds, ErrorSink e,
                                                        uint64_t timeout, long long* t_out) {
  const int me = blockIdx.x, lane = threadIdx.x;
  const long long t0 = (long long)now_ticks();
  uint32_t polls = 0;
  for (int r = 1; r <= rounds; ++r) {
    const int seq = bseq0 + r;
    int ok = 1;
    if (lane < n) {
      slot_publish(bslot + lane * n + me, seq, false);
      ok = wait_ge(bslot + me * n + lane, seq, now_ticks() + timeout, e, 0x60000000 | me, &polls);
    }
    if (ballot(!ok)) return;
  }
  if (me == 0 && lane == 0) t_out[0] = (long long)now_ticks() - t0;
}

// Slot ping-pong between workgroup 0 and workgroup 1 (different XCDs). Every
// poll is followed by the shortest s_sleep (64 clocks): the wait backs off
// like every other wait, but does not double, since the round trip it
// measures is a few hundred nanoseconds and a longer sleep would be measured
// with it.
template <int SYS>
__device__ __forceinline__ int pp_load(const int* p) {
  return SYS ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : poll_relaxed(p);
}
template <int SYS>
__device__ __forceinline__ void pp_store(int* p, int v) {
  if (SYS) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// one lane: wait until *p >= seq; false on timeout
template <int SYS>
__device__ __forceinline__ bool pp_wait(const int* p, int seq, uint64_t timeout, const ErrorSink& e, int id) {
  const uint64_t dl = now_ticks() + timeout;
  while (pp_load<SYS>(p) < seq) {
    if (now_ticks() > dl) { raise_error(e, kErrTimeout, id); return false; }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

template <int SYS>
__global__ __launch_bounds__(64, 1) void pingpong_kernel(int* a_slot, int* b_slot, int base, int rounds, ErrorSink e,
                                                         uint64_t timeout, long long* t_out) {
  if (threadIdx.x != 0) return;
  const long long t0 = (long long)now_ticks();
  for (int r = 1; r <= rounds; ++r) {
    const int seq = base + r;
    if (blockIdx.x == 0) {
      pp_store<SYS>(a_slot, seq);
      if (!pp_wait<SYS>(b_slot, seq, timeout, e, 0x70000000)) return;
    } else {
      if (!pp_wait<SYS>(a_slot, seq, timeout, e, 0x70000001)) return;
      pp_store<SYS>(b_slot, seq);
    }
  }
  if (blockIdx.x == 0) t_out[0] = (long long)now_ticks() - t0;
}

// ---------------------------------------------------------------------------
// Message-passing litmus test of the acquire side (an isolated debug entry,
// "PCIe sync protocols" §7; the data-then-signal chain of §3). Workgroup 0
// (XCD 0) writes a 16 KB block with device-scope write-through stores, waits
// for their acknowledgement and stores round k into a flag; workgroup 1 (XCD 1)
// first reads the block with plain loads, so that its L1 and L2 hold the old
// contents, tells the writer, polls the flag, then reads the block again with
// the policy under test and counts the words that are not k.
//   MODE 0: device-scope loads (how the library reads signalled data);
//   MODE 1: plain loads (shows that the test sees the reader's caches);
//   MODE 2: plain loads after the formal agent-scope acquire fence.
// ---------------------------------------------------------------------------
constexpr int kLitmusVec = 16;                                // 16-byte vectors per lane
constexpr uint32_t kLitmusBytes = 64u * kLitmusVec * 16u;     // 16 KB block

template <int MODE>
__global__ __launch_bounds__(64, 1) void litmus_kernel(int* data, int* flag, int* ready,
                                                        unsigned long long* stale_out, int base, int rounds,
                                                        ErrorSink e, uint64_t timeout) {
  const int lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(data, kLitmusBytes);
  unsigned long long stale = 0;
  for (int i = 1; i <= rounds; ++i) {
    const int k = base + i;
    if (blockIdx.x == 1) {
#pragma unroll
      for (int u = 0; u < kLitmusVec; ++u) {
        const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(u * 64 + lane) * 16, 0, 0);
        asm volatile("" : : "v"(v));   // the old contents must really be loaded
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (lane == 0) __hip_atomic_store(ready, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int ok = 1;
      uint32_t polls = 0;
      if (lane == 0) ok = wait_ge(flag, k, now_ticks() + timeout, e, 0x71000001, &polls);
      if (!readlane(ok, 0)) break;
      if (MODE == 2) acquire_agent();
#pragma unroll
      for (int u = 0; u < kLitmusVec; ++u) {
        const v4i v = MODE == 0 ? __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(u * 64 + lane) * 16, 0, kPolSC1)
                                : __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(u * 64 + lane) * 16, 0, 0);
#pragma unroll
        for (int h = 0; h < 4; ++h) stale += (v[h] != k);
      }
    } else if (blockIdx.x == 0) {
      int ok = 1;
      uint32_t polls = 0;
      if (lane == 0) ok = wait_ge(ready, k, now_ticks() + timeout, e, 0x71000000, &polls);
      if (!readlane(ok, 0)) break;
      const v4i val = {k, k, k, k};
#pragma unroll
      for (int u = 0; u < kLitmusVec; ++u) store16_coherent(r, (uint32_t)(u * 64 + lane) * 16, val);
      release_coherent(false);
      if (lane == 0) slot_publish(flag, k, false);
    }
  }
  if (blockIdx.x == 1 && stale) atomicAdd(stale_out, stale);
}

// ---------------------------------------------------------------------------
// Protocol stress ("PCIe sync protocols" §3 validation scale, §4 chunked slots).
// Workgroups [0, P) are producers, [P, P + C) consumers. Slot id
// sid = (p * C + c) * KC + k. Producer waves split a chunk's rows 16 each and
// elect the last finisher as publisher; consumers wait slot by slot.
// ---------------------------------------------------------------------------
struct StressArgs {
  const int* chunk_rows;
  const int* delays_ns;
  int* payload;
  int* slot;
  int* elect_cur;
  int* elect_nxt;
  int* pub;
  unsigned long long* stats;
  ErrorSink err;
  int P, C, KC;
  int seq;
  uint32_t flags;
  uint64_t timeout_ticks;
  uint32_t payload_bytes;
  int64_t wall_khz;          // device wall-clock ticks per millisecond
};

__device__ __forceinline__ int stress_word(int seq, int sid, int r) {
  return (int)(((uint32_t)seq << 20) ^ (uint32_t)(sid * kChunk + r));
}

constexpr int kStressThreads = 256;   // four waves: a chunk's 64 rows are written 16 per wave

__global__ __launch_bounds__(kStressThreads, 1) void stress_kernel(StressArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool strict = a.flags & kStrict;
  const __amdgpu_buffer_rsrc_t rP = buffer_rsrc(a.payload, a.payload_bytes);
  if ((int)blockIdx.x < a.P) {
    const int p = blockIdx.x;
    for (int i = threadIdx.x; i < a.C * a.KC; i += kStressThreads) a.elect_nxt[p * a.C * a.KC + i] = 0;
    for (int c = 0; c < a.C; ++c) {
      for (int k = 0; k < a.KC; ++k) {
        const int sid = (p * a.C + c) * a.KC + k;
        const int n = a.chunk_rows[sid];
        if (n <= 0) continue;
        // producer delay, spun on the device wall clock at its queried rate
        const int d_ns = min(max(a.delays_ns[sid], 0), 10000000);   // clamp to [0, 10 ms]
        const uint64_t until = now_ticks() + (uint64_t)((long long)d_ns * a.wall_khz / 1000000);
        while (now_ticks() < until) __builtin_amdgcn_s_sleep(1);
        const int r = wave * 16 + lane;
        const int nw = max(0, min(16, n - wave * 16));
        if (lane < 16 && r < n) {
          const uint32_t off = (uint32_t)((((c * a.P + p) * a.KC + k) * kChunk + r) * 4);
          __builtin_amdgcn_raw_buffer_store_b32(stress_word(a.seq, sid, r), rP, off, 0, kPolCoherentStore);
        }
        release_coherent(strict);
        if (nw > 0 && lane == 0) {
          const int old = strict ? fetch_add_acq_rel(a.elect_cur + sid, nw) : fetch_add_relaxed(a.elect_cur + sid, nw);
          if (old + nw == n) {
            if (!((a.flags & kDropPublish) && sid == 0)) slot_publish(a.slot + sid, a.seq, strict);
            atomicAdd(a.pub + sid, 1);
          } else if (old + nw > n) {
            raise_error(a.err, kErrProtocol, 0x08000000 | sid);
          }
        }
      }
    }
  } else {
    const int c = blockIdx.x - a.P;
    uint32_t polls = 0;
    int stale = 0;
    for (int p = wave; p < a.P; p += 4) {
      for (int k = 0; k < a.KC; ++k) {
        const int sid = (p * a.C + c) * a.KC + k;
        const int n = a.chunk_rows[sid];
        if (n <= 0) continue;
        int ok = 1;
        if (lane == 0) ok = wait_ge(a.slot + sid, a.seq, now_ticks() + a.timeout_ticks, a.err, sid, &polls);
        ok = readlane(ok, 0);
        if (!ok) { p = a.P; break; }
        acquire_agent();
        if (lane < n) {
          const int v = a.payload[(((c * a.P + p) * a.KC + k) * kChunk) + lane];
          stale += (v != stress_word(a.seq, sid, lane));
        }
      }
    }
    if (stale) atomicAdd(a.stats + ST_STALE, (unsigned long long)stale);
    if (lane == 0 && polls) atomicAdd(a.stats + ST_SLOT_POLLS, (unsigned long long)polls);
  }
}

}  // namespace fg
