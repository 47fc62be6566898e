// Kernels of the fused producer/consumer gather-GEMM and of its protocol
// entry points (layout, fused persistent kernel, slot barrier, ping-pong,
// protocol stress). Included once, by fg.hip.
#pragma once

#include "fg_gemm.hpp"
#include "fg.h"

namespace fg {

constexpr int kChunk = FG_CHUNK_ROWS;
constexpr int kRB = FG_ROW_BLOCK;
constexpr int kThreads = 256;

// per-call flag bits as seen by the device
constexpr uint32_t kCommOnly = FG_CALL_COMM_ONLY;
constexpr uint32_t kGemmOnly = FG_CALL_GEMM_ONLY;
constexpr uint32_t kVerify = FG_CALL_VERIFY;
constexpr uint32_t kStrict = FG_CALL_STRICT;
constexpr uint32_t kDropPublish = FG_FAULT_DROP_PUBLISH;

// Device statistics block (int64 counters, cumulative).
enum { ST_PUBLISHES = 0, ST_GATE_POLLS, ST_SLOT_POLLS, ST_GATE_PASSES, ST_STALE, ST_COUNT };

struct FusedArgs {
  const uint16_t* shards[FG_MAX_SHARDS];
  const uint16_t* W;
  uint16_t* gathered;
  uint16_t* out;
  int K, N, n_shards, chunk_cap, rs_cap, rb_cap, m_pad_cap;
  int shard_rows;            // rows of every source shard (bounds of the row loads)
  int* slot;
  int* counter_cur;
  int* counter_nxt;
  int* elect_cur;
  int* elect_nxt;
  int* pub_count;
  const int* seed;
  const int* inv;
  const int* group_of_rb;
  const int* src_row;
  const int* stream_len;
  const int* desc;           // [0] = m_pad of this iteration
  unsigned long long* stats;
  long long* wgtime;         // [grid][4]: start, end, gate-wait ticks, tiles
  ErrorSink err;
  int seq;
  int n_comm, n_gemm;
  int rows_per_batch;
  uint32_t flags;
  uint64_t timeout_ticks;
};

// ---------------------------------------------------------------------------
// Communication role ("PCIe sync protocols" §3 election + publish, §4 chunk
// watermark, §5 arrival counters). Rows are walked in gathered-row order, the
// order in which the compute role consumes row blocks (§6 audit item 3); a
// communication workgroup never waits on anything (§6 audit item 2).
// ---------------------------------------------------------------------------
// Copy one batch of RB gathered rows (g0 .. g0+RB-1), each at most 64*UPR
// 16-byte vectors, branch-free: every row gets its own buffer descriptors, and
// a padding row (or the part of a row beyond K) gets a zero-sized one, so its
// loads read 0 and its stores are dropped by the buffer unit. All loads of the
// batch are issued before its stores (RB*UPR vectors per lane in flight).
template <int UPR, int RB>
__device__ __forceinline__ void copy_batch(const FusedArgs& a, const uint16_t* const* sh_shard, int g0, int info,
                                           int srow, uint32_t row_bytes, int lane) {
  __amdgpu_buffer_rsrc_t rs[RB], rd[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int rinfo = readlane(info, r);
    const bool valid = rinfo >= 0;
    const int s = valid ? (rinfo >> 24) : 0;
    const int sr = readlane(srow, r);
    const uint64_t base = (uint64_t)sh_shard[s];
    const uint16_t* shard = (const uint16_t*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                                              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base));
    rs[r] = buffer_rsrc(shard + (size_t)sr * a.K, valid ? row_bytes : 0u);
    rd[r] = buffer_rsrc(a.gathered + (size_t)(g0 + r) * a.K, valid ? row_bytes : 0u);
  }
  v4i v[RB][UPR];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int u = 0; u < UPR; ++u)
      v[r][u] = __builtin_amdgcn_raw_buffer_load_b128(rs[r], (uint32_t)(u * 64 + lane) * 16, 0, kPolNT);
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int u = 0; u < UPR; ++u)
      store16_coherent(rd[r], (uint32_t)(u * 64 + lane) * 16, v[r][u]);
}

__device__ void comm_role(const FusedArgs& a, const uint16_t* const* sh_shard) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = blockIdx.x;
  const bool strict = a.flags & kStrict;

  // Re-arm the other parity for the next iteration: nothing else touches it
  // during this kernel, and stream order publishes it to the next one.
  for (int i = cw * kThreads + threadIdx.x; i < a.rb_cap; i += a.n_comm * kThreads)
    a.counter_nxt[i] = a.seed[i];
  for (int i = cw * kThreads + threadIdx.x; i < a.n_shards * a.chunk_cap; i += a.n_comm * kThreads)
    a.elect_nxt[i] = 0;
  if (a.flags & kGemmOnly) return;

  const int m_pad = __builtin_amdgcn_readfirstlane(a.desc[0]);
  const int RB = a.rows_per_batch;
  const int n_batches = m_pad / RB;
  const int upr = (a.K / 8 + 63) / 64;       // 64-lane units of 16 bytes per row
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const int nw = a.n_comm * 4;
  const bool verify = a.flags & kVerify;

  for (int b = cw * 4 + wave; b < n_batches; b += nw) {
    const int g0 = b * RB;
    // lane r < RB describes gathered row g0 + r
    int info = -1, srow = 0;
    if (lane < RB) {
      info = a.inv[g0 + lane];
      if (info >= 0) srow = a.src_row[(info >> 24) * a.rs_cap + (info & 0xFFFFFF)];
    }
    // bitwise row copy: 16-byte streaming loads, device-coherent 16-byte stores
    if (upr <= 1)       copy_batch<1, 16>(a, sh_shard, g0, info, srow, row_bytes, lane);
    else if (upr <= 2)  copy_batch<2, 16>(a, sh_shard, g0, info, srow, row_bytes, lane);
    else if (upr <= 4)  copy_batch<4, 8>(a, sh_shard, g0, info, srow, row_bytes, lane);
    else if (upr <= 8)  copy_batch<8, 4>(a, sh_shard, g0, info, srow, row_bytes, lane);
    else if (upr <= 16) copy_batch<16, 2>(a, sh_shard, g0, info, srow, row_bytes, lane);
    else                copy_batch<32, 1>(a, sh_shard, g0, info, srow, row_bytes, lane);
    release_coherent(strict);
    // arrival count for the batch's row block (RB divides the row block)
    const uint64_t real = ballot(lane < RB && info >= 0);
    const int n_real = __popcll(real);
    if (lane == 0 && n_real > 0) {
      const int rb = g0 / kRB;
      const int old = fetch_add_relaxed(a.counter_cur + rb, n_real);
      if (old + n_real > kRB) raise_error(a.err, kErrProtocol, rb);
    }
    // election: per chunk touched by the batch, one add of the rows it finished;
    // the add that completes the chunk elects this wave as its single publisher
    const int chunk = (lane < RB && info >= 0) ? (info >> 24) * a.chunk_cap + ((info & 0xFFFFFF) / kChunk) : -1;
    uint64_t pending = ballot(chunk >= 0);
    while (pending) {
      const int leader = __ffsll((long long)pending) - 1;
      const int ch = readlane(chunk, leader);
      const uint64_t mask = ballot(chunk == ch) & pending;
      if (lane == leader) {
        const int cnt = __popcll(mask);
        const int old = strict ? fetch_add_acq_rel(a.elect_cur + ch, cnt) : fetch_add_relaxed(a.elect_cur + ch, cnt);
        const int s = ch / a.chunk_cap, c = ch - s * a.chunk_cap;
        const int expect = min(kChunk, a.stream_len[s] - kChunk * c);
        if (old + cnt == expect) {
          if (!((a.flags & kDropPublish) && ch == 0)) slot_publish(a.slot + ch, a.seq, strict);
          if (verify) {
            atomicAdd(a.pub_count + ch, 1);
            atomicAdd(a.stats + ST_PUBLISHES, 1ull);
          }
        } else if (old + cnt > expect) {
          raise_error(a.err, kErrProtocol, 0x10000000 | ch);
        }
      }
      pending &= ~mask;
    }
  }
}

// ---------------------------------------------------------------------------
// Compute role: for each tile in row-block-major order, wait until every row
// block it reads has counter == 128 ("PCIe sync protocols" §5 gate), acquire,
// run the MFMA tile.
// ---------------------------------------------------------------------------
template <int BM, int BN>
__device__ void gemm_role(const FusedArgs& a, char* lds0, char* lds1, int* sh_flag, long long* gate_ticks,
                          int* tiles_done) {
  const int gj = blockIdx.x - a.n_comm;
  if (a.flags & kCommOnly) return;
  const int m_pad = __builtin_amdgcn_readfirstlane(a.desc[0]);
  const int n_tn = a.N / BN;
  const int n_tiles = (m_pad / BM) * n_tn;
  const bool verify = a.flags & kVerify;
  const bool skip_gate = false;
  const uint32_t row_bytes = (uint32_t)a.K * 2;
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(a.gathered, (uint32_t)m_pad * row_bytes);
  const __amdgpu_buffer_rsrc_t rO = buffer_rsrc(a.out, (uint32_t)m_pad * (uint32_t)a.N * 2);
  for (int tile = gj; tile < n_tiles; tile += a.n_gemm) {
    const int mt = tile / n_tn, nt = tile - mt * n_tn;
    const int m0 = mt * BM, n0 = nt * BN;
    if (threadIdx.x == 0) {
      int ok = 1;
      if (!skip_gate) {
        const long long t0 = (long long)now_ticks();
        uint32_t polls = 0;
        for (int rb = m0 / kRB; rb < (m0 + BM) / kRB && ok; ++rb)
          ok = wait_eq(a.counter_cur + rb, kRB, now_ticks() + a.timeout_ticks, a.err, rb, &polls);
        *gate_ticks += (long long)now_ticks() - t0;
        if (verify) {
          atomicAdd(a.stats + ST_GATE_POLLS, (unsigned long long)polls);
          if (ok) atomicAdd(a.stats + ST_GATE_PASSES, 1ull);
        }
      }
      *sh_flag = ok;
    }
    __syncthreads();
    if (!*sh_flag) break;
    acquire_agent();
    const int g = __builtin_amdgcn_readfirstlane(a.group_of_rb[m0 / kRB]);
    const __amdgpu_buffer_rsrc_t rB =
        buffer_rsrc(a.W + (size_t)g * a.N * a.K, (uint32_t)a.N * row_bytes);
    Acc<BM, BN> acc;
#pragma unroll
    for (int i = 0; i < Tile<BM, BN>::FM; ++i)
#pragma unroll
      for (int j = 0; j < Tile<BM, BN>::FN; ++j) acc.v[i][j] = f32x16{};
    tile_mainloop<BM, BN>(rA, (uint32_t)m0 * row_bytes, rB, (uint32_t)n0 * row_bytes, a.K, lds0, lds1, acc);
    tile_store<BM, BN>(rO, a.N, m0, n0, acc, a.inv);
    if (threadIdx.x == 0) ++*tiles_done;
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void fused_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) char lds0[Tile<BM, BN>::STAGE];
  __shared__ __attribute__((aligned(16))) char lds1[Tile<BM, BN>::STAGE];
  __shared__ const uint16_t* sh_shard[FG_MAX_SHARDS];
  __shared__ int sh_flag;
  long long t_start = (long long)now_ticks();
  long long gate_ticks = 0;
  int tiles = 0;
  if (blockIdx.x < a.n_comm) {
    if (threadIdx.x < a.n_shards) sh_shard[threadIdx.x] = a.shards[threadIdx.x];
    __syncthreads();
    comm_role(a, sh_shard);
  } else {
    gemm_role<BM, BN>(a, lds0, lds1, &sh_flag, &gate_ticks, &tiles);
  }
  if (threadIdx.x == 0) {
    long long* t = a.wgtime + (size_t)blockIdx.x * 4;
    t[0] = t_start;
    t[1] = (long long)now_ticks();
    t[2] = gate_ticks;
    t[3] = tiles;
  }
}

// ---------------------------------------------------------------------------
// Layout step (step a1). Single workgroup of 1024 threads; phases separated by
// workgroup barriers. Writes the route tables, the inverse map, the padding
// seeds and arms the current parity (counters = seed, election counts = 0).
// ---------------------------------------------------------------------------
struct RouteArgs {
  int mode;                  // FG_ROUTE_*
  int n_shards, rs_cap, chunk_cap, rb_cap, m_pad_cap;
  int rows_per_shard;        // CONTIG / TOPK
  int m_pad;                 // CONTIG / EXPLICIT
  int n_groups;
  int group_off[FG_MAX_GROUPS + 1];   // EXPLICIT (host-given)
  int stream_len_in[FG_MAX_SHARDS];   // EXPLICIT (host-given)
  const int* src_in;         // EXPLICIT device
  const int* dst_in;
  const int* topk;           // TOPK device [S][T][KK]
  int topk_k, expert_base;
  int* src_row;
  int* dst_row;
  int* stream_len;
  int* group_off_out;
  int* inv;
  int* seed;
  int* group_of_rb;
  int* rbcount;
  int* counter_cur;
  int* elect_cur;
  int* desc;
  ErrorSink err;
};

constexpr int kRouteThreads = 1024;

__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  // sh: >= 32 ints of LDS scratch (16 waves)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kRouteThreads / 64; ++w) { const int t = sh[w]; sh[w] = run; run += t; }
    sh[16] = run;
  }
  __syncthreads();
  const int r = sh[wave] + x - v;
  *total = sh[16];
  __syncthreads();
  return r;
}

__device__ void route_finish(const RouteArgs& a, int m_pad, const int* goff, int n_groups) {
  // seeds, group of each row block, arming of the current parity
  const int n_rb = m_pad / kRB;
  for (int rb = threadIdx.x; rb < a.rb_cap; rb += kRouteThreads) {
    int sd = 0, g = 0;
    if (rb < n_rb) {
      sd = kRB - __hip_atomic_load(a.rbcount + rb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int j = 0; j < n_groups; ++j)
        if (rb * kRB >= goff[j] && rb * kRB < goff[j + 1]) g = j;
    }
    a.seed[rb] = sd;
    a.group_of_rb[rb] = g;
    a.counter_cur[rb] = sd;
  }
  for (int i = threadIdx.x; i < a.n_shards * a.chunk_cap; i += kRouteThreads) a.elect_cur[i] = 0;
  if (threadIdx.x <= n_groups) a.group_off_out[threadIdx.x] = goff[threadIdx.x];
  if (threadIdx.x == 0) a.desc[0] = m_pad;
}

__device__ __forceinline__ bool is_local(int e, int E) { return e >= 0 && e < E; }

__global__ __launch_bounds__(kRouteThreads, 1) void route_kernel(RouteArgs a) {
  __shared__ int sh[64];
  __shared__ int sh_goff[FG_MAX_GROUPS + 1];
  __shared__ int sh_ne[FG_MAX_GROUPS];
  __shared__ int sh_shard_base[FG_MAX_SHARDS + 1];
  __shared__ int sh_fail;
  const int tid = threadIdx.x;
  if (tid == 0) sh_fail = 0;
  for (int g = tid; g < a.m_pad_cap; g += kRouteThreads) a.inv[g] = -1;
  for (int rb = tid; rb < a.rb_cap; rb += kRouteThreads) a.rbcount[rb] = 0;
  if (a.mode == FG_ROUTE_CONTIG || a.mode == FG_ROUTE_EXPLICIT) {
    const int m_pad = a.m_pad;
    if (tid <= a.n_groups) sh_goff[tid] = (a.mode == FG_ROUTE_CONTIG) ? (tid == 0 ? 0 : m_pad) : a.group_off[tid];
    __syncthreads();
    for (int s = 0; s < a.n_shards; ++s) {
      const int n = (a.mode == FG_ROUTE_CONTIG) ? a.rows_per_shard : a.stream_len_in[s];
      if (tid == 0) a.stream_len[s] = n;
      for (int i = tid; i < n; i += kRouteThreads) {
        int src, dst;
        if (a.mode == FG_ROUTE_CONTIG) { src = i; dst = s * a.rows_per_shard + i; }
        else { src = a.src_in[s * a.rs_cap + i]; dst = a.dst_in[s * a.rs_cap + i]; }
        if (dst < 0 || dst >= m_pad || src < 0 || src >= a.rows_per_shard) {
          raise_error(a.err, kErrProtocol, 0x20000000 | s);
          sh_fail = 1;
          continue;
        }
        a.src_row[s * a.rs_cap + i] = src;
        a.dst_row[s * a.rs_cap + i] = dst;
        const int old = atomicExch(a.inv + dst, (s << 24) | i);
        if (old != -1) { raise_error(a.err, kErrProtocol, 0x30000000 | dst); sh_fail = 1; }
        atomicAdd(a.rbcount + dst / kRB, 1);
      }
    }
    __syncthreads();
    route_finish(a, sh_fail ? 0 : m_pad, sh_goff, a.n_groups);
    return;
  }
  // ---- TOPK: expert-dispatch layout. Token g = s*T + t is handled by thread
  // g / per; each thread walks its tokens in order, so every count below is an
  // exclusive prefix in global token order.
  const int S = a.n_shards, T = a.rows_per_shard, KK = a.topk_k, E = a.n_groups;
  const int G = S * T;
  const int per = (G + kRouteThreads - 1) / kRouteThreads;
  const int g_lo = min(G, tid * per), g_hi = min(G, g_lo + per);
  int picks = 0;
  for (int g = g_lo; g < g_hi; ++g)
    for (int k = 0; k < KK; ++k) picks += is_local(a.topk[(size_t)g * KK + k] - a.expert_base, E);
  int total_pairs;
  const int pick_base = block_exclusive_scan(picks, sh, &total_pairs);
  {
    int run = pick_base;
    for (int g = g_lo; g < g_hi; ++g) {
      if (g % T == 0) sh_shard_base[g / T] = run;
      for (int k = 0; k < KK; ++k) run += is_local(a.topk[(size_t)g * KK + k] - a.expert_base, E);
    }
    if (tid == 0) sh_shard_base[S] = total_pairs;
  }
  __syncthreads();
  if (tid < S) {
    const int n = sh_shard_base[tid + 1] - sh_shard_base[tid];
    a.stream_len[tid] = n;
    if (n > a.rs_cap) { raise_error(a.err, kErrProtocol, 0x40000000 | tid); sh_fail = 1; }
  }
  if (tid == 0) sh_goff[0] = 0;
  __syncthreads();
  const bool cap_fail = sh_fail;
  int off = 0;
  for (int e = 0; e < E; ++e) {
    int c = 0;
    for (int g = g_lo; g < g_hi; ++g)
      for (int k = 0; k < KK; ++k) c += (a.topk[(size_t)g * KK + k] - a.expert_base == e);
    int n_e;
    int rank = block_exclusive_scan(c, sh, &n_e);
    const int seg = ((n_e + kRB - 1) / kRB) * kRB;
    const bool overflow = off + seg > a.m_pad_cap;   // uniform across the block
    if (overflow && tid == 0) raise_error(a.err, kErrProtocol, 0x50000000 | e);
    if (!overflow && !cap_fail) {
      int run_pick = pick_base;   // stream index (global) of the next local pair
      for (int g = g_lo; g < g_hi; ++g) {
        const int s = g / T, t = g - s * T;
        for (int k = 0; k < KK; ++k) {
          const int ek = a.topk[(size_t)g * KK + k] - a.expert_base;
          if (!is_local(ek, E)) continue;
          if (ek == e) {
            const int i = run_pick - sh_shard_base[s];
            const int dst = off + rank;
            ++rank;
            a.src_row[s * a.rs_cap + i] = t;
            a.dst_row[s * a.rs_cap + i] = dst;
            a.inv[dst] = (s << 24) | i;
          }
          ++run_pick;
        }
      }
    }
    if (tid == 0) { sh_ne[e] = n_e; sh_goff[e + 1] = off + seg; }
    off += seg;
    if (overflow) { if (tid == 0) sh_fail = 1; break; }
  }
  __syncthreads();
  const int m_pad = sh_fail ? 0 : off;
  // real rows per row block: expert j's n_j real rows open its segment
  for (int rb = tid; rb < m_pad / kRB; rb += kRouteThreads) {
    int real = 0;
    for (int j = 0; j < E; ++j)
      if (rb * kRB >= sh_goff[j] && rb * kRB < sh_goff[j + 1])
        real = min(kRB, max(0, sh_ne[j] - (rb * kRB - sh_goff[j])));
    a.rbcount[rb] = real;
  }
  __syncthreads();
  route_finish(a, m_pad, sh_goff, E);
}

// Small helpers: fill, poke (fault injection on a counter).
__global__ void fill_kernel(int* p, int n, int v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
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

// Slot ping-pong between workgroup 0 and workgroup 1 (different XCDs).
template <int SYS>
__global__ __launch_bounds__(64, 1) void pingpong_kernel(int* a_slot, int* b_slot, int base, int rounds, ErrorSink e,
                                                         uint64_t timeout, long long* t_out) {
  if (threadIdx.x != 0) return;
  const long long t0 = (long long)now_ticks();
  uint32_t polls = 0;
  for (int r = 1; r <= rounds; ++r) {
    const int seq = base + r;
    if (blockIdx.x == 0) {
      if (SYS) __hip_atomic_store(a_slot, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else __hip_atomic_store(a_slot, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t dl = now_ticks() + timeout;
      int lvl = 0;
      while ((SYS ? __hip_atomic_load(b_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : poll_relaxed(b_slot)) < seq) {
        if (now_ticks() > dl) { raise_error(e, kErrTimeout, 0x70000000); return; }
        (void)lvl;
      }
    } else {
      const uint64_t dl = now_ticks() + timeout;
      while ((SYS ? __hip_atomic_load(a_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : poll_relaxed(a_slot)) < seq) {
        if (now_ticks() > dl) { raise_error(e, kErrTimeout, 0x70000001); return; }
      }
      if (SYS) __hip_atomic_store(b_slot, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else __hip_atomic_store(b_slot, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  (void)polls;
  if (blockIdx.x == 0) t_out[0] = (long long)now_ticks() - t0;
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
};

__device__ __forceinline__ int stress_word(int seq, int sid, int r) {
  return (int)(((uint32_t)seq << 20) ^ (uint32_t)(sid * kChunk + r));
}

__global__ __launch_bounds__(kThreads, 1) void stress_kernel(StressArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool strict = a.flags & kStrict;
  const __amdgpu_buffer_rsrc_t rP = buffer_rsrc(a.payload, a.payload_bytes);
  if ((int)blockIdx.x < a.P) {
    const int p = blockIdx.x;
    for (int i = threadIdx.x; i < a.C * a.KC; i += kThreads) a.elect_nxt[p * a.C * a.KC + i] = 0;
    for (int c = 0; c < a.C; ++c) {
      for (int k = 0; k < a.KC; ++k) {
        const int sid = (p * a.C + c) * a.KC + k;
        const int n = a.chunk_rows[sid];
        if (n <= 0) continue;
        // producer delay (bounded: at most the given nanoseconds, 100 MHz clock)
        const int d_ns = min(max(a.delays_ns[sid], 0), 10000000);   // clamp to [0, 10 ms]
        const uint64_t until = now_ticks() + (uint64_t)(d_ns / 10);
        while (now_ticks() < until) __builtin_amdgcn_s_sleep(1);
        const int r = wave * 16 + lane;
        const int nw = max(0, min(16, n - wave * 16));
        if (lane < 16 && r < n) {
          const uint32_t off = (uint32_t)((((c * a.P + p) * a.KC + k) * kChunk + r) * 4);
          __builtin_amdgcn_raw_buffer_store_b32(stress_word(a.seq, sid, r), rP, off, 0, kPolCoherentStream);
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
