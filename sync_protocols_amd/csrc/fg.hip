// Host implementation of the fg C ABI (include/fg.h) for gfx950.
//
// The context owns only the control plane ("NVLink atomic publish" §3.1: control
// separate from data, each array on its own 256-byte boundary): slots, the two
// parities of arrival counters and election counts, publisher counts, route
// tables, barrier slots, statistics, and one host-visible status word. All data
// buffers (shards, weights, gathered rows, outputs, routes) belong to the caller.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>

#include "fg_combine.hpp"

using namespace fg;

namespace {

// Copy workgroups: the gather is latency-bound per workgroup (load, write-through
// store, acknowledgement, counter add), so many workgroups keep enough bytes in
// flight; they join the compute role when their rows are copied.
constexpr int kDefaultSplitParts = 8;
constexpr int64_t kDefaultTimeoutNs = 2000000000LL;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Plane {
  int* slot;
  int* counter;    // [2][rb_cap][kCtr]
  int* elect;      // [2][S * chunk_cap]
  int* pub_count;
  int* seed;
  unsigned long long* inv;   // versioned inverse map
  int* src_of;     // [m_pad_cap] source row of each gathered row
  int* group_of_rb;
  int* src_row;
  int* dst_row;
  int* stream_len;
  int* group_off;
  int* rbcount;
  int* wgcount;
  int* wgbase;
  int* ticket;
  int* gtick;      // [2] x kTickInts: compute-item tickets (global + one per XCD), one set per parity
  int* skc;        // [2][split_slots] split-K part counters
  long long* trace;    // [trace_cap][4]
  long long* rb_time;  // [rb_cap]
  int* desc;       // [0] m_pad, [1] row slabs
  int* slab;       // [rb_cap] row slab table
  int* gslab;      // [FG_MAX_GROUPS + 1] first slab of each group
  int* err;        // [2]
  unsigned long long* stats;
  int* bslot;
  int* pp;         // ping-pong slots (two, 256 bytes apart)
  long long* tdev; // [4] barrier / ping-pong timings
  long long* wgtime;
  int* s_slot;
  int* s_elect;    // [2][P*C*KC]
  int* s_pub;
  int* src_k;      // [S][rs_cap] TOPK: top-k position of each stream entry
  int* tok_first;  // [S][rs_cap + 1] TOPK: first stream entry of each token
  int* cslot;      // combine plane: slots, election counts x2, publisher counts
  int* celect;
  int* cpub;
  int* litmus;     // message-passing litmus test: 16 KB block, flag, ready, stale count
  unsigned long long* rtail;   // [2][ring_cap][kRingTailStride] FIFO ring tails (finish << 32 | tail)
  int* rhead;                  // [2][ring_cap][kCtr] FIFO ring heads
};

}  // namespace

struct fg_ctx {
  fg_config cfg;
  int device = 0;
  int cu_count = 0;
  int chunk_cap = 0, rb_cap = 0, m_pad_cap = 0, s_slots = 0;
  int n_comm = 0, n_gemm = 0, tile_n = 256;
  int split_parts = 1, split_tiles = 0, split_slots = 1, split_blocks = 0, trace_cap = 0;
  float* skws = nullptr;       // split-K partial sums
  size_t skws_bytes = 0;
  int64_t wall_khz = 100000;
  char* plane_mem = nullptr;
  Plane p{};
  int* host_status = nullptr;
  int seq = 0, bseq = 0, sseq = 0, ppseq = 0, cseq = 0, lseq = 0;
  long long litmus_words = 0;
  int topk_rows = 0, topk_k = 0;   // tokens per shard and k of the last TOPK route
  int combine_wg = 0;
  int ring_cap = 0;            // rings the copy workgroups can serve (a producer and a consumer each)
  int route_resident = 0;      // layout workgroups that can be resident at once (one-kernel layout)
  uint32_t route_ver = 0;
  int route_wg_cap = 0;
  fg_status sticky = FG_OK;
  bool no_alloc = false;       // state of fg_gather_gemm_noalloc: the status word is the caller's device word
  bool stream_bound = false;
  hipStream_t stream = nullptr;
  // cached CONTIG route (so that repeated all-gathers skip the layout step)
  int route_cached_mode = -1;
  int route_cached_rows = -1;
  int last_grid = 0;
  int last_n_comm = 0;   // copy-role workgroups of the last fused kernel (all of them with the in-tile copy)
  int last_m_pad = 0;
  int last_tcopy = 0, last_lead_rows = 0;
  unsigned long long host_stats[ST_COUNT] = {};
};

#define HIPCHK(x)                                   \
  do {                                              \
    hipError_t e_ = (x);                            \
    if (e_ != hipSuccess) return FG_EHIP;           \
  } while (0)

// After a call has advanced a sequence number whose parity arms the control
// plane, a failed launch leaves that plane one parity behind: the context is
// then unusable and answers FG_ESTATE from the next call on.
#define HIPCHK_STICKY(ctx, x)                       \
  do {                                              \
    hipError_t e_ = (x);                            \
    if (e_ != hipSuccess) {                         \
      (ctx)->sticky = FG_EHIP;                      \
      return FG_EHIP;                               \
    }                                               \
  } while (0)

static int round_up(int x, int b) { return (x + b - 1) / b * b; }

static int m_pad_capacity(const fg_config& c) {
  const long long m = (long long)c.n_shards * c.max_rows_per_shard;
  long long cap = (long long)round_up((int)std::min<long long>(m, 1 << 30), FG_ROW_BLOCK);
  if (c.n_groups > 1) cap = round_up((int)(m + (long long)c.n_groups * (FG_ROW_BLOCK - 1)), FG_ROW_BLOCK);
  return (int)cap;
}

// Row data moves in 16-byte vectors (buffer loads and stores of four dwords,
// global -> LDS loads of 16 bytes per lane), so every row buffer must start on
// a 16-byte boundary; rows are K * 2 or N * 2 bytes apart, multiples of 256.
static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static bool config_ok(const fg_config* c) {
  if (!c) return false;
  if (c->n_shards < 1 || c->n_shards > FG_MAX_SHARDS) return false;
  if (c->max_rows_per_shard < 1 || c->max_rows_per_shard > (1 << 24) - 1) return false;
  if (c->K < 128 || c->K % 128 != 0 || c->K > 16384) return false;
  if (c->N < 128 || c->N % 128 != 0) return false;
  if (c->n_groups < 1 || c->n_groups > FG_MAX_GROUPS) return false;
  if (c->tile_n != 0 && c->tile_n != 128 && c->tile_n != 256) return false;
  if (c->tile_n == 256 && c->N % 256 != 0) return false;
  if (c->n_comm_wg < 0 || c->n_gemm_wg < 0) return false;
  if (c->timeout_ns < 0) return false;
  if (c->split_parts < 0 || c->split_parts > 8 || c->split_tiles < 0 || c->split_tiles > 4096) return false;
  if (c->tile_order < 0 || c->tile_order > 1) return false;
  if (c->copy_rows != 0 && c->copy_rows != 1 && c->copy_rows != 2 && c->copy_rows != 4 && c->copy_rows != 8 &&
      c->copy_rows != 16) return false;
  if (c->combine_wg < 0 || c->combine_wg > 65536) return false;
  if (c->copy_mode < 0 || c->copy_mode > 1) return false;
  if (c->stress_producers < 0 || c->stress_consumers < 0 || c->stress_max_chunks < 0) return false;
  const long long m = (long long)c->n_shards * c->max_rows_per_shard + (long long)c->n_groups * FG_ROW_BLOCK;
  if (m * c->K * 2 >= (1ll << 32)) return false;   // 32-bit buffer offsets
  if (m * c->N * 2 >= (1ll << 32)) return false;
  if ((long long)c->N * c->K * 2 >= (1ll << 32)) return false;
  return true;
}

template <int BN>
static hipError_t occupancy(int* per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, fused_kernel<BN>, kThreads, 0);
}

static fg_status map_device_error(int code) {
  if (code == kErrTimeout) return FG_ETIMEOUT;
  if (code == kErrProtocol) return FG_EPROTOCOL;
  return code ? FG_EPROTOCOL : FG_OK;
}

// A device-side error recorded by an earlier launch becomes sticky here.
static fg_status check_sticky(fg_ctx* ctx) {
  if (ctx->sticky != FG_OK) return FG_ESTATE;
  if (ctx->no_alloc) return FG_OK;   // device-side errors go to the caller's status word
  const int code = __atomic_load_n(ctx->host_status, __ATOMIC_ACQUIRE);
  if (code != 0) {
    ctx->sticky = map_device_error(code);
    return ctx->sticky;
  }
  return FG_OK;
}

static fg_status bind_stream(fg_ctx* ctx, hipStream_t s) {
  if (!ctx->stream_bound) {
    ctx->stream = s;
    ctx->stream_bound = true;
    return FG_OK;
  }
  return ctx->stream == s ? FG_OK : FG_EINVAL;
}

static ErrorSink sink(fg_ctx* ctx) { return ErrorSink{ctx->p.err, ctx->host_status}; }

static uint64_t timeout_ticks(const fg_ctx* ctx) {
  const int64_t ns = ctx->cfg.timeout_ns ? ctx->cfg.timeout_ns : kDefaultTimeoutNs;
  return (uint64_t)(ns / 1000000.0 * ctx->wall_khz);
}

static fg_status launch_route(fg_ctx* ctx, const fg_route* route, int mode, int rows, int m_pad, hipStream_t st,
                              uint32_t flags) {
  RouteArgs ra{};
  const fg_config& c = ctx->cfg;
  ra.mode = mode;
  ra.n_shards = c.n_shards; ra.rs_cap = c.max_rows_per_shard; ra.chunk_cap = ctx->chunk_cap;
  ra.rb_cap = ctx->rb_cap; ra.m_pad_cap = ctx->m_pad_cap;
  ra.rows_per_shard = rows; ra.m_pad = m_pad;
  ra.n_groups = (mode == FG_ROUTE_CONTIG) ? 1 : c.n_groups;
  if (mode == FG_ROUTE_EXPLICIT) {
    for (int s = 0; s < c.n_shards; ++s) ra.stream_len_in[s] = route->stream_len[s];
    if (route->group_off) {
      for (int g = 0; g <= c.n_groups; ++g) ra.group_off[g] = route->group_off[g];
    } else {
      ra.n_groups = 1; ra.group_off[0] = 0; ra.group_off[1] = m_pad;
    }
    ra.src_in = route->src_row; ra.dst_in = route->dst_row;
  }
  if (mode == FG_ROUTE_TOPK) {
    ra.topk = route->topk; ra.topk_k = route->topk_k; ra.expert_base = route->expert_base;
    ctx->topk_rows = rows; ctx->topk_k = route->topk_k;
  }
  ra.src_k = ctx->p.src_k; ra.tok_first = ctx->p.tok_first;
  const int cur = ctx->seq & 1;
  ctx->route_ver += 1;
  ra.ver = ctx->route_ver;
  ra.src_row = ctx->p.src_row; ra.dst_row = ctx->p.dst_row; ra.stream_len = ctx->p.stream_len;
  ra.group_off_out = ctx->p.group_off; ra.inv = ctx->p.inv; ra.src_of = ctx->p.src_of; ra.seed = ctx->p.seed;
  ra.group_of_rb = ctx->p.group_of_rb; ra.rbcount = ctx->p.rbcount;
  ra.wgcount = ctx->p.wgcount; ra.wgbase = ctx->p.wgbase; ra.ticket = ctx->p.ticket;
  ra.counter_cur = ctx->p.counter + (size_t)cur * ctx->rb_cap * kCtr;
  ra.elect_cur = ctx->p.elect + (size_t)cur * c.n_shards * ctx->chunk_cap;
  ra.desc = ctx->p.desc; ra.slab = ctx->p.slab; ra.gslab = ctx->p.gslab; ra.err = sink(ctx);
  auto blocks = [](long long work) { return (int)std::max(1LL, std::min(1024LL, (work + kRouteThreads - 1) / kRouteThreads)); };
  if (mode == FG_ROUTE_CONTIG) {
    const long long work = std::max<long long>({(long long)c.n_shards * rows, ctx->rb_cap,
                                                (long long)c.n_shards * ctx->chunk_cap});
    hipLaunchKernelGGL(route_contig_kernel, dim3(blocks(work)), dim3(kRouteThreads), 0, st, ra);
  } else if (mode == FG_ROUTE_EXPLICIT) {
    hipLaunchKernelGGL(route_explicit_kernel, dim3(blocks((long long)c.n_shards * c.max_rows_per_shard)),
                       dim3(kRouteThreads), 0, st, ra);
  } else {
    ra.wpb = (rows + kRouteThreads - 1) / kRouteThreads;
    const int n_wg = c.n_shards * ra.wpb;
    ra.n_wg = n_wg;
    ra.timeout_ticks = timeout_ticks(ctx);
    if (n_wg <= ctx->route_resident && !(flags & FG_CALL_LAYOUT_TWO_PASS)) {
      // one kernel: the layout grid is co-resident, so its workgroups can wait for the scan
      hipLaunchKernelGGL(route_topk_kernel, dim3(n_wg), dim3(kRouteThreads), 0, st, ra);
    } else {
      hipLaunchKernelGGL(route_topk_count_kernel, dim3(n_wg), dim3(kRouteThreads), 0, st, ra);
      HIPCHK(hipGetLastError());
      hipLaunchKernelGGL(route_topk_place_kernel, dim3(n_wg), dim3(kRouteThreads), 0, st, ra);
    }
  }
  HIPCHK(hipGetLastError());
  return FG_OK;
}

template <int BN>
static fg_status launch_fused(const FusedArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((fused_kernel<BN>), dim3(a.n_comm + a.n_gemm), dim3(kThreads), 0, st, a);
  HIPCHK(hipGetLastError());
  return FG_OK;
}

// Scratch of fg_gather_gemm_noalloc: the control plane of one call (slots,
// arrival counters and election counts of both parities, route tables,
// tickets, statistics); 4 MiB covers 8 shards x 4096 rows at K = N = 8192.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kNoAllocMaxDevices = 64;
struct NoAllocDevice {
  bool ready = false;
  char* ptr = nullptr;   // device address of this GPU's copy of `scratch`
  fg_ctx ctx;            // sequence numbers, route version and the per-call sizes
};
NoAllocDevice g_noalloc[kNoAllocMaxDevices];
}  // namespace

// Context set-up shared by fg_init and the no-allocation entry point:
// device attributes, the grid split, the residency audit ("PCIe sync
// protocols" §6 items 1 and 2) and the derived capacities. no_alloc: no
// split-K workspace (split_parts 1) and no trace.
static fg_status ctx_setup(fg_ctx* ctx, const fg_config* cfg, int hip_device, bool no_alloc) {
  ctx->cfg = *cfg;
  ctx->device = hip_device;
  int wall = 0;
  if (hipDeviceGetAttribute(&ctx->cu_count, hipDeviceAttributeMultiprocessorCount, hip_device) != hipSuccess ||
      hipDeviceGetAttribute(&wall, hipDeviceAttributeWallClockRate, hip_device) != hipSuccess) {
    return FG_EHIP;
  }
  if (wall > 0) ctx->wall_khz = wall;
  // default: three quarters of the compute units copy first (192 of 256): the
  // copy is bandwidth-bound, and more copy workgroups bring the first row
  // blocks in sooner and join the compute role earlier (measured fused time on
  // TP / EP / Large: 243 / 311 / 3574 us at 128, 237 / 304 / 3553 us at 192)
  ctx->n_comm = cfg->n_comm_wg ? cfg->n_comm_wg : std::max(1, ctx->cu_count * 3 / 4);
  ctx->n_gemm = cfg->n_gemm_wg ? cfg->n_gemm_wg : ctx->cu_count - ctx->n_comm;
  ctx->tile_n = cfg->tile_n ? cfg->tile_n : (cfg->N % 256 == 0 ? 256 : 128);
  // "PCIe sync protocols" §6 audit: every spinning workgroup must leave room
  // for the suppliers, and the whole persistent grid must be resident at once.
  if (ctx->n_gemm < 1 || ctx->n_gemm >= ctx->cu_count || ctx->n_comm < 1) return FG_ERESIDENCY;
  {
    int per_cu = 0, worst = 1 << 30;
    hipError_t e = hipSuccess;
    e = ctx->tile_n == 256 ? occupancy<256>(&per_cu) : occupancy<128>(&per_cu);
    worst = std::min(worst, per_cu);
    if (e != hipSuccess) return FG_EHIP;
    if ((long long)worst * ctx->cu_count < ctx->n_comm + ctx->n_gemm) return FG_ERESIDENCY;
  }
  // combine kernel: its waves wait on pushes done by other waves, so the whole
  // grid must be resident (same audit)
  ctx->combine_wg = cfg->combine_wg ? cfg->combine_wg : 2 * ctx->cu_count;
  {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, combine_kernel, kCombThreads, 0) != hipSuccess) {
      return FG_EHIP;
    }
    if ((long long)per_cu * ctx->cu_count < ctx->combine_wg) return FG_ERESIDENCY;
  }
  {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, route_topk_kernel, kRouteThreads, 0) != hipSuccess) {
      return FG_EHIP;
    }
    ctx->route_resident = per_cu * ctx->cu_count;
  }
  if (cfg->stress_producers + cfg->stress_consumers > ctx->cu_count ||
      cfg->stress_consumers >= ctx->cu_count) return FG_ERESIDENCY;
  if (cfg->n_shards > ctx->cu_count) return FG_ERESIDENCY;

  const int S = cfg->n_shards;
  ctx->chunk_cap = (cfg->max_rows_per_shard + FG_CHUNK_ROWS - 1) / FG_CHUNK_ROWS;
  ctx->m_pad_cap = m_pad_capacity(*cfg);
  ctx->rb_cap = ctx->m_pad_cap / FG_ROW_BLOCK;
  ctx->s_slots = cfg->stress_producers * cfg->stress_consumers * cfg->stress_max_chunks;
  const int grid_max = ctx->n_comm + ctx->n_gemm;
  // split-K tail capacity: by default at most grid/2 split tiles and grid
  // partial blocks (P <= grid / split tiles); a given split_tiles adds
  // split_tiles tiles of split_parts blocks each
  ctx->split_parts = no_alloc ? 1 : cfg->split_parts ? cfg->split_parts : kDefaultSplitParts;
  ctx->split_tiles = ctx->split_parts > 1 ? cfg->split_tiles : 0;
  ctx->split_slots = std::max({1, grid_max / 2, ctx->split_tiles});
  ctx->split_blocks = ctx->split_parts > 1 ? std::max(grid_max, ctx->split_tiles * ctx->split_parts) : 0;
  ctx->skws_bytes = (size_t)ctx->split_blocks * 256 * ctx->tile_n * 4;
  // 32-bit buffer offsets; offsets from 0xFFFFFFF0 up read as zeros in the partial sums
  if (ctx->skws_bytes >= 0xFFFFFFF0ull) return FG_EINVAL;
  ctx->trace_cap = no_alloc ? 0 : (ctx->m_pad_cap / 128) * (cfg->N / 128) + ctx->split_blocks;
  return FG_OK;
}

// Offsets of the control-plane arrays, each on a 256-byte boundary ("NVLink
// atomic publish" §3.1); with a base address the context's pointers are set.
// Returns the plane's size in bytes.
static size_t plane_layout(fg_ctx* ctx, char* base) {
  const fg_config* cfg = &ctx->cfg;
  const int S = cfg->n_shards;
  const int grid_max = ctx->n_comm + ctx->n_gemm;
  const size_t nch = (size_t)S * ctx->chunk_cap;
  const size_t nrs = (size_t)S * cfg->max_rows_per_shard;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  ctx->route_wg_cap = S * ((cfg->max_rows_per_shard + kRouteThreads - 1) / kRouteThreads);
  const size_t wgc = (size_t)ctx->route_wg_cap * (FG_MAX_GROUPS + 1) * 4;
  const size_t o_slot = take(nch * 4), o_counter = take(2 * (size_t)ctx->rb_cap * kCtr * 4),
               o_elect = take(2 * nch * 4), o_pub = take(nch * 4), o_seed = take((size_t)ctx->rb_cap * 4),
               o_inv = take((size_t)ctx->m_pad_cap * 8), o_srcof = take((size_t)ctx->m_pad_cap * 4),
               o_grp = take((size_t)ctx->rb_cap * 4),
               o_src = take(nrs * 4), o_dst = take(nrs * 4), o_slen = take((size_t)S * 4),
               o_goff = take((FG_MAX_GROUPS + 1) * 4), o_rbc = take((size_t)ctx->rb_cap * kRbSlots * 4), o_desc = take(64), o_slab = take((size_t)ctx->rb_cap * 4), o_gslab = take((FG_MAX_GROUPS + 1) * 4),
               o_wgc = take(wgc), o_wgb = take(wgc), o_tick = take(64), o_gtick = take(2 * kTickInts * 4),
               o_skc = take(2 * (size_t)ctx->split_slots * 4),
               o_trace = take((size_t)ctx->trace_cap * kTraceFields * 8), o_rbt = take((size_t)ctx->rb_cap * 8),
               o_err = take(64), o_stats = take(ST_COUNT * 8), o_bslot = take((size_t)S * S * 4),
               o_pp = take(512), o_tdev = take(64), o_wg = take((size_t)grid_max * kWgTimeFields * 8),
               o_sslot = take((size_t)ctx->s_slots * 4), o_select = take(2 * (size_t)ctx->s_slots * 4),
               o_spub = take((size_t)ctx->s_slots * 4), o_srck = take(nrs * 4),
               o_tokf = take((size_t)S * (cfg->max_rows_per_shard + 1) * 4), o_cslot = take(nch * kCombStride * 4),
               o_celect = take(2 * nch * kCombStride * 4), o_cpub = take(nch * 4), o_lit = take(kLitmusBytes + 768);
  ctx->ring_cap = std::max(1, ctx->n_comm / 2);
  const size_t o_rtail = take(2 * (size_t)ctx->ring_cap * kRingTailStride * 8),
               o_rhead = take(2 * (size_t)ctx->ring_cap * kCtr * 4);
  if (!base) return off;
  char* b = base;
  Plane& p = ctx->p;
  p.slot = (int*)(b + o_slot); p.counter = (int*)(b + o_counter); p.elect = (int*)(b + o_elect);
  p.pub_count = (int*)(b + o_pub); p.seed = (int*)(b + o_seed); p.inv = (unsigned long long*)(b + o_inv);
  p.src_of = (int*)(b + o_srcof);
  p.wgcount = (int*)(b + o_wgc); p.wgbase = (int*)(b + o_wgb); p.ticket = (int*)(b + o_tick);
  p.gtick = (int*)(b + o_gtick); p.skc = (int*)(b + o_skc);
  p.trace = (long long*)(b + o_trace); p.rb_time = (long long*)(b + o_rbt);
  p.group_of_rb = (int*)(b + o_grp); p.src_row = (int*)(b + o_src); p.dst_row = (int*)(b + o_dst);
  p.stream_len = (int*)(b + o_slen); p.group_off = (int*)(b + o_goff); p.rbcount = (int*)(b + o_rbc);
  p.desc = (int*)(b + o_desc); p.slab = (int*)(b + o_slab); p.gslab = (int*)(b + o_gslab); p.err = (int*)(b + o_err); p.stats = (unsigned long long*)(b + o_stats);
  p.bslot = (int*)(b + o_bslot); p.pp = (int*)(b + o_pp); p.tdev = (long long*)(b + o_tdev);
  p.wgtime = (long long*)(b + o_wg); p.s_slot = (int*)(b + o_sslot); p.s_elect = (int*)(b + o_select);
  p.s_pub = (int*)(b + o_spub);
  p.src_k = (int*)(b + o_srck); p.tok_first = (int*)(b + o_tokf); p.cslot = (int*)(b + o_cslot);
  p.celect = (int*)(b + o_celect); p.cpub = (int*)(b + o_cpub); p.litmus = (int*)(b + o_lit);
  p.rtail = (unsigned long long*)(b + o_rtail); p.rhead = (int*)(b + o_rhead);
  return off;
}

extern "C" {

const char* fg_strerror(fg_status s) {
  switch (s) {
    case FG_OK: return "ok";
    case FG_EINVAL: return "invalid argument";
    case FG_ENOMEM: return "out of memory";
    case FG_EHIP: return "HIP runtime error";
    case FG_ERESIDENCY: return "persistent grid not co-resident";
    case FG_ETIMEOUT: return "device wait timed out";
    case FG_EPROTOCOL: return "protocol violation (counter overshoot or bad route)";
    case FG_ESTATE: return "context carries an earlier device-side error";
  }
  return "unknown";
}

fg_status fg_capacity(const fg_config* cfg, int32_t* m_pad_cap) {
  if (!config_ok(cfg) || !m_pad_cap) return FG_EINVAL;
  *m_pad_cap = m_pad_capacity(*cfg);
  return FG_OK;
}

fg_status fg_init(const fg_config* cfg, int hip_device, fg_ctx** out) {
  if (!out) return FG_EINVAL;
  *out = nullptr;
  if (!config_ok(cfg)) return FG_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || hip_device < 0 || hip_device >= ndev) return FG_EINVAL;
  HIPCHK(hipSetDevice(hip_device));
  fg_ctx* ctx = new (std::nothrow) fg_ctx();
  if (!ctx) return FG_ENOMEM;
  const fg_status st = ctx_setup(ctx, cfg, hip_device, false);
  if (st != FG_OK) { delete ctx; return st; }
  const size_t bytes = plane_layout(ctx, nullptr);
  if (hipMalloc(&ctx->plane_mem, bytes) != hipSuccess) { delete ctx; return FG_ENOMEM; }
  if (hipMemset(ctx->plane_mem, 0, bytes) != hipSuccess) { (void)hipFree(ctx->plane_mem); delete ctx; return FG_EHIP; }
  plane_layout(ctx, ctx->plane_mem);
  if (hipHostMalloc((void**)&ctx->host_status, 64, hipHostMallocCoherent) != hipSuccess) {
    (void)hipFree(ctx->plane_mem); delete ctx; return FG_ENOMEM;
  }
  memset(ctx->host_status, 0, 64);
  if (ctx->skws_bytes && hipMalloc(&ctx->skws, ctx->skws_bytes) != hipSuccess) {
    ctx->skws = nullptr;
    fg_destroy(ctx);
    return FG_ENOMEM;
  }
  if (hipDeviceSynchronize() != hipSuccess) { fg_destroy(ctx); return FG_EHIP; }
  *out = ctx;
  return FG_OK;
}

fg_status fg_destroy(fg_ctx* ctx) {
  if (!ctx) return FG_EINVAL;
  (void)hipSetDevice(ctx->device);
  if (ctx->stream_bound) (void)hipStreamSynchronize(ctx->stream);
  if (ctx->plane_mem) (void)hipFree(ctx->plane_mem);
  if (ctx->host_status) (void)hipHostFree(ctx->host_status);
  if (ctx->skws) (void)hipFree(ctx->skws);
  delete ctx;
  return FG_OK;
}

struct RingCall {
  void* ring = nullptr;
  int n_channels = 0, ring_chunks = 0;
};

static fg_status gather_gemm_launch(fg_ctx* ctx, const void* const* shards, const fg_route* route, const void* W,
                                    void* const* staging, int self_shard, void* gathered, void* out, uint32_t flags,
                                    hipStream_t stream, const RingCall& rc, int mode, int rows, int m_pad);

static fg_status gather_gemm_impl(fg_ctx* ctx, const void* const* shards, const fg_route* route, const void* W,
                                  void* const* staging, int self_shard, void* gathered, void* out, uint32_t flags,
                                  hipStream_t stream, const RingCall& rc = RingCall()) {
  if (!ctx) return FG_EINVAL;
  fg_status s = check_sticky(ctx);
  if (s != FG_OK) return s;
  const fg_config& c = ctx->cfg;
  if (!shards || !W || !gathered || !out) return FG_EINVAL;
  if (!al16(W) || !al16(gathered) || !al16(out) || !al16(rc.ring)) return FG_EINVAL;
  for (int i = 0; i < c.n_shards; ++i) if (!shards[i] || !al16(shards[i])) return FG_EINVAL;
  if (staging)
    for (int i = 0; i < c.n_shards; ++i) if (!al16(staging[i])) return FG_EINVAL;
  if ((flags & FG_CALL_COMM_ONLY) && (flags & FG_CALL_GEMM_ONLY)) return FG_EINVAL;
  const int mode = route ? route->mode : FG_ROUTE_CONTIG;
  // watermark gating needs the contiguous layout and the one-stage copy (whose slots cover the rows)
  if ((flags & FG_CALL_GATE_WATERMARK) && (mode != FG_ROUTE_CONTIG || staging || rc.ring)) return FG_EINVAL;
  int rows = c.max_rows_per_shard, m_pad = 0;
  if (mode == FG_ROUTE_CONTIG) {
    if (route) rows = route->rows_per_shard;
    if (rows < 1 || rows > c.max_rows_per_shard) return FG_EINVAL;
    m_pad = round_up(c.n_shards * rows, FG_ROW_BLOCK);
  } else if (mode == FG_ROUTE_EXPLICIT) {
    if (!route->stream_len || !route->src_row || !route->dst_row) return FG_EINVAL;
    rows = route->rows_per_shard;
    if (rows < 1) return FG_EINVAL;
    for (int i = 0; i < c.n_shards; ++i)
      if (route->stream_len[i] < 0 || route->stream_len[i] > c.max_rows_per_shard) return FG_EINVAL;
    m_pad = route->m_pad;
    if (m_pad < FG_ROW_BLOCK || m_pad % FG_ROW_BLOCK || m_pad > ctx->m_pad_cap) return FG_EINVAL;
    if (route->group_off) {
      if (route->group_off[0] != 0 || route->group_off[c.n_groups] != m_pad) return FG_EINVAL;
      for (int g = 0; g < c.n_groups; ++g)
        if (route->group_off[g + 1] < route->group_off[g] || route->group_off[g + 1] % FG_ROW_BLOCK) return FG_EINVAL;
    } else if (c.n_groups != 1) {
      return FG_EINVAL;
    }
  } else if (mode == FG_ROUTE_TOPK) {
    if (!route->topk || route->topk_k < 1 || route->topk_k > 64) return FG_EINVAL;
    rows = route->rows_per_shard;
    if (rows < 1 || rows > c.max_rows_per_shard) return FG_EINVAL;
    if (c.n_groups < 1) return FG_EINVAL;
  } else {
    return FG_EINVAL;
  }
  if (bind_stream(ctx, stream) != FG_OK) return FG_EINVAL;
  HIPCHK(hipSetDevice(ctx->device));
  s = gather_gemm_launch(ctx, shards, route, W, staging, self_shard, gathered, out, flags, stream, rc, mode, rows,
                         m_pad);
  // once seq has advanced the parity arming assumes this call's kernel ran:
  // a launch that failed leaves the control plane one parity behind, so the
  // context is unusable from here on
  if (s == FG_EHIP) ctx->sticky = FG_EHIP;
  return s;
}

static fg_status gather_gemm_launch(fg_ctx* ctx, const void* const* shards, const fg_route* route, const void* W,
                                    void* const* staging, int self_shard, void* gathered, void* out, uint32_t flags,
                                    hipStream_t stream, const RingCall& rc, int mode, int rows, int m_pad) {
  const fg_config& c = ctx->cfg;
  fg_status s = FG_OK;
  ctx->seq += 1;
  const int cur = ctx->seq & 1, nxt = cur ^ 1;
  const bool same = flags & FG_CALL_SAME_ROUTE;
  if (mode == FG_ROUTE_CONTIG) {
    if (ctx->route_cached_mode != FG_ROUTE_CONTIG || ctx->route_cached_rows != rows) {
      if ((s = launch_route(ctx, route, mode, rows, m_pad, stream, flags)) != FG_OK) return s;
      ctx->route_cached_mode = FG_ROUTE_CONTIG;
      ctx->route_cached_rows = rows;
    }
  } else {
    if (!same || ctx->route_cached_mode != mode) {
      if ((s = launch_route(ctx, route, mode, rows, m_pad, stream, flags)) != FG_OK) return s;
    }
    ctx->route_cached_mode = mode;
    ctx->route_cached_rows = rows;
  }
  int* counter_cur = ctx->p.counter + (size_t)cur * ctx->rb_cap * kCtr;
  if (flags & (FG_FAULT_SEED_LOW | FG_FAULT_SEED_HIGH)) {
    hipLaunchKernelGGL(poke_kernel, dim3(1), dim3(64), 0, stream, counter_cur, (flags & FG_FAULT_SEED_HIGH) ? 1 : -1);
    HIPCHK(hipGetLastError());
  }
  if (flags & FG_CALL_GEMM_ONLY) {
    hipLaunchKernelGGL(fill_kernel, dim3(std::max(1, std::min(64, ctx->rb_cap / 256 + 1))), dim3(256), 0, stream,
                       counter_cur, ctx->rb_cap, FG_ROW_BLOCK, kCtr);
    HIPCHK(hipGetLastError());
  }
  FusedArgs a{};
  for (int i = 0; i < c.n_shards; ++i) a.shards[i] = (const uint16_t*)shards[i];
  a.W = (const uint16_t*)W; a.gathered = (uint16_t*)gathered; a.out = (uint16_t*)out;
  a.K = c.K; a.N = c.N; a.n_shards = c.n_shards; a.chunk_cap = ctx->chunk_cap; a.rs_cap = c.max_rows_per_shard;
  a.rb_cap = ctx->rb_cap; a.m_pad_cap = ctx->m_pad_cap;
  a.shard_rows = rows;
  a.slot = ctx->p.slot;
  a.counter_cur = counter_cur;
  a.counter_nxt = ctx->p.counter + (size_t)nxt * ctx->rb_cap * kCtr;
  a.elect_cur = ctx->p.elect + (size_t)cur * c.n_shards * ctx->chunk_cap;
  a.elect_nxt = ctx->p.elect + (size_t)nxt * c.n_shards * ctx->chunk_cap;
  a.pub_count = ctx->p.pub_count; a.seed = ctx->p.seed; a.inv = ctx->p.inv; a.route_ver = ctx->route_ver;
  a.src_of = ctx->p.src_of;
  a.group_of_rb = ctx->p.group_of_rb;
  a.src_row = ctx->p.src_row; a.dst_row = ctx->p.dst_row; a.stream_len = ctx->p.stream_len; a.desc = ctx->p.desc; a.slab = ctx->p.slab; a.gslab = ctx->p.gslab; a.stats = ctx->p.stats;
  a.wgtime = ctx->p.wgtime; a.err = sink(ctx); a.seq = ctx->seq;
  a.n_comm = ctx->n_comm; a.n_gemm = ctx->n_gemm;
  // rows per communication batch: matches the copy template chosen on the
  // device (about 32 KB of loads in flight per wave)
  const int upr = (c.K / 8 + 63) / 64;
  const int rb_max = upr <= 2 ? 16 : upr <= 4 ? 8 : upr <= 8 ? 4 : upr <= 16 ? 2 : 1;
  a.rows_per_batch = c.copy_rows ? std::min(c.copy_rows, rb_max) : rb_max;
  a.flags = flags;
  a.timeout_ticks = timeout_ticks(ctx);
  a.tick_cur = ctx->p.gtick + cur * kTickInts;
  a.tick_nxt = ctx->p.gtick + nxt * kTickInts;
  a.tile_order = c.tile_order;
  a.skc_cur = ctx->p.skc + (size_t)cur * ctx->split_slots;
  a.skc_nxt = ctx->p.skc + (size_t)nxt * ctx->split_slots;
  a.skws = ctx->skws;
  a.skws_bytes = (uint32_t)ctx->skws_bytes;
  a.split_tiles = ctx->split_tiles;
  a.split_slots = ctx->split_slots;
  a.split_parts = ctx->split_parts;
  a.split_forced = ctx->split_tiles != 0;
  a.trace = ctx->p.trace; a.rb_time = ctx->p.rb_time; a.trace_cap = ctx->trace_cap;
  a.two_stage = staging != nullptr;
  a.self_shard = (staging || rc.ring) ? self_shard : -1;
  a.ring_mode = rc.ring != nullptr;
  a.ring = (uint16_t*)rc.ring;
  a.n_channels = rc.ring ? rc.n_channels : 1;
  a.ring_chunks = rc.ring ? rc.ring_chunks : 1;
  a.ring_cap = ctx->ring_cap;
  a.rtail_cur = ctx->p.rtail + (size_t)cur * ctx->ring_cap * kRingTailStride;
  a.rtail_nxt = ctx->p.rtail + (size_t)nxt * ctx->ring_cap * kRingTailStride;
  a.rhead_cur = ctx->p.rhead + (size_t)cur * ctx->ring_cap * kCtr;
  a.rhead_nxt = ctx->p.rhead + (size_t)nxt * ctx->ring_cap * kCtr;
  if (staging)
    for (int i = 0; i < c.n_shards; ++i) a.staging[i] = (uint16_t*)staging[i];
  // in-tile copy (copy_mode 1) where the shape allows it: a one-group dense
  // route, per-XCD tile lists without a forced split, whole 1 KB segments per
  // row and at least three per row (the copy of a row spans that many stages),
  // the one-stage copy and counter gates. Every workgroup then copies the lead
  // rows first (the grid's copy role), and the compute items copy the rest.
  {
    const int grid = a.n_comm + a.n_gemm;
    const bool one_group = mode == FG_ROUTE_CONTIG || (mode == FG_ROUTE_EXPLICIT && (!route->group_off ||
                                                                                     c.n_groups == 1));
    const bool ok = c.copy_mode == 1 && one_group && !staging && !rc.ring && !(flags & FG_CALL_GATE_WATERMARK) &&
                    grid % kXcds == 0 && c.tile_order == 0 && !a.split_forced && c.K % 512 == 0 && c.K >= 1536;
    if (ok) {
      const int per_list = grid / kXcds, n_tn = c.N / ctx->tile_n;
      const long long lead = plan_lead_slabs(per_list, n_tn);
      a.tcopy = 1;
      a.lead_rows = (int)std::min<long long>(m_pad, 2048LL * lead);
      a.n_comm = grid;
      a.n_gemm = 0;
    }
    ctx->last_tcopy = a.tcopy;
    ctx->last_lead_rows = a.tcopy ? a.lead_rows : 0;
  }
  ctx->last_grid = a.n_comm + a.n_gemm;
  ctx->last_n_comm = a.n_comm;
  ctx->last_m_pad = m_pad;
  return ctx->tile_n == 256 ? launch_fused<256>(a, stream) : launch_fused<128>(a, stream);
}

fg_status fg_gather_gemm(fg_ctx* ctx, const void* const* shards, const fg_route* route, const void* W,
                         void* gathered, void* out, uint32_t flags, hipStream_t stream) {
  return gather_gemm_impl(ctx, shards, route, W, nullptr, -1, gathered, out, flags, stream);
}

fg_status fg_gather_gemm_staged(fg_ctx* ctx, const void* const* shards, const fg_route* route, const void* W,
                                void* const* staging, int32_t self_shard, void* gathered, void* out,
                                uint32_t flags, hipStream_t stream) {
  if (!ctx || !staging) return FG_EINVAL;
  if (self_shard < -1 || self_shard >= ctx->cfg.n_shards) return FG_EINVAL;
  for (int i = 0; i < ctx->cfg.n_shards; ++i)
    if (i != self_shard && !staging[i]) return FG_EINVAL;
  return gather_gemm_impl(ctx, shards, route, W, staging, self_shard, gathered, out, flags, stream);
}

fg_status fg_ring_bytes(const fg_config* cfg, int32_t n_channels, int32_t ring_chunks, int64_t* bytes) {
  if (!config_ok(cfg) || !bytes || n_channels < 1 || ring_chunks < 1) return FG_EINVAL;
  *bytes = (int64_t)cfg->n_shards * n_channels * ring_chunks * FG_CHUNK_ROWS * cfg->K * 2;
  return FG_OK;
}

fg_status fg_gather_gemm_ring(fg_ctx* ctx, const void* const* shards, const fg_route* route, const void* W,
                              void* ring, int32_t n_channels, int32_t ring_chunks, int32_t self_shard,
                              void* gathered, void* out, uint32_t flags, hipStream_t stream) {
  if (!ctx || !ring || n_channels < 1 || ring_chunks < 1) return FG_EINVAL;
  if (self_shard < -1 || self_shard >= ctx->cfg.n_shards) return FG_EINVAL;
  // a producer and a consumer copy workgroup per ring
  if ((long long)ctx->cfg.n_shards * n_channels > ctx->ring_cap) return FG_EINVAL;
  RingCall rc;
  rc.ring = ring;
  rc.n_channels = n_channels;
  rc.ring_chunks = ring_chunks;
  return gather_gemm_impl(ctx, shards, route, W, nullptr, self_shard, gathered, out, flags, stream, rc);
}

fg_status fg_barrier(fg_ctx* ctx, int32_t rounds, hipStream_t stream) {
  if (!ctx || rounds < 1 || rounds > 1000000) return FG_EINVAL;
  fg_status s = check_sticky(ctx);
  if (s != FG_OK) return s;
  if (bind_stream(ctx, stream) != FG_OK) return FG_EINVAL;
  HIPCHK(hipSetDevice(ctx->device));
  const int n = ctx->cfg.n_shards;
  hipLaunchKernelGGL(barrier_kernel, dim3(n), dim3(64), 0, stream, ctx->p.bslot, n, ctx->bseq, rounds, sink(ctx),
                     timeout_ticks(ctx), ctx->p.tdev);
  HIPCHK(hipGetLastError());
  ctx->bseq += rounds;
  ctx->host_stats[0] = (unsigned long long)rounds;
  return FG_OK;
}

fg_status fg_pingpong(fg_ctx* ctx, int32_t round_trips, int32_t sys_scope, hipStream_t stream) {
  if (!ctx || round_trips < 1 || round_trips > 10000000) return FG_EINVAL;
  fg_status s = check_sticky(ctx);
  if (s != FG_OK) return s;
  if (bind_stream(ctx, stream) != FG_OK) return FG_EINVAL;
  HIPCHK(hipSetDevice(ctx->device));
  int* a = ctx->p.pp;
  int* b = ctx->p.pp + 64;
  if (sys_scope)
    hipLaunchKernelGGL(pingpong_kernel<1>, dim3(2), dim3(64), 0, stream, a, b, ctx->ppseq, round_trips, sink(ctx),
                       timeout_ticks(ctx), ctx->p.tdev + 1);
  else
    hipLaunchKernelGGL(pingpong_kernel<0>, dim3(2), dim3(64), 0, stream, a, b, ctx->ppseq, round_trips, sink(ctx),
                       timeout_ticks(ctx), ctx->p.tdev + 1);
  HIPCHK(hipGetLastError());
  ctx->ppseq += round_trips;
  ctx->host_stats[1] = (unsigned long long)round_trips;
  return FG_OK;
}

fg_status fg_stress(fg_ctx* ctx, const int32_t* chunk_rows, const int32_t* delays_ns, int32_t* payload,
                    uint32_t flags, hipStream_t stream) {
  if (!ctx || !chunk_rows || !delays_ns || !payload) return FG_EINVAL;
  if (ctx->s_slots == 0) return FG_EINVAL;
  fg_status s = check_sticky(ctx);
  if (s != FG_OK) return s;
  if (bind_stream(ctx, stream) != FG_OK) return FG_EINVAL;
  HIPCHK(hipSetDevice(ctx->device));
  ctx->sseq += 1;
  const int cur = ctx->sseq & 1;
  StressArgs a{};
  a.chunk_rows = chunk_rows; a.delays_ns = delays_ns; a.payload = payload;
  a.slot = ctx->p.s_slot;
  a.elect_cur = ctx->p.s_elect + (size_t)cur * ctx->s_slots;
  a.elect_nxt = ctx->p.s_elect + (size_t)(cur ^ 1) * ctx->s_slots;
  a.pub = ctx->p.s_pub; a.stats = ctx->p.stats; a.err = sink(ctx);
  a.P = ctx->cfg.stress_producers; a.C = ctx->cfg.stress_consumers; a.KC = ctx->cfg.stress_max_chunks;
  a.seq = ctx->sseq; a.flags = flags; a.timeout_ticks = timeout_ticks(ctx);
  a.payload_bytes = (uint32_t)((size_t)ctx->s_slots * FG_CHUNK_ROWS * 4);
  a.wall_khz = ctx->wall_khz;
  hipLaunchKernelGGL(stress_kernel, dim3(a.P + a.C), dim3(kStressThreads), 0, stream, a);
  HIPCHK_STICKY(ctx, hipGetLastError());
  return FG_OK;
}

fg_status fg_combine(fg_ctx* ctx, const void* out, const float* weights, void* const* staging, void* const* y,
                     uint32_t flags, hipStream_t stream) {
  if (!ctx) return FG_EINVAL;
  fg_status s = check_sticky(ctx);
  if (s != FG_OK) return s;
  const fg_config& c = ctx->cfg;
  if (!out || !weights || !staging || !y) return FG_EINVAL;
  if (!al16(out) || ((uintptr_t)weights & 3)) return FG_EINVAL;
  for (int i = 0; i < c.n_shards; ++i)
    if (!staging[i] || !y[i] || !al16(staging[i]) || !al16(y[i])) return FG_EINVAL;
  if ((flags & FG_CALL_COMM_ONLY) && (flags & FG_CALL_GEMM_ONLY)) return FG_EINVAL;
  if (ctx->route_cached_mode != FG_ROUTE_TOPK || ctx->topk_rows < 1) return FG_EINVAL;
  if (bind_stream(ctx, stream) != FG_OK) return FG_EINVAL;
  HIPCHK(hipSetDevice(ctx->device));
  ctx->cseq += 1;
  const int cur = ctx->cseq & 1, nxt = cur ^ 1;
  const size_t nch = (size_t)c.n_shards * ctx->chunk_cap;
  CombineArgs a{};
  a.out = (const uint16_t*)out; a.weights = weights;
  for (int i = 0; i < c.n_shards; ++i) { a.staging[i] = (uint16_t*)staging[i]; a.y[i] = (uint16_t*)y[i]; }
  a.N = c.N; a.n_shards = c.n_shards; a.T = ctx->topk_rows; a.KK = ctx->topk_k; a.rs_cap = c.max_rows_per_shard;
  a.chunk_cap = ctx->chunk_cap;
  a.desc = ctx->p.desc; a.stream_len = ctx->p.stream_len; a.dst_row = ctx->p.dst_row; a.src_k = ctx->p.src_k;
  a.tok_first = ctx->p.tok_first;
  a.cslot = ctx->p.cslot; a.celect_cur = ctx->p.celect + cur * nch * kCombStride; a.celect_nxt = ctx->p.celect + nxt * nch * kCombStride;
  a.cpub = ctx->p.cpub;
  a.stats = ctx->p.stats; a.err = sink(ctx); a.seq = ctx->cseq; a.flags = flags; a.timeout_ticks = timeout_ticks(ctx);
  hipLaunchKernelGGL(combine_kernel, dim3(ctx->combine_wg), dim3(kCombThreads), 0, stream, a);
  HIPCHK_STICKY(ctx, hipGetLastError());
  return FG_OK;
}

fg_status fg_litmus(fg_ctx* ctx, int32_t rounds, int32_t mode, hipStream_t stream) {
  if (!ctx || rounds < 1 || rounds > 1000000 || mode < 0 || mode > 2) return FG_EINVAL;
  fg_status s = check_sticky(ctx);
  if (s != FG_OK) return s;
  if (bind_stream(ctx, stream) != FG_OK) return FG_EINVAL;
  HIPCHK(hipSetDevice(ctx->device));
  int* data = ctx->p.litmus;
  int* flag = data + kLitmusBytes / 4;
  int* ready = flag + 64;
  unsigned long long* stale = (unsigned long long*)(ready + 64);
  auto* k = mode == 0 ? litmus_kernel<0> : mode == 1 ? litmus_kernel<1> : litmus_kernel<2>;
  hipLaunchKernelGGL(k, dim3(2), dim3(64), 0, stream, data, flag, ready, stale, ctx->lseq, rounds, sink(ctx),
                     timeout_ticks(ctx));
  HIPCHK(hipGetLastError());
  ctx->lseq += rounds;
  ctx->litmus_words += (long long)rounds * (kLitmusBytes / 4);
  return FG_OK;
}

fg_status fg_stats(fg_ctx* ctx, fg_stats_t* out, int wait) {
  if (!ctx || !out) return FG_EINVAL;
  HIPCHK(hipSetDevice(ctx->device));
  if (wait && ctx->stream_bound) HIPCHK(hipStreamSynchronize(ctx->stream));
  memset(out, 0, sizeof(*out));
  out->seq = ctx->seq; out->bseq = ctx->bseq; out->stress_seq = ctx->sseq; out->combine_seq = ctx->cseq;
  out->litmus_words = ctx->litmus_words;
  out->n_comm_wg = ctx->n_comm; out->n_gemm_wg = ctx->n_gemm; out->cu_count = ctx->cu_count;
  out->copy_in_tiles = ctx->last_tcopy; out->lead_rows = ctx->last_lead_rows;
  out->m_pad_cap = ctx->m_pad_cap;
  if (!wait) { out->m_pad = ctx->last_m_pad; return FG_OK; }
  int err[4] = {0, 0, 0, 0}, desc = 0;
  unsigned long long st[ST_COUNT];
  long long td[4];
  HIPCHK(hipMemcpy(err, ctx->p.err, sizeof(err), hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(&desc, ctx->p.desc, 4, hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(st, ctx->p.stats, sizeof(st), hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(td, ctx->p.tdev, sizeof(td), hipMemcpyDeviceToHost));
  out->error_code = err[0]; out->error_id = err[1];
  out->timeouts = err[2];
  out->first_timeout_id = err[2] ? err[3] : -1;
  {
    unsigned long long ls = 0;
    HIPCHK(hipMemcpy(&ls, ctx->p.litmus + kLitmusBytes / 4 + 128, 8, hipMemcpyDeviceToHost));
    out->litmus_stale = (int64_t)ls;
  }
  out->m_pad = desc;
  out->publishes = (int64_t)st[ST_PUBLISHES]; out->gate_polls = (int64_t)st[ST_GATE_POLLS];
  out->slot_polls = (int64_t)st[ST_SLOT_POLLS]; out->gate_passes = (int64_t)st[ST_GATE_PASSES];
  out->stale = (int64_t)st[ST_STALE];
  out->expected_publishes = (int64_t)st[ST_EXPECTED];
  const double us_per_tick = 1000.0 / (double)ctx->wall_khz;
  if (ctx->host_stats[0]) out->t_barrier_us = td[0] * us_per_tick / (double)ctx->host_stats[0];
  if (ctx->host_stats[1]) out->t_rtt_us = td[1] * us_per_tick / (double)ctx->host_stats[1];
  if (ctx->last_grid) {
    const int g = ctx->last_grid;
    long long* wg = new (std::nothrow) long long[(size_t)g * kWgTimeFields];
    if (!wg) return FG_ENOMEM;
    if (hipMemcpy(wg, ctx->p.wgtime, (size_t)g * kWgTimeFields * 8, hipMemcpyDeviceToHost) != hipSuccess) {
      delete[] wg;
      return FG_EHIP;
    }
    long long t0 = wg[WT_START], t1 = wg[WT_END], c1 = 0, g0 = -1, g1 = 0, wmax = 0;
    double busy = 0, waitt = 0;
    long long tiles = 0, parts = 0, peff = 1;
    int nw = 0;
    double cyc = 0, wall = 0;
    for (int i = 0; i < g; ++i) {
      const long long* t = wg + (size_t)i * kWgTimeFields;
      t0 = std::min(t0, t[WT_START]);
      t1 = std::max(t1, t[WT_END]);
      if (i < ctx->last_n_comm) c1 = std::max(c1, t[WT_COMM_END]);
      cyc += (double)(t[WT_CLK1] - t[WT_CLK0]);
      wmax = std::max(wmax, t[WT_MAXWAIT]);
      wall += (double)(t[WT_END] - t[WT_START]);
      if (t[WT_TILES] + t[WT_PARTS] > 0) {
        g0 = g0 < 0 ? t[WT_GEMM_START] : std::min(g0, t[WT_GEMM_START]);
        g1 = std::max(g1, t[WT_END]);
        busy += (double)(t[WT_END] - t[WT_GEMM_START] - t[WT_GATE]);
        waitt += (double)t[WT_GATE];
        tiles += t[WT_TILES];
        parts += t[WT_PARTS];
        peff = std::max(peff, t[WT_P]);
        ++nw;
      }
    }
    out->t_kernel_us = (t1 - t0) * us_per_tick;
    out->max_wait_ns = (int64_t)(wmax * us_per_tick * 1000.0);
    out->t_comm_span_us = c1 > t0 ? (c1 - t0) * us_per_tick : 0.0;
    out->t_gemm_span_us = g0 >= 0 ? (g1 - g0) * us_per_tick : 0.0;
    const long long P = std::max(1LL, peff);
    const double units = (double)tiles + (double)parts / P;
    if (nw) {
      out->t_gemm_busy_us = units > 0 ? busy / units * us_per_tick : 0.0;
      out->t_gate_wait_us = waitt / nw * us_per_tick;
    }
    if (wall > 0) out->clock_mhz = cyc / wall * (double)ctx->wall_khz / 1000.0;
    out->tiles_whole = (int32_t)tiles;
    out->tiles_split = (int32_t)(parts / P);
    out->split_parts = (int32_t)P;
    delete[] wg;
  }
  return FG_OK;
}

fg_status fg_views(fg_ctx* ctx, fg_views_t* v) {
  if (!ctx || !v) return FG_EINVAL;
  const Plane& p = ctx->p;
  v->slot = p.slot; v->counter = p.counter; v->elect = p.elect; v->pub_count = p.pub_count; v->seed = p.seed;
  v->inv_row = (const uint64_t*)p.inv; v->route_ver = ctx->route_ver; v->group_of_rb = p.group_of_rb; v->src_row = p.src_row; v->dst_row = p.dst_row;
  v->stream_len = p.stream_len; v->group_off = p.group_off; v->bslot = p.bslot; v->stress_slot = p.s_slot;
  v->stress_pub = p.s_pub;
  v->chunk_cap = ctx->chunk_cap; v->rb_cap = ctx->rb_cap; v->m_pad_cap = ctx->m_pad_cap;
  v->wg_time = (const int64_t*)p.wgtime; v->trace = (const int64_t*)p.trace; v->rb_time = (const int64_t*)p.rb_time;
  v->grid = ctx->n_comm + ctx->n_gemm; v->trace_cap = ctx->trace_cap; v->wall_khz = ctx->wall_khz;
  v->desc = p.desc; v->slab = p.slab; v->group_slab = p.gslab;
  v->combine_slot = p.cslot; v->combine_elect = p.celect; v->combine_pub = p.cpub; v->src_k = p.src_k;
  v->tok_first = p.tok_first;
  v->ring_tail = (const uint64_t*)p.rtail; v->ring_head = p.rhead; v->ring_cap = ctx->ring_cap;
  v->src_of = p.src_of;
  return FG_OK;
}

// ---------------------------------------------------------------------------
// fg_gather_gemm without allocation. The control plane lives in `scratch`, a
// file-scope device array: every GPU the library runs on holds its own copy
// until the process ends. Host code never passes the array's name to a kernel
// (in host code it names a host-side stand-in): the device address of each
// GPU's copy is looked up once per device with hipGetSymbolAddress and kept in
// g_noalloc[device].ptr, which is what the kernels and fills receive.
// ---------------------------------------------------------------------------
fg_status fg_gather_gemm_noalloc(const fg_config* cfg, int hip_device, const void* const* shards,
                                 const fg_route* route, const void* W, void* gathered, void* out, int32_t* status,
                                 uint32_t flags, hipStream_t stream) {
  if (!config_ok(cfg) || !status) return FG_EINVAL;
  if (flags & ~(uint32_t)(FG_CALL_STRICT | FG_CALL_GATE_WATERMARK)) return FG_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return FG_EHIP;
  if (hip_device < 0 || hip_device >= ndev || hip_device >= kNoAllocMaxDevices) return FG_EINVAL;
  HIPCHK(hipSetDevice(hip_device));
  NoAllocDevice& d = g_noalloc[hip_device];
  if (!d.ready) {
    void* ptr = nullptr;
    HIPCHK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return FG_EHIP;
    d.ptr = (char*)ptr;
    d.ready = true;
  }
  fg_ctx* ctx = &d.ctx;
  // the sequence number and the route version carry over from the last call
  // on this device (monotonic, never reset); everything else is per call
  const fg_status st = ctx_setup(ctx, cfg, hip_device, true);
  if (st != FG_OK) return st;
  const size_t bytes = plane_layout(ctx, nullptr);
  if (bytes > kScratchBytes) return FG_EINVAL;
  plane_layout(ctx, d.ptr);
  ctx->no_alloc = true;
  ctx->sticky = FG_OK;
  ctx->stream_bound = false;
  ctx->route_cached_mode = -1;        // the layout step runs on every call
  ctx->plane_mem = nullptr;
  ctx->skws = nullptr;
  ctx->host_status = status;          // device word: the kernels store their first error code here
  // clear what must start at zero (everything but the slots, whose monotonic
  // sequence numbers stay) and the caller's status word, with fill kernels
  const size_t slot_end = align256((size_t)cfg->n_shards * ctx->chunk_cap * 4);
  const int n_words = (int)((bytes - slot_end) / 4);
  hipLaunchKernelGGL(fill_kernel, dim3(std::max(1, std::min(1024, n_words / 256 + 1))), dim3(256), 0, stream,
                     (int*)(d.ptr + slot_end), n_words, 0, 1);
  HIPCHK(hipGetLastError());
  hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(64), 0, stream, (int*)status, 1, 0, 1);
  HIPCHK(hipGetLastError());
  return gather_gemm_impl(ctx, shards, route, W, nullptr, -1, gathered, out, flags, stream);
}

}  // extern "C"
