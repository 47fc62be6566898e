// Combine: the reverse of the expert dispatch, with the same signalling.
//
// "PCIe sync protocols" §3 (layer-1 combine: the producer pushes its rows into
// the receiver's buffer, counts them locally and the last writer of each chunk
// stores seq into the chunk's single-writer slot) and §4 (one signal per 64
// entries of a stream). Here the producer side is this GPU's expert outputs,
// laid out in gathered-row order by the dispatch, and the receiver side is one
// staging buffer per source shard, indexed by that shard's stream entries; the
// shard's side then forms, per token, the gate-weighted sum of its local picks.
//
// One kernel; every wave takes push items i, i + waves, ..., then reduce items
// i, i + waves, ... (both in shard-major order):
//  * push items (4 stream entries of one shard per wave): copy
//    out[dst_row[s][i]] -> staging[s][i] bitwise with device-coherent stores,
//    release, add the wave's rows to the chunk's election count; the add that
//    completes the chunk elects the wave, whose leader stores seq in the slot;
//  * reduce items (4 tokens of one shard per wave): wait until the slot of
//    every chunk holding the tokens' entries carries seq, then write
//    y[s][t] = bf16(sum over the token's entries e, in k order, of
//    w[s][t][k(e)] * staging[s][e]) with fp32 products and sums, the staging
//    rows read with device-scope loads.
// A wave starts its reduce items only after its push items, and the host
// checks that the whole grid is co-resident, so every wait has a running
// supplier that does not wait ("PCIe sync protocols" §6 audit). Static item assignment keeps atomics off the item
// hand-out: one ticket counter shared by every workgroup serialises at its
// memory channel. Slots and election counts sit one per 256-byte line, so the
// pollers of one slot do not load the channel of its neighbours.
#pragma once

#include "fg_kernels.hpp"

namespace fg {

constexpr int kCombWaves = 4;
constexpr int kCombThreads = 64 * kCombWaves;
// Build-time shape of the work items (defaults measured fastest on the EP workload).
#ifndef FG_COMB_PUSH
#define FG_COMB_PUSH 4
#endif
#ifndef FG_COMB_TOKENS
#define FG_COMB_TOKENS 4
#endif
#ifndef FG_COMB_U
#define FG_COMB_U 4
#endif
constexpr int kCombStride = FG_COUNTER_STRIDE;            // ints per combine slot / election count (own line)
constexpr int kPushPerWave = FG_COMB_PUSH;                // stream entries per push item (one wave)
constexpr int kRedPerWave = FG_COMB_TOKENS;               // tokens per reduce item (one wave)
constexpr int kCombU = FG_COMB_U;                         // 16-byte vectors per lane and row per column step

static_assert(kChunk % kPushPerWave == 0, "a push item lies inside one chunk");
static_assert(kPushPerWave <= 64 && kRedPerWave * 16 <= 64 && kRedPerWave < 64, "lane layout");

struct CombineArgs {
  const uint16_t* out;            // [m_pad][N] expert outputs, gathered-row order
  const float* weights;           // [S][T][KK] gate weights
  uint16_t* staging[FG_MAX_SHARDS];  // per shard [rs_cap][N], stream-entry order
  uint16_t* y[FG_MAX_SHARDS];     // per shard [T][N]
  int N, n_shards, T, KK, rs_cap, chunk_cap;
  const int* desc;                // [0] = m_pad of the route in use
  const int* stream_len;
  const int* dst_row;             // [S][rs_cap]
  const int* src_k;               // [S][rs_cap] top-k position of each stream entry
  const int* tok_first;           // [S][rs_cap + 1] first stream entry of each token, [T] = stream length
  int* cslot;                     // [S][chunk_cap]
  int* celect_cur;                // [S][chunk_cap]
  int* celect_nxt;
  int* cpub;
  unsigned long long* stats;
  ErrorSink err;
  int seq;
  uint32_t flags;
  uint64_t timeout_ticks;
};

__device__ __forceinline__ const uint16_t* uniform_ptr(const void* p) {
  const uint64_t b = (uint64_t)p;
  return (const uint16_t*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b));
}

// One wave: push entries eb .. eb + kPushPerWave - 1 of shard s.
__device__ __forceinline__ void combine_push(const CombineArgs& a, const uint16_t* stg, int s, int eb, int n_s,
                                             uint32_t out_bytes, int lane) {
  const bool strict = a.flags & kStrict;
  const uint32_t row_bytes = (uint32_t)a.N * 2;
  int g = -1;
  if (lane < kPushPerWave && eb + lane < n_s) {
    g = a.dst_row[s * a.rs_cap + eb + lane];
    if (g < 0 || (uint32_t)g * row_bytes >= out_bytes) {
      raise_error(a.err, kErrProtocol, 0x60000000 | s);
      g = -1;
    }
  }
  __amdgpu_buffer_rsrc_t rs[kPushPerWave], rd[kPushPerWave];
#pragma unroll
  for (int r = 0; r < kPushPerWave; ++r) {
    const int gr = readlane(g, r);
    const bool valid = gr >= 0;
    rs[r] = buffer_rsrc(a.out + (size_t)(valid ? gr : 0) * a.N, valid ? row_bytes : 0u);
    rd[r] = buffer_rsrc(stg + (size_t)(eb + r) * a.N, valid ? row_bytes : 0u);
  }
  const int nvec = a.N / 8;
  for (int c0 = 0; c0 < nvec; c0 += 64 * 2 * kCombU) {
    v4i v[kPushPerWave][2 * kCombU];
#pragma unroll
    for (int r = 0; r < kPushPerWave; ++r)
#pragma unroll
      for (int u = 0; u < 2 * kCombU; ++u)
        v[r][u] = __builtin_amdgcn_raw_buffer_load_b128(rs[r], (uint32_t)(c0 + u * 64 + lane) * 16, 0, 0);
#pragma unroll
    for (int r = 0; r < kPushPerWave; ++r)
#pragma unroll
      for (int u = 0; u < 2 * kCombU; ++u) store16_coherent(rd[r], (uint32_t)(c0 + u * 64 + lane) * 16, v[r][u]);
  }
  release_coherent(strict);
  const int n_done = __popcll(ballot(g >= 0));
  if (lane == 0 && n_done > 0) {
    const int c = eb / kChunk, ch = s * a.chunk_cap + c;
    int* const el = a.celect_cur + (size_t)ch * kCombStride;
    const int old = strict ? fetch_add_acq_rel(el, n_done) : fetch_add_relaxed(el, n_done);
    const int expect = min(kChunk, n_s - kChunk * c);
    if (old + n_done == expect) {
      if (!((a.flags & kDropPublish) && ch == 0)) slot_publish(a.cslot + (size_t)ch * kCombStride, a.seq, strict);
      if (a.flags & kVerify) {
        atomicAdd(a.cpub + ch, 1);
        atomicAdd(a.stats + ST_PUBLISHES, 1ull);
      }
    } else if (old + n_done > expect) {
      raise_error(a.err, kErrProtocol, 0x10000000 | ch);
    }
  }
}

__device__ __forceinline__ void bf16x8_fma(float* acc, v4i x, float w) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t b = (uint32_t)x[h];
    acc[2 * h] += w * __builtin_bit_cast(float, b << 16);
    acc[2 * h + 1] += w * __builtin_bit_cast(float, b & 0xFFFF0000u);
  }
}

// First stream entry of tokens tb .. tb + kRedPerWave of shard s, in lanes
// 0 .. kRedPerWave. The tables come from the layout step; clamping keeps every
// access inside the buffers even if a failed layout left them stale (it also
// raised an error).
__device__ __forceinline__ int reduce_first_entries(const CombineArgs& a, int s, int tb, int lane) {
  int tf = 0;
  if (lane <= kRedPerWave) tf = a.tok_first[(size_t)s * (a.rs_cap + 1) + min(tb + lane, a.T)];
  return tf;
}

// Gate weight of entry j of token r in lane 16 r + j (j < 16); entries 16.. of
// a token (more than 16 local picks) load their weight when used.
__device__ __forceinline__ float reduce_weights(const CombineArgs& a, int s, int tb, int tf, int lane) {
  const int r = lane >> 4, j = lane & 15;
  const int my_ea = __shfl(tf, r, 64);
  const int my_ne = (r < kRedPerWave && tb + r < a.T) ? __shfl(tf, r + 1, 64) - my_ea : 0;
  float wl = 0.f;
  if (j < my_ne) {
    const int k = min(max(a.src_k[s * a.rs_cap + my_ea + j], 0), a.KK - 1);
    wl = a.weights[((size_t)s * a.T + tb + r) * a.KK + k];
  }
  return wl;
}

// One wave: y rows of tokens tb .. tb + kRedPerWave - 1 of shard s from the
// published staging rows; tf and wl from the two functions above.
__device__ __forceinline__ void combine_reduce(const CombineArgs& a, const uint16_t* stg, uint16_t* yb, int s, int tb,
                                               int tf, float wl, int lane) {
  const uint32_t row_bytes = (uint32_t)a.N * 2;
  int ea[kRedPerWave], ne[kRedPerWave];
  int maxn = 0;
#pragma unroll
  for (int r = 0; r < kRedPerWave; ++r) {
    ea[r] = readlane(tf, r);
    ne[r] = tb + r < a.T ? max(0, readlane(tf, r + 1) - ea[r]) : 0;
    maxn = max(maxn, ne[r]);
  }
  const int nvec = a.N / 8;
  for (int c0 = 0; c0 < nvec; c0 += 64 * kCombU) {
    float acc[kRedPerWave][kCombU][8];
#pragma unroll
    for (int r = 0; r < kRedPerWave; ++r)
#pragma unroll
      for (int u = 0; u < kCombU; ++u)
#pragma unroll
        for (int h = 0; h < 8; ++h) acc[r][u][h] = 0.f;
    for (int j = 0; j < maxn; ++j) {
      v4i v[kRedPerWave][kCombU];
      float w[kRedPerWave];
#pragma unroll
      for (int r = 0; r < kRedPerWave; ++r) {
        const bool valid = j < ne[r];
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(stg + (size_t)(valid ? ea[r] + j : 0) * a.N, valid ? row_bytes : 0u);
#pragma unroll
        for (int u = 0; u < kCombU; ++u)
          v[r][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(c0 + u * 64 + lane) * 16, 0, kPolSC1 | kPolNT);
        float wr = 0.f;
        if (valid) {
          if (j < 16) {
            wr = __builtin_bit_cast(float, readlane(__builtin_bit_cast(int, wl), 16 * r + j));
          } else {
            const int k = min(max(a.src_k[s * a.rs_cap + ea[r] + j], 0), a.KK - 1);
            wr = a.weights[((size_t)s * a.T + tb + r) * a.KK + k];
          }
        }
        w[r] = wr;
      }
#pragma unroll
      for (int r = 0; r < kRedPerWave; ++r)
#pragma unroll
        for (int u = 0; u < kCombU; ++u) bf16x8_fma(acc[r][u], v[r][u], w[r]);
    }
#pragma unroll
    for (int r = 0; r < kRedPerWave; ++r) {
      const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(yb + (size_t)min(tb + r, a.T - 1) * a.N, tb + r < a.T ? row_bytes : 0u);
#pragma unroll
      for (int u = 0; u < kCombU; ++u) {
        v4i o;
#pragma unroll
        for (int h = 0; h < 4; ++h) o[h] = (int)pack_bf16x2(acc[r][u][2 * h], acc[r][u][2 * h + 1]);
        store16_stream(ro, (uint32_t)(c0 + u * 64 + lane) * 16, o);
      }
    }
  }
}

__global__ __launch_bounds__(kCombThreads) void combine_kernel(CombineArgs a) {
  __shared__ const uint16_t* sh_stg[FG_MAX_SHARDS];
  __shared__ uint16_t* sh_y[FG_MAX_SHARDS];
  __shared__ int sh_base[FG_MAX_SHARDS + 1];     // push items before shard s
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  // arm the other parity for the next call (nothing else touches it here)
  for (int i = blockIdx.x * kCombThreads + threadIdx.x; i < a.n_shards * a.chunk_cap; i += G * kCombThreads)
    a.celect_nxt[(size_t)i * kCombStride] = 0;
  if ((int)threadIdx.x < a.n_shards) {
    sh_stg[threadIdx.x] = a.staging[threadIdx.x];
    sh_y[threadIdx.x] = a.y[threadIdx.x];
  }
  if (threadIdx.x == 0) {
    int n = 0;
    unsigned long long want = 0;
    for (int s = 0; s < a.n_shards; ++s) {
      sh_base[s] = n;
      n += (a.stream_len[s] + kPushPerWave - 1) / kPushPerWave;
      want += (a.stream_len[s] + kChunk - 1) / kChunk;
    }
    sh_base[a.n_shards] = n;
    // VERIFY: one publish per active 64-entry chunk of every stream
    if (blockIdx.x == 0 && (a.flags & kVerify) && !(a.flags & kGemmOnly)) atomicAdd(a.stats + ST_EXPECTED, want);
  }
  __syncthreads();
  if (error_raised(a.err)) return;
  const int m_pad = __builtin_amdgcn_readfirstlane(a.desc[0]);
  const uint32_t out_bytes = (uint32_t)m_pad * (uint32_t)a.N * 2;
  const int n_push = sh_base[a.n_shards];
  const int nw = G * kCombWaves, wid = blockIdx.x * kCombWaves + wave;
  const int ntb = (a.T + kRedPerWave - 1) / kRedPerWave;
  const int n_red = a.n_shards * ntb;
  // the route tables are ready before the kernel starts: the first entries of
  // this wave's first reduce item load while the push phase runs
  int tf_next = 0;
  if (wid < n_red) tf_next = reduce_first_entries(a, wid / ntb, (wid % ntb) * kRedPerWave, lane);

  if (!(a.flags & kGemmOnly)) {
    for (int it = wid; it < n_push; it += nw) {
      int s = 0;
      while (s + 1 < a.n_shards && sh_base[s + 1] <= it) ++s;
      s = __builtin_amdgcn_readfirstlane(s);
      const int n_s = __builtin_amdgcn_readfirstlane(a.stream_len[s]);
      combine_push(a, uniform_ptr(sh_stg[s]), s, (it - sh_base[s]) * kPushPerWave, n_s, out_bytes, lane);
    }
  }
  if (a.flags & kCommOnly) return;

  const bool wait = !(a.flags & kGemmOnly);
  const bool verify = a.flags & kVerify;
  const bool strict = a.flags & kStrict;
  for (int it = wid; it < n_red; it += nw) {
    const int s = it / ntb, tb = (it - s * ntb) * kRedPerWave;
    const int tf = min(max(tf_next, 0), a.rs_cap);
    // gate weights first: their loads run while the slots are polled
    const float wl = reduce_weights(a, s, tb, tf, lane);
    if (it + nw < n_red) tf_next = reduce_first_entries(a, (it + nw) / ntb, ((it + nw) % ntb) * kRedPerWave, lane);
    if (wait) {
      int ok = 1;
      const int e_lo = readlane(tf, 0), e_hi = readlane(tf, min(kRedPerWave, a.T - tb));
      if (lane == 0) {
        uint32_t polls = 0;
        const uint64_t deadline = now_ticks() + a.timeout_ticks;
        for (int c = e_lo / kChunk; c * kChunk < e_hi && ok; ++c) {
          const int ch = s * a.chunk_cap + c;
          ok = wait_ge(a.cslot + (size_t)ch * kCombStride, a.seq, deadline, a.err, 0x70000000 | ch, &polls);
        }
        if (verify) atomicAdd(a.stats + ST_SLOT_POLLS, (unsigned long long)polls);
      }
      if (!readlane(ok, 0)) break;
      // the staging rows are read with device-scope loads, issued after the
      // poll returned seq (the rows were written through before seq was
      // stored); the formal acquire fence is the strict variant
      if (strict) acquire_agent();
    }
    combine_reduce(a, uniform_ptr(sh_stg[s]), (uint16_t*)uniform_ptr(sh_y[s]), s, tb, tf, wl, lane);
  }
}

}  // namespace fg
