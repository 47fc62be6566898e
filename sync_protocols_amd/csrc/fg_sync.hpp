// Device-side signal primitives for gfx950 (single-writer slots, monotonic
// sequence numbers, seeded arrival counters, bounded waits).
//
// Basis: "PCIe sync protocols" (compute-comm fused operators, part 4) §2 (slot
// publish / wait, monotonic never-reset seq), §3 (local election, memory-order
// chain), §5 (arrival counter gate), §6 (every wait needs a supplier); "NVLink
// atomic publish" §5.2 (one publish wrapper for every publish), §5.4 (few,
// centralised, backed-off polls); "DeepEP FIFO pipeline" (bounded spin with a
// timeout on every wait).
//
// Memory model on gfx950 (measured on the part):
//  * every XCD has its own L2; a plain or non-temporal store can sit in the
//    writer's L2 where another XCD does not see it;
//  * a store issued with the device-scope cache policy (sc1) writes through to
//    the device coherence point before it is acknowledged;
//  * the compiler's agent-scope release fence writes back the whole L2
//    (buffer_wbl2) and serialises across the chip: one per 8 KB caps a copy at
//    about 0.4 TB/s, so it cannot sit on a per-batch path.
// The default release used here is therefore: every data store of the window
// is a device-scope (sc1) store, and the release waits until all of this wave's
// vector memory operations are acknowledged (s_waitcnt vmcnt(0)); only then is
// the signal written. That is exactly the effect the agent-scope release
// provides for write-through stores, without the L2 write-back. The strict
// variant (formal __builtin_amdgcn_fence release) is kept behind a flag and
// gives bit-identical results. On the acquire side, data written in the same
// kernel by other workgroups is read with device-scope (sc1) loads issued
// after the relaxed poll has returned the signal: such a load does not return
// a line that the reader's L1 or L2 held from before the writer's
// write-through stores (measured: 0 stale words in 20,000 cross-XCD
// message-passing rounds, where plain loads return the stale line every
// time). The agent-scope acquire fence invalidates caches and, issued by
// thousands of waves, cost 5-25 % of a kernel; it is kept as the strict variant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

typedef int v4i __attribute__((ext_vector_type(4)));

// Cache-policy immediates of the gfx950 buffer instructions.
constexpr int kPolSC0 = 1;
constexpr int kPolNT = 2;
constexpr int kPolSC1 = 16;
// Stores that other workgroups read in the same kernel: device scope, so they
// write through to the coherence point. The non-temporal hint is left off: on
// the part it made the fused gather-GEMM 3 % slower at the same copy rate.
constexpr int kPolCoherentStore = kPolSC1;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte device-coherent store at byte offset `off` of the buffer.
__device__ __forceinline__ void store16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, v4i v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolCoherentStore);
}

// 16-byte non-temporal store (no cross-XCD visibility guarantee; outputs only).
__device__ __forceinline__ void store16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, v4i v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolNT);
}


__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Release of this wave's earlier device-coherent stores (see the header note).
// The wait is the compiler's own s_waitcnt (vmcnt 0, the other counters left
// alone), so that its wait placement knows every earlier vector memory result
// has arrived; the empty asm statements keep memory operations from moving
// across it.
constexpr int kWaitVmcnt0 = 0x0F70;   // vmcnt = 0, expcnt = 7, lgkmcnt = 15 (no wait on those)
__device__ __forceinline__ void release_coherent(bool strict) {
  if (strict) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  } else {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    asm volatile("" ::: "memory");
  }
}

__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ int poll_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The one publish operation: store the iteration's sequence number into a
// single-writer slot. Called after release_coherent() of the data it covers.
__device__ __forceinline__ void slot_publish(int* slot, int seq, bool strict) {
  if (strict)
    __hip_atomic_store(slot, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  else
    __hip_atomic_store(slot, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A kernel's single by-value argument, read in place from the kernel argument
// segment (constant memory, scalar loads). Read through the parameter, the
// argument is first copied into a private local; when the compiler cannot
// show every use to be a read it keeps that copy, and every field read from
// it becomes a per-lane value.
template <typename T>
__device__ __forceinline__ const T& kernel_arg() {
  return *(const T*)__builtin_amdgcn_kernarg_segment_ptr();
}

// A zero the compiler cannot see through (a per-lane value to its divergence
// analysis): added to an address, it keeps a single-lane atomic from being
// rewritten into a wave-wide one that needs the result at once.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// A uniform value the compiler cannot prove loop-invariant.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  uint32_t y;
  asm volatile("s_mov_b32 %0, %1" : "=s"(y) : "s"(x));
  return y;
}

__device__ __forceinline__ int fetch_add_relaxed(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int fetch_add_acq_rel(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

// Exponential s_sleep backoff (s_sleep needs an immediate): 64 clocks doubling
// up to 64 << max_lvl. Signal waits whose latency matters stop at 512 clocks
// (kBackoffShort); gate waits, which last tens of microseconds and have many
// waiters, go up to 4096 clocks (kBackoffLong) so that their polls do not load
// the memory channel the producers' counter updates go to.
constexpr int kBackoffShort = 3;
constexpr int kBackoffLong = 6;
__device__ __forceinline__ void backoff(int& lvl, int max_lvl) {
  switch (lvl) {
    case 0: __builtin_amdgcn_s_sleep(1); break;
    case 1: __builtin_amdgcn_s_sleep(2); break;
    case 2: __builtin_amdgcn_s_sleep(4); break;
    case 3: __builtin_amdgcn_s_sleep(8); break;
    case 4: __builtin_amdgcn_s_sleep(16); break;
    case 5: __builtin_amdgcn_s_sleep(32); break;
    default: __builtin_amdgcn_s_sleep(64); break;
  }
  lvl += (lvl < max_lvl);
}

// Error reporting shared by every kernel: first error wins; the code is also
// stored (system scope, the only system-scope write) into a host-visible word.
// Watchdog timeouts are also counted, and the id of the first wait that timed
// out is kept apart from the first error of any kind ("NVLink atomic publish"
// §7: observation counters of the library).
struct ErrorSink {
  int* dev;          // [0] = code, [1] = id of the wait or slot that failed,
                     // [2] = waits that timed out (cumulative), [3] = id of the first of them
  int* host;         // host-visible status word (pinned, coherent)
};

constexpr int kErrTimeoutCode = -5;   // fg_status FG_ETIMEOUT

__device__ __forceinline__ void raise_error(const ErrorSink& e, int code, int id) {
  if (code == kErrTimeoutCode) {
    if (atomicAdd(e.dev + 2, 1) == 0) __hip_atomic_store(e.dev + 3, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (atomicCAS(e.dev, 0, code) == 0) {
    __hip_atomic_store(e.dev + 1, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(e.host, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__device__ __forceinline__ bool error_raised(const ErrorSink& e) { return poll_relaxed(e.dev) != 0; }

// Wait outcome codes (match fg_status values in the public header).
constexpr int kErrTimeout = kErrTimeoutCode;
constexpr int kErrProtocol = -6;

// Bounded wait, one lane: spin until *p == target (a gate) using relaxed polls
// and backoff. Returns 1 on success, 0 on timeout / error elsewhere / overshoot.
// On success the caller reads the signalled data with device-scope loads (the
// strict variant issues acquire_agent() first). *polls counts the loads.
__device__ __forceinline__ int wait_eq(const int* p, int target, uint64_t deadline,
                                       const ErrorSink& e, int id, uint32_t* polls, int max_lvl = kBackoffShort) {
  int lvl = 0;
  uint32_t n = 0;
  while (true) {
    int v = poll_relaxed(p);
    ++n;
    if (v == target) { *polls += n; return 1; }
    if (v > target) { raise_error(e, kErrProtocol, id); *polls += n; return 0; }
    if ((n & 15) == 0) {
      if (now_ticks() > deadline) { raise_error(e, kErrTimeout, id); *polls += n; return 0; }
      if (error_raised(e)) { *polls += n; return 0; }
    }
    backoff(lvl, max_lvl);
  }
}

// Bounded wait, one lane: spin until *p >= seq (a monotonic slot; old values
// are harmless, nothing is ever cleared).
__device__ __forceinline__ int wait_ge(const int* p, int seq, uint64_t deadline,
                                       const ErrorSink& e, int id, uint32_t* polls) {
  int lvl = 0;
  uint32_t n = 0;
  while (true) {
    int v = poll_relaxed(p);
    ++n;
    if (v >= seq) { *polls += n; return 1; }
    if ((n & 15) == 0) {
      if (now_ticks() > deadline) { raise_error(e, kErrTimeout, id); *polls += n; return 0; }
      if (error_raised(e)) { *polls += n; return 0; }
    }
    backoff(lvl, kBackoffShort);
  }
}

// Wave-level helpers (64 lanes).
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

}  // namespace fg
