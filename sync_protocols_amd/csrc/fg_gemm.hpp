// bf16 x bf16 -> fp32 MFMA tile for gfx950, LDS-staged, two stages.
//
// The contraction is the dense GEMM the compute workgroups run once a row
// block's gate opens (the GEMM behind the gate of "PCIe sync protocols" §5):
//   out[m][n] = sum_k A[m][k] * W[k][n],  A = gathered rows (bf16, K contiguous),
//   W stored as [N][K] (K contiguous), fp32 accumulation, bf16 RNE output.
//
// Tile BM x BN, eight waves as 2 x 4 (two per SIMD), each wave (BM/2) x (BN/4) built from
// v_mfma_f32_16x16x32_bf16 fragments (the default), or from
// v_mfma_f32_32x32x16_bf16 fragments in the build variants below. At the
// part's power cap a stream of 16x16x32 MFMAs holds a higher clock than the
// same FLOP in 32x32x16 ones (measured: 1.99 against 1.73 PFLOP/s of MFMA work
// alone), since each instruction moves fewer accumulator bytes per product.
// The weight tile is the MFMA "A" operand and the gathered tile the "B"
// operand, so that each lane's four consecutive accumulator values are four
// consecutive output columns of one row; the epilogue (tile_store) regroups
// them through LDS into 16-byte pieces of whole rows. Lane layouts: 32x32x16,
// operand lane l holds row/col l % 32 and k = 8 * (l / 32) + 0..7, result
// register v of lane l is D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32];
// 16x16x32, operand lane l holds row/col l % 16 and k = 8 * (l / 16) + 0..7,
// result register v of lane l is D[4 * (l / 16) + v][l % 16].
//
// LDS: two stages; per stage each operand tile is stored as rows of 64 k (one
// 128-byte line = 8 slots of 16 bytes; full lines keep the L2 request rate at
// its best), logical chunk c of row r in slot c ^ ((r >> 1) & 7) (see swz).
// Global -> LDS moves use buffer_load ... lds (16 bytes per lane, lane i writes
// base + 16 i), so the swizzle is applied by choosing which chunk a lane fetches.
#pragma once

#include <type_traits>

#include "fg_sync.hpp"

namespace fg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

#ifndef FG_BK
#define FG_BK 64
#endif
constexpr int kBK = FG_BK;          // k per LDS stage: 64 (two stages of 128-byte rows) or 32 (a ring of
                                    // four stages of 64-byte rows: same LDS, three stages of load lead)
constexpr int kRowB = kBK * 2;      // bytes per tile row per stage
constexpr int kRowsPerLoad = 1024 / kRowB;   // rows covered by one 64-lane 16-byte load
constexpr int kKSteps = kBK / 16;   // k-steps per stage (each a quarter of a 64-k stage's MFMAs, either shape)
constexpr int kStages = kBK == 64 ? 2 : 4;
constexpr int kChunks = kRowB / 16;          // 16-byte chunks per row and stage
static_assert(kBK == 64 || kBK == 32, "stage depth");

#ifndef FG_WAVES
#define FG_WAVES 8
#endif
#ifndef FG_PINGPONG
#define FG_PINGPONG 0
#endif
#ifndef FG_MFMA16
#define FG_MFMA16 1
#endif
constexpr bool kPingPong = FG_PINGPONG != 0 && FG_WAVES == 8;   // the ping-pong stage schedule below
constexpr int kWaves = FG_WAVES;    // waves per workgroup: 8 = two per SIMD, so one wave's memory
                                    // instructions issue while the other's MFMAs run; 4 = one per SIMD
                                    // with a 128 x 128 wave tile (fewer LDS reads per MFMA)
// 16x16x32 MFMAs in the default schedule (64-k stages, eight waves, the
// interleaved stage schedule); the other variants keep 32x32x16
constexpr bool kMfma16 = FG_MFMA16 != 0 && FG_BK == 64 && FG_WAVES == 8 && !kPingPong;

template <int BM, int BN>
struct Tile {
  static constexpr int WGN = kWaves == 8 ? 4 : 2;     // waves along n
  static constexpr int WGM = kWaves / WGN;            // waves along m
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // per-wave tile
  static constexpr int FM = WM / 32, FN = WN / 32;   // 32 x 32 accumulator blocks per wave
  static constexpr int VW = kMfma16 ? 2 * FM : FM;    // output rows per lane (row version words)
  static constexpr int A_BYTES = BM * kRowB;
  static constexpr int B_BYTES = BN * kRowB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LOADS_A = BM / kRowsPerLoad / kWaves;   // buffer_load_lds per wave per stage for A
  static constexpr int LOADS_B = BN / kRowsPerLoad / kWaves;
  static constexpr int LOADS = LOADS_A + LOADS_B;
  static_assert(FM >= 1 && FN >= 1 && LOADS_A >= 1 && LOADS_B >= 1, "tile too small for the wave layout");
};

typedef __attribute__((address_space(3))) void lds_void;

// Slot of logical 16-byte chunk c (0..7) of tile row r. The LDS serves a
// ds_read_b128 sixteen lanes (256 bytes, all 64 banks) at a time; the 16 rows
// read together (same c) must land in 16 distinct 16-byte bank groups. With
// 128-byte rows, rows of equal parity share a half of the bank space, so the
// slot is permuted by (r >> 1) & 7; with 64-byte rows, rows r mod 4 share a
// quarter, permuted by (r >> 2) & 3.
constexpr int kPolA = kPolSC1;   // gathered-row loads: device scope (see stage_load)

__device__ __forceinline__ int swz(int c, int r) { return c ^ ((r / (256 / kRowB)) & (kChunks - 1)); }

// Issue this wave's share of one stage: ROWS rows starting at byte offset
// row0_off of the buffer, k slice [k0, k0 + 64), into LDS at `lds`. Each row
// of the stage is one full 128-byte line (8 lanes x 16 bytes).
// POL is the cache policy of the loads: the gathered rows (written in the same
// kernel by other workgroups, possibly on other XCDs) are read with
// device-scope loads, the weights with the default policy.
template <int ROWS, int POL>
__device__ __forceinline__ void stage_load(__amdgpu_buffer_rsrc_t r, uint32_t row0_off, uint32_t row_stride,
                                           uint32_t k0_bytes, char* lds, int wave, int lane) {
  constexpr int PER_WAVE = ROWS / kRowsPerLoad / kWaves;
  const int sub = lane / kChunks;      // row within the block of one load
  const int slot = lane % kChunks;
#pragma unroll
  for (int q = 0; q < PER_WAVE; ++q) {
    const int blk = wave * PER_WAVE + q;
    const int row = blk * kRowsPerLoad + sub;
    const int chunk = swz(slot, row);  // the xor is its own inverse
    const uint32_t voff = row0_off + (uint32_t)row * row_stride + (uint32_t)chunk * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + blk * 1024), 16, voff, k0_bytes, 0, POL);
  }
}

// One 16-byte operand fragment: row `row`, logical k chunk c (0..7) of the stage.
__device__ __forceinline__ bf16x8 frag_read(const char* lds, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(lds + row * kRowB + swz(c, row) * 16);
}

// Accumulators per wave, one 32 x 32 output block per (fm, fn): with 32x32x16
// MFMAs one f32x16; with 16x16x32 the block's four 16 x 16 quarters, quarter
// 2 i + j covering output columns 16 i .. 16 i + 15 and rows 16 j .. 16 j + 15
// of the block.
template <int BM, int BN>
struct Acc32 {
  f32x16 v[Tile<BM, BN>::FM][Tile<BM, BN>::FN];
};
template <int BM, int BN>
struct Acc16 {
  f32x4 v[Tile<BM, BN>::FM][Tile<BM, BN>::FN][4];
};
template <int BM, int BN>
using Acc = std::conditional_t<kMfma16, Acc16<BM, BN>, Acc32<BM, BN>>;

// Accumulator group g (0..3) of block (fm, fn): four consecutive output
// columns of one output row of the block, at row acc_row(g, lane) and first
// column acc_col(g, lane) of the block.
__device__ __forceinline__ int acc_row(int g, int lane) { return kMfma16 ? 16 * (g & 1) + (lane & 15) : (lane & 31); }
__device__ __forceinline__ int acc_col(int g, int lane) {
  return kMfma16 ? 16 * (g >> 1) + 4 * (lane >> 4) : 8 * g + 4 * (lane >> 5);
}
// The row version word (tile_row_versions) of group g of fragment row fm.
__device__ __forceinline__ int acc_vw(int fm, int g) { return kMfma16 ? 2 * fm + (g & 1) : fm; }

template <int BM, int BN>
__device__ __forceinline__ f32x4 acc_group(const Acc32<BM, BN>& acc, int fm, int fn, int g) {
  const f32x16& c = acc.v[fm][fn];
  return f32x4{c[4 * g + 0], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
}
template <int BM, int BN>
__device__ __forceinline__ f32x4 acc_group(const Acc16<BM, BN>& acc, int fm, int fn, int g) {
  return acc.v[fm][fn][g];
}
template <int BM, int BN>
__device__ __forceinline__ void acc_zero(Acc32<BM, BN>& acc) {
#pragma unroll
  for (int i = 0; i < Tile<BM, BN>::FM; ++i)
#pragma unroll
    for (int j = 0; j < Tile<BM, BN>::FN; ++j) acc.v[i][j] = f32x16{};
}
template <int BM, int BN>
__device__ __forceinline__ void acc_zero(Acc16<BM, BN>& acc) {
#pragma unroll
  for (int i = 0; i < Tile<BM, BN>::FM; ++i)
#pragma unroll
    for (int j = 0; j < Tile<BM, BN>::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc.v[i][j][q] = f32x4{};
}

// Fragments of one k-step. 32x32x16: the k-step is 16 k of the stage, with
// the weight fragments b[fn] and the gathered-row fragments a[fm]. 16x16x32:
// the k-step is half of the MFMAs of one 32-k half of the stage (k-step kk:
// k half kk / 2, fragment rows fm of half kk % 2); w[2 fn + i] holds weight
// rows 16 i .. 16 i + 15 of column block fn (read at even k-steps and kept for
// the odd one), g[2 f + j] rows 16 j .. 16 j + 15 of the half's f-th fragment
// row.
template <int BM, int BN>
struct Frags32 {
  bf16x8 b[Tile<BM, BN>::FN];
  bf16x8 a[Tile<BM, BN>::FM];
};
template <int BM, int BN>
struct Frags16 {
  bf16x8 w[2 * Tile<BM, BN>::FN];
  bf16x8 g[Tile<BM, BN>::FM];
};
template <int BM, int BN>
using Frags = std::conditional_t<kMfma16, Frags16<BM, BN>, Frags32<BM, BN>>;

// MFMAs per k-step, and the fragment reads that k-step kk needs.
template <int BM, int BN>
struct KStep {
  using T = Tile<BM, BN>;
  static constexpr int NM = kMfma16 ? 2 * T::FM * T::FN : T::FM * T::FN;
  __device__ static constexpr int nr(int kk) {
    return kMfma16 ? (kk % 2 == 0 ? T::FM + 2 * T::FN : T::FM) : T::FM + T::FN;
  }
};

template <int BM, int BN>
__device__ __forceinline__ void frags_read(const char* ldsA, const char* ldsB, Frags<BM, BN>& f, int kk, int wm,
                                           int wn, int lane) {
  using T = Tile<BM, BN>;
  const int lr = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int fn = 0; fn < T::FN; ++fn) f.b[fn] = frag_read(ldsB, wn * T::WN + fn * 32 + lr, kk * 2 + kh);
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm) f.a[fm] = frag_read(ldsA, wm * T::WM + fm * 32 + lr, kk * 2 + kh);
}

template <int BM, int BN>
__device__ __forceinline__ void frags_mfma(const Frags<BM, BN>& f, Acc<BM, BN>& acc) {
  using T = Tile<BM, BN>;
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn)
      acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc.v[fm][fn], 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

#define FG_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// K loop for one tile (or one k-range of it; the stage count is even).
// rA: gathered rows (row stride K*2 bytes), a_off = byte offset of the tile's
// first row; rB: weight rows [N][K], b_off likewise. lds0/lds1: the two stage
// buffers (distinct objects, so the compiler can tell them apart when it places
// its own waits).
//
// Stage k lives in slot k&1 and k-step 0 of its fragments is already in
// registers when the stage starts. Per stage: read k-steps 1..3 and load the
// weight rows of stage k+1 into the other slot during the MFMAs of k-steps 0
// to 2, wait for this wave's loads of stage k+1, one workgroup barrier
// (publishes stage k+1 from every wave and retires slot k&1, whose fragments
// are all in registers by now), load the gathered rows of stage k+2 into slot
// k&1 and read k-step 0 of stage k+1 during the MFMAs of k-step 3.
// --- explicitly interleaved stage schedule -------------------------------
// With one wave per SIMD nothing else fills the matrix pipe while a wave
// issues memory instructions, so every LDS read and every global->LDS load is
// issued in the shadow of one 32-cycle MFMA: the stage is a fixed sequence of
// MFMA slots, each followed by at most one memory instruction, fenced so the
// compiler keeps the order.
// MFMA i of k-step KK.
template <int BM, int BN, int KK = 0>
__device__ __forceinline__ void mfma_one(const Frags<BM, BN>& f, Acc<BM, BN>& acc, int i) {
  using T = Tile<BM, BN>;
  if constexpr (kMfma16) {
    // i -> (fn, column quarter qi, f, row quarter qj), qj fastest: the MFMAs of
    // a k-step each update a different accumulator, and each weight fragment
    // is used by consecutive MFMAs, so that at an odd k-step the weights die
    // one by one and the next stage's weight fragments, read last, can take
    // their registers
    constexpr int H = T::FM / 2;
    const int qj = i & 1, fl = (i >> 1) % H, qi = (i / (2 * H)) & 1, fn = i / (4 * H);
    const int fm = (KK & 1) * H + fl;
    acc.v[fm][fn][2 * qi + qj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[2 * fn + qi], f.g[2 * fl + qj],
                                                                         acc.v[fm][fn][2 * qi + qj], 0, 0, 0);
  } else {
    const int fm = i / T::FN, fn = i % T::FN;
    acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc.v[fm][fn], 0, 0, 0);
  }
}

// Element e of k-step kk's fragment reads: 32x32x16, b[0..FN) then a[0..FM),
// in the order the MFMAs consume them; 16x16x32, g[0..FM), then at even
// k-steps w[0..2 FN) (w is carried over to the odd one), read last so that
// they can reuse the registers of the weights that the MFMAs before them
// release.
template <int BM, int BN>
__device__ __forceinline__ void frag_read_one(const char* ldsA, const char* ldsB, Frags<BM, BN>& f, int kk, int e,
                                              int wm, int wn, int lane) {
  using T = Tile<BM, BN>;
  if constexpr (kMfma16) {
    const int l16 = lane & 15, c = 4 * (kk >> 1) + (lane >> 4);   // 16-byte chunk of the stage row
    if (e < T::FM) {
      const int fm = (kk & 1) * (T::FM / 2) + (e >> 1);
      f.g[e] = frag_read(ldsA, wm * T::WM + fm * 32 + 16 * (e & 1) + l16, c);
    } else {
      const int e2 = e - T::FM;
      f.w[e2] = frag_read(ldsB, wn * T::WN + (e2 >> 1) * 32 + 16 * (e2 & 1) + l16, c);
    }
  } else {
    const int lr = lane & 31, kh = lane >> 5;
    if (e < T::FN) f.b[e] = frag_read(ldsB, wn * T::WN + e * 32 + lr, kk * 2 + kh);
    else f.a[e - T::FN] = frag_read(ldsA, wm * T::WM + (e - T::FN) * 32 + lr, kk * 2 + kh);
  }
}

// All of k-step kk's fragment reads.
template <int BM, int BN>
__device__ __forceinline__ void frags_read_kstep(const char* ldsA, const char* ldsB, Frags<BM, BN>& f, int kk, int wm,
                                                 int wn, int lane) {
#pragma unroll
  for (int e = 0; e < KStep<BM, BN>::nr(kk); ++e) frag_read_one<BM, BN>(ldsA, ldsB, f, kk, e, wm, wn, lane);
}

// 16x16x32: the odd k-step of a k half uses the weight fragments read for the
// even one.
template <int BM, int BN>
__device__ __forceinline__ void carry_weights(Frags<BM, BN>& dst, const Frags<BM, BN>& src) {
  if constexpr (kMfma16) {
#pragma unroll
    for (int e = 0; e < 2 * Tile<BM, BN>::FN; ++e) dst.w[e] = src.w[e];
  }
}

// Load q (0..LOADS) of this wave's share of a stage; the stage's k offset is
// the scalar offset of the buffer instruction.
template <int BM, int BN>
__device__ __forceinline__ void stage_load_one(__amdgpu_buffer_rsrc_t rA, uint32_t a_off, __amdgpu_buffer_rsrc_t rB,
                                               uint32_t b_off, uint32_t stride, uint32_t k0_bytes, char* lds,
                                               int wave, int lane, int q) {
  using T = Tile<BM, BN>;
  const bool isA = q < T::LOADS_A;
  const int blk = isA ? wave * T::LOADS_A + q : wave * T::LOADS_B + (q - T::LOADS_A);
  const int row = blk * kRowsPerLoad + lane / kChunks;
  const int chunk = swz(lane % kChunks, row);
  const uint32_t voff = (isA ? a_off : b_off) + (uint32_t)row * stride + (uint32_t)chunk * 16;
  if (isA)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(lds + blk * 1024), 16, voff, k0_bytes, 0, kPolA);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(lds + T::A_BYTES + blk * 1024), 16, voff, k0_bytes, 0, 0);
}

// Memory operations of one MFMA window: NR fragment reads and NL global->LDS
// loads, interleaved (a load after every read while both last) so that loads
// are not issued in bursts. mix_load(o) says whether op o is a load; its index
// among the loads (or reads) is mix_index(o).
template <int NR, int NL>
struct Mix {
  static constexpr int P = NR < NL ? NR : NL;
  static constexpr int OPS = NR + NL;
  __device__ static constexpr bool load(int o) { return o < 2 * P ? (o & 1) : NL > NR; }
  __device__ static constexpr int index(int o) { return o < 2 * P ? o / 2 : P + (o - 2 * P); }
};

// Stage k in `cur`, its k-step 0 fragments already in f0.
//   phase A: MFMAs of k-steps 0, 1, 2; the reads of k-step s+1 are issued in
//            the shadow of k-step s's MFMAs (two fragment sets live at a time);
//            in the shadow of k-steps 0 and 1, the weight half of stage k+1's
//            loads into `nxt` (that slot's previous stage was retired by the
//            last barrier, and it is first read in phase B);
//   wait for this wave's loads of stage k+1; workgroup barrier (publishes
//   stage k+1 from every wave and retires `cur`: all of its fragments are in
//   registers now);
//   phase B: MFMAs of k-step 3; in their shadow the reads of k-step 0 of stage
//            k+1 and the gathered-row half of stage k+2's loads into `cur`.
// A stage's loads take about half of it at the unit's 64 bytes per clock; the
// split keeps that many loads from queueing behind one another in phase B,
// where each wave would stall at the issue of its next load and leave the
// matrix pipe idle.
// The hook (the in-tile copy of rows for later tiles) adds memory
// instructions to the stages: store<P>(k) and load<P>(k) right after the
// first MFMA of phase B (P = the stage's parity), in that MFMA's shadow, and
// mid(k) between phase A's wait for this wave's loads and its workgroup
// barrier, where the compiler waits for every memory operation anyway, so
// that what mid issues leaves nothing pending for the rest of the loop.
// Items that copy nothing run the loop with NoHook: with the copy's
// instructions issued empty in every stage the tile was 4-8 % slower.
struct NoHook {
  template <int P>
  __device__ __forceinline__ void store(int) {}
  template <int P>
  __device__ __forceinline__ void load(int) {}
  __device__ __forceinline__ void mid(int) {}
  __device__ __forceinline__ void finish() {}
};

// Phase A of stage k (in `cur`, its k-step 0 fragments in f0): the MFMAs of
// k-steps 0-2, the reads of k-steps 1-3 (f3 holds k-step 3's on return), the
// weight half of stage k+1's loads into `nxt_w` during k-steps 0 and 1; then
// (has_next) the wait for this wave's loads and the hook's mid, and the
// workgroup barrier, which publishes stage k+1 and retires `cur`.
template <int BM, int BN, bool has_next, class Hook>
__device__ __forceinline__ void phase_a(const char* cur, Frags<BM, BN>& f0, Frags<BM, BN>& f3, Acc<BM, BN>& acc,
                                        int wm, int wn, int lane, __amdgpu_buffer_rsrc_t rA, uint32_t a_off,
                                        __amdgpu_buffer_rsrc_t rB, uint32_t b_off, uint32_t stride,
                                        uint32_t k1_bytes, char* nxt_w, int wave, Hook& hook, int kst) {
  using T = Tile<BM, BN>;
  using KS = KStep<BM, BN>;
  constexpr int NM = KS::NM;               // MFMAs per k-step
  constexpr int LB0 = T::LOADS_B / 2;      // weight loads in k-step 0's shadow, the rest in k-step 1's
  using M0 = Mix<KS::nr(1), has_next ? LB0 : 0>;
  using M1 = Mix<KS::nr(2), has_next ? T::LOADS_B - LB0 : 0>;
  constexpr int NR3 = KS::nr(3);
  const char* curB = cur + T::A_BYTES;
  Frags<BM, BN> f1, f2;
  carry_weights<BM, BN>(f1, f0);
  // k-step 0 (reads k-step 1, weight loads of stage k+1)
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma_one<BM, BN, 0>(f0, acc, j);
#pragma unroll
    for (int o = (j * M0::OPS) / NM; o < ((j + 1) * M0::OPS) / NM; ++o) {
      if (M0::load(o)) stage_load_one<BM, BN>(rA, a_off, rB, b_off, stride, k1_bytes, nxt_w, wave, lane,
                                              T::LOADS_A + M0::index(o));
      else frag_read_one<BM, BN>(cur, curB, f1, 1, M0::index(o), wm, wn, lane);
    }
    FG_SCHED_FENCE();
  }
  // k-step 1 (reads k-step 2, the other weight loads of stage k+1)
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma_one<BM, BN, 1>(f1, acc, j);
#pragma unroll
    for (int o = (j * M1::OPS) / NM; o < ((j + 1) * M1::OPS) / NM; ++o) {
      if (M1::load(o)) stage_load_one<BM, BN>(rA, a_off, rB, b_off, stride, k1_bytes, nxt_w, wave, lane,
                                              T::LOADS_A + LB0 + M1::index(o));
      else frag_read_one<BM, BN>(cur, curB, f2, 2, M1::index(o), wm, wn, lane);
    }
    FG_SCHED_FENCE();
  }
  // k-step 2 (reads k-step 3)
  carry_weights<BM, BN>(f3, f2);
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma_one<BM, BN, 2>(f2, acc, j);
#pragma unroll
    for (int o = (j * NR3) / NM; o < ((j + 1) * NR3) / NM; ++o)
      frag_read_one<BM, BN>(cur, curB, f3, 3, o, wm, wn, lane);
    FG_SCHED_FENCE();
  }
  if constexpr (has_next) {
    wait_vmcnt<0>();
    hook.mid(kst);   // only after the wait for this wave's memory operations
  }
  __syncthreads();
}

// Phase B of stage k: the MFMAs of k-step 3 (f3); in their shadow the hook's
// copy instructions, the reads of k-step 0 of stage k+1 from `nxt` into f0
// (has_next) and the gathered-row half of stage k+2's loads into `cur_w`
// (refill), the slot phase A's barrier retired.
template <int BM, int BN, bool has_next, bool refill, int PAR, class Hook>
__device__ __forceinline__ void phase_b(const char* nxt, Frags<BM, BN>& f3, Frags<BM, BN>& f0, Acc<BM, BN>& acc,
                                        int wm, int wn, int lane, __amdgpu_buffer_rsrc_t rA, uint32_t a_off,
                                        __amdgpu_buffer_rsrc_t rB, uint32_t b_off, uint32_t stride,
                                        uint32_t k2_bytes, char* cur_w, int wave, Hook& hook, int kst) {
  using T = Tile<BM, BN>;
  using KS = KStep<BM, BN>;
  constexpr int NM = KS::NM;
  using MB = Mix<KS::nr(0), refill ? T::LOADS_A : 0>;
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma_one<BM, BN, 3>(f3, acc, j);
    if (j == 0) {
      FG_SCHED_FENCE();
      hook.template store<PAR>(kst);
      hook.template load<PAR>(kst);
      FG_SCHED_FENCE();
    }
#pragma unroll
    for (int o = (j * MB::OPS) / NM; o < ((j + 1) * MB::OPS) / NM; ++o) {
      if (MB::load(o)) stage_load_one<BM, BN>(rA, a_off, rB, b_off, stride, k2_bytes, cur_w, wave, lane, MB::index(o));
      else if constexpr (has_next) frag_read_one<BM, BN>(nxt, nxt + T::A_BYTES, f0, 0, MB::index(o), wm, wn, lane);
    }
    FG_SCHED_FENCE();
  }
}

// Ring stage of the 32-k variant: stage k in `cur`, its k-step 0 fragments in
// f0. Phase A: MFMAs of k-step 0, reads of k-step 1 in their shadow; wait
// until this wave's loads of stage k+1 are done (WAIT later stages may still be
// in flight), one workgroup barrier (publishes stage k+1, and every wave has
// read `cur`); phase B: MFMAs of k-step 1, in their shadow the reads of k-step
// 0 of stage k+1 and the refill of `cur` with stage k+4. Loads therefore lead
// their use by three stages.
template <int BM, int BN, bool has_next, bool refill, int WAIT>
__device__ __forceinline__ void stage_body4(const char* cur, const char* nxt, Frags<BM, BN>& f0, Acc<BM, BN>& acc,
                                            int wm, int wn, int lane, __amdgpu_buffer_rsrc_t rA, uint32_t a_off,
                                            __amdgpu_buffer_rsrc_t rB, uint32_t b_off, uint32_t stride,
                                            uint32_t k4_bytes, char* cur_w, int wave) {
  using T = Tile<BM, BN>;
  constexpr int NM = T::FM * T::FN;
  constexpr int NR = T::FM + T::FN;
  constexpr int OPS_B = NR + T::LOADS;
  const char* curB = cur + T::A_BYTES;
  Frags<BM, BN> f1;
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma_one<BM, BN>(f0, acc, j);
#pragma unroll
    for (int o = (j * NR) / NM; o < ((j + 1) * NR) / NM; ++o) frag_read_one<BM, BN>(cur, curB, f1, 1, o, wm, wn, lane);
    FG_SCHED_FENCE();
  }
  if constexpr (has_next) wait_vmcnt<WAIT * T::LOADS>();
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    mfma_one<BM, BN>(f1, acc, j);
#pragma unroll
    for (int o = (j * OPS_B) / NM; o < ((j + 1) * OPS_B) / NM; ++o) {
      if (o < NR) {
        if constexpr (has_next) frag_read_one<BM, BN>(nxt, nxt + T::A_BYTES, f0, 0, o, wm, wn, lane);
      } else {
        if constexpr (refill) stage_load_one<BM, BN>(rA, a_off, rB, b_off, stride, k4_bytes, cur_w, wave, lane, o - NR);
      }
    }
    FG_SCHED_FENCE();
  }
}

// --- ping-pong schedule ----------------------------------------------------
// The eight waves form two groups of four (group g = waves 4g .. 4g+3; with
// waves placed on the SIMDs in turn, every SIMD holds one wave of each group),
// and group g computes output rows [g BM/2, (g+1) BM/2) of the tile. Time is
// cut into phases ended by workgroup barriers; group 1 runs one phase behind
// group 0, so in every phase one group issues its MFMAs (16 per wave: two
// k-steps) while the other group reads the fragments of its next two k-steps
// from LDS and issues global->LDS loads. On each SIMD the matrix pipe is then
// fed by one wave while the other wave's memory instructions issue, instead of
// both waves interleaving both kinds.
// Stage t is read in phases 4t .. 4t+3 (group 0 halves in 4t and 4t+2, group 1
// in 4t+1 and 4t+3); the other slot, free from phase 4t on (stage t-1 was last
// read in 4t-1), is refilled with stage t+1 during stage t. Loads follow their
// readers: group 0 loads its own A rows and all of B in phase 4t, group 1 its
// own A rows in phase 4t+1; each wave waits for its loads after its last MFMAs
// of stage t, before the barrier that ends phase 4t+3 (group 0) or 4t+4
// (group 1), so every load leads its first reader by four or more phases.
// Every wave waits for its fragment reads before the barrier that ends its
// memory phase, so no slot is refilled while a read of it is outstanding.
constexpr int kWaitLgkm0 = 0xC07F;   // s_waitcnt immediate: lgkmcnt = 0, vmcnt and expcnt left alone

__device__ __forceinline__ void pp_barrier() {
  FG_SCHED_FENCE();
  __builtin_amdgcn_s_barrier();
  FG_SCHED_FENCE();
}

// Rows [r0, r0 + ROWS) of an operand for one stage, spread over the four
// waves of a group (w = wave index within the group).
template <int ROWS, int POL>
__device__ __forceinline__ void group_load(__amdgpu_buffer_rsrc_t r, uint32_t row0_off, uint32_t row_stride,
                                           uint32_t k0_bytes, char* lds, int r0, int w, int lane) {
  constexpr int PER_WAVE = ROWS / kRowsPerLoad / 4;
  static_assert(PER_WAVE >= 1 && ROWS % (kRowsPerLoad * 4) == 0, "group share");
  const int sub = lane / kChunks;
  const int slot = lane % kChunks;
#pragma unroll
  for (int q = 0; q < PER_WAVE; ++q) {
    const int blk = (r0 / kRowsPerLoad) + w * PER_WAVE + q;
    const int row = blk * kRowsPerLoad + sub;
    const int chunk = swz(slot, row);
    const uint32_t voff = row0_off + (uint32_t)row * row_stride + (uint32_t)chunk * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + blk * 1024), 16, voff, k0_bytes, 0, POL);
  }
}

// Stage t in `cur` (its loads complete and published); `nxt` is refilled with
// stage t+1 when `refill` (t >= 1: stage 1 comes with the prologue).
template <int BM, int BN>
__device__ __forceinline__ void pp_stage(const char* cur, char* nxt, bool refill, int grp, Acc<BM, BN>& acc, int wm,
                                         int wn, int lane, __amdgpu_buffer_rsrc_t rA, uint32_t a_off,
                                         __amdgpu_buffer_rsrc_t rB, uint32_t b_off, uint32_t stride,
                                         uint32_t k_bytes) {
  using T = Tile<BM, BN>;
  const char* curB = cur + T::A_BYTES;
  Frags<BM, BN> f0, f1;
  // memory: k-steps 0 and 1; this group's loads of stage t+1
  frags_read<BM, BN>(cur, curB, f0, 0, wm, wn, lane);
  frags_read<BM, BN>(cur, curB, f1, 1, wm, wn, lane);
  if (refill) {
    group_load<BM / 2, kPolA>(rA, a_off, stride, k_bytes, nxt, grp * (BM / 2), wn, lane);
    if (grp == 0) group_load<BN, 0>(rB, b_off, stride, k_bytes, nxt + T::A_BYTES, 0, wn, lane);
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  pp_barrier();
  // compute: k-steps 0 and 1
  frags_mfma<BM, BN>(f0, acc);
  frags_mfma<BM, BN>(f1, acc);
  pp_barrier();
  // memory: k-steps 2 and 3
  frags_read<BM, BN>(cur, curB, f0, 2, wm, wn, lane);
  frags_read<BM, BN>(cur, curB, f1, 3, wm, wn, lane);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  pp_barrier();
  // compute: k-steps 2 and 3, then this wave's loads of stage t+1
  frags_mfma<BM, BN>(f0, acc);
  frags_mfma<BM, BN>(f1, acc);
  if (refill) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  pp_barrier();
}

template <int BM, int BN>
__device__ __forceinline__ void tile_mainloop_pp(__amdgpu_buffer_rsrc_t rA, uint32_t a_off,
                                                 __amdgpu_buffer_rsrc_t rB, uint32_t b_off, uint32_t stride, int nk,
                                                 char* l0, char* l1, Acc<BM, BN>& acc) {
  using T = Tile<BM, BN>;
  static_assert(T::WGM == 2 && T::WGN == 4, "two groups of four waves, group = row half");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WGN, wn = wave % T::WGN;
  const int grp = wm;
  stage_load<BM, kPolA>(rA, a_off, stride, 0, l0, wave, lane);
  stage_load<BN, 0>(rB, b_off, stride, 0, l0 + T::A_BYTES, wave, lane);
  stage_load<BM, kPolA>(rA, a_off, stride, kRowB, l1, wave, lane);
  stage_load<BN, 0>(rB, b_off, stride, kRowB, l1 + T::A_BYTES, wave, lane);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  pp_barrier();
  if (grp == 1) pp_barrier();
  // nk is even; stage t lives in l0 for even t, l1 for odd t
  for (int t = 0; t < nk; t += 2) {
    pp_stage<BM, BN>(l0, l1, t >= 1 && t + 1 < nk, grp, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                     (uint32_t)(t + 1) * kRowB);
    pp_stage<BM, BN>(l1, l0, t + 2 < nk, grp, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                     (uint32_t)(t + 2) * kRowB);
  }
  if (grp == 0) pp_barrier();
}

// nk: k-iterations of 64 to run (even, >= 2) starting at the byte offsets
// a_off / b_off (which include the k origin); stride: row stride of both
// buffers in bytes (K * 2). l0..l3: the LDS stage buffers (distinct objects,
// so the compiler can tell them apart when it places its own waits); the
// 64-k variant uses l0 and l1.
// The rows' version words (tile_row_versions, loaded before the K loop) as
// one bit per word: bit v set = row word v is not the current route version
// (a padding row). Computed once the words have arrived, so that the words
// themselves do not hold registers through the K loop.
template <int BM, int BN>
__device__ __forceinline__ uint32_t pad_mask(const uint32_t (&ver_w)[Tile<BM, BN>::VW], uint32_t ver) {
  uint32_t m = 0;
#pragma unroll
  for (int v = 0; v < Tile<BM, BN>::VW; ++v) m |= (ver_w[v] != ver ? 1u : 0u) << v;
  return m;
}

// ver_w / ver: a whole tile's row version words and the route version, folded
// into `padmask` (pad_mask) once the first stage's loads, issued after the
// words, have arrived; split-K parts pass has_rows = false.
template <int BM, int BN, class Hook>
__device__ __forceinline__ void tile_mainloop(__amdgpu_buffer_rsrc_t rA, uint32_t a_off,
                                              __amdgpu_buffer_rsrc_t rB, uint32_t b_off, uint32_t stride, int nk64,
                                              char* l0, char* l1, char* l2, char* l3, Acc<BM, BN>& acc, Hook& hook,
                                              bool has_rows, const uint32_t (&ver_w)[Tile<BM, BN>::VW], uint32_t ver,
                                              uint32_t& padmask) {
  using T = Tile<BM, BN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WGN, wn = wave % T::WGN;
  Frags<BM, BN> f0;
  if constexpr (!(kBK == 64 && !kPingPong)) {
    if (has_rows) padmask = pad_mask<BM, BN>(ver_w, ver);
  }
  if constexpr (kBK == 64 && kPingPong) {
    tile_mainloop_pp<BM, BN>(rA, a_off, rB, b_off, stride, nk64, l0, l1, acc);
  } else if constexpr (kBK == 64) {
    const int nk = nk64;   // even
    char* const lds0 = l0;
    char* const lds1 = l1;
    // stage 0 whole, stage 1's gathered rows; its weight rows follow in stage 0's phase A
    stage_load<BM, kPolA>(rA, a_off, stride, 0, lds0, wave, lane);
    stage_load<BN, 0>(rB, b_off, stride, 0, lds0 + T::A_BYTES, wave, lane);
    stage_load<BM, kPolA>(rA, a_off, stride, kRowB, lds1, wave, lane);
    wait_vmcnt<T::LOADS_A>();
    __syncthreads();
    if (has_rows) padmask = pad_mask<BM, BN>(ver_w, ver);   // the words came before stage 0's loads
    frags_read_kstep<BM, BN>(lds0, lds0 + T::A_BYTES, f0, 0, wm, wn, lane);
    // Rotated so that every iteration ends with phase A's workgroup barrier,
    // before which the compiler waits for all memory operations: nothing the
    // copy hook issues in phase B is still in flight where the loop's paths
    // meet, which would make the compiler wait for every load at the top of
    // the next stage.
    Frags<BM, BN> f3;
    phase_a<BM, BN, true>(lds0, f0, f3, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, (uint32_t)1 * kRowB, lds1,
                          wave, hook, 0);
    int kt = 0;
    for (; kt < nk - 2; kt += 2) {
      phase_b<BM, BN, true, true, 0>(lds1, f3, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                                     (uint32_t)(kt + 2) * kRowB, lds0, wave, hook, kt);
      phase_a<BM, BN, true>(lds1, f0, f3, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                            (uint32_t)(kt + 2) * kRowB, lds0, wave, hook, kt + 1);
      phase_b<BM, BN, true, true, 1>(lds0, f3, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                                     (uint32_t)(kt + 3) * kRowB, lds1, wave, hook, kt + 1);
      phase_a<BM, BN, true>(lds0, f0, f3, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                            (uint32_t)(kt + 3) * kRowB, lds1, wave, hook, kt + 2);
    }
    // stages nk - 2 (phase A done) and nk - 1
    phase_b<BM, BN, true, false, 0>(lds1, f3, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, 0, lds0, wave,
                                    hook, nk - 2);
    phase_a<BM, BN, false>(lds1, f0, f3, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, 0, lds0, wave, hook,
                           nk - 1);
    phase_b<BM, BN, false, false, 1>(lds0, f3, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, 0, lds1, wave,
                                     hook, nk - 1);
  } else {
    const int nk = 2 * nk64;   // stages of 32 k; a multiple of 4
    char* const L[4] = {l0, l1, l2, l3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      stage_load<BM, kPolA>(rA, a_off, stride, (uint32_t)i * kRowB, L[i], wave, lane);
      stage_load<BN, 0>(rB, b_off, stride, (uint32_t)i * kRowB, L[i] + T::A_BYTES, wave, lane);
    }
    wait_vmcnt<3 * T::LOADS>();
    __syncthreads();
    frags_read<BM, BN>(l0, l0 + T::A_BYTES, f0, 0, wm, wn, lane);
    int kt = 0;
    for (; kt < nk - 4; kt += 4) {
      stage_body4<BM, BN, true, true, 2>(l0, l1, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                                         (uint32_t)(kt + 4) * kRowB, l0, wave);
      stage_body4<BM, BN, true, true, 2>(l1, l2, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                                         (uint32_t)(kt + 5) * kRowB, l1, wave);
      stage_body4<BM, BN, true, true, 2>(l2, l3, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                                         (uint32_t)(kt + 6) * kRowB, l2, wave);
      stage_body4<BM, BN, true, true, 2>(l3, l0, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride,
                                         (uint32_t)(kt + 7) * kRowB, l3, wave);
    }
    stage_body4<BM, BN, true, false, 2>(l0, l1, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, 0, l0, wave);
    stage_body4<BM, BN, true, false, 1>(l1, l2, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, 0, l1, wave);
    stage_body4<BM, BN, true, false, 0>(l2, l3, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, 0, l2, wave);
    stage_body4<BM, BN, false, false, 0>(l3, l0, f0, acc, wm, wn, lane, rA, a_off, rB, b_off, stride, 0, l3, wave);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // one v_cvt_pk_bf16_f32 (round to nearest even) for the pair
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Version words (the upper half of the inverse-map entry) of the rows this
// lane stores, loaded when the tile starts so that the store does not wait for
// them: row m is padding when its word is not the current route version.
template <int BM, int BN>
__device__ __forceinline__ void tile_row_versions(const unsigned long long* inv, int m0,
                                                  uint32_t (&ver_w)[Tile<BM, BN>::VW]) {
  using T = Tile<BM, BN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / T::WGN;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(inv);
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int g = 0; g < (kMfma16 ? 2 : 1); ++g)
      ver_w[acc_vw(fm, g)] = words[2 * (m0 + wm * T::WM + fm * 32 + acc_row(g, lane)) + 1];
}

// Direct store of the accumulators, 8 bytes per lane: rows as in tile_store,
// for the variants whose stage buffers cannot hold a wave block per wave.
template <int BM, int BN>
__device__ __forceinline__ void tile_store_direct(__amdgpu_buffer_rsrc_t rO, int N, int m0, int n0,
                                                  const Acc<BM, BN>& acc, uint32_t padmask) {
  using T = Tile<BM, BN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / T::WGN, wn = wave % T::WGN;
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = m0 + wm * T::WM + fm * 32 + acc_row(g, lane);
        const int n = n0 + wn * T::WN + fn * 32 + acc_col(g, lane);
        const bool pad = (padmask >> acc_vw(fm, g)) & 1;
        const f32x4 c = acc_group<BM, BN>(acc, fm, fn, g);
        v2i w;
        w[0] = pad ? 0 : (int)pack_bf16x2(c[0], c[1]);
        w[1] = pad ? 0 : (int)pack_bf16x2(c[2], c[3]);
        __builtin_amdgcn_raw_buffer_store_b64(w, rO, (uint32_t)m * (uint32_t)N * 2 + (uint32_t)n * 2, 0, 0);
      }
    }
  }
}

// Store the tile: padding rows (no current inverse-map entry) are written as zeros.
// rO: output rows [*, N] (row stride N*2 bytes); m0, n0: tile origin; padmask:
// the rows' padding bits (pad_mask); l0, l1: the two LDS stage
// buffers, free once the K loop's last barrier has passed (waves 0-3 use l0,
// waves 4-7 l1).
//
// A lane's accumulators hold 4 consecutive columns of one row per register
// group, so stored directly every 8-byte store instruction would touch 32
// rows (32 partial lines). Instead each wave rounds its (BM/2) x (BN/4) block to
// bf16 into a private LDS block and reads it back with BN/32 lanes per row:
// every global store instruction then writes whole rows of the wave's block
// (8 x 128 bytes for BN = 256).
// LDS block: one 32-row sub-block per fragment row fm, rows of BN/2 bytes;
// logical 16-byte chunk c of row r sits in slot c ^ ((r / (256 / row bytes)) &
// (chunks - 1)) as in swz, and in rows 16..31 the two 8-byte halves of every
// chunk trade places. A write instruction (half-wave passes of 32 rows x 8
// bytes of one chunk) then covers all 64 banks once, and a read pass (16 lanes
// x 16 bytes) covers whole rows in distinct bank ranges. The rows of one read
// are all below or all above row 16, so its halves are swapped back by the
// choice of registers. Where a stage buffer cannot hold four waves' blocks
// (the 32-k variant), the waves reuse one 32-row sub-block: LDS operations of
// one wave complete in issue order, which keeps the reuse safe. The stage
// buffers are next written by the following item's loads, after the
// scheduler's workgroup barrier.
template <int BM, int BN>
__device__ __forceinline__ void tile_store(__amdgpu_buffer_rsrc_t rO, int N, int m0, int n0,
                                           const Acc<BM, BN>& acc, uint32_t padmask, char* l0, char* l1) {
  using T = Tile<BM, BN>;
  constexpr int RB = T::WN * 2;          // bytes per row of the wave's block
  constexpr int CPR = RB / 16;           // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;          // rows per 64-lane 16-byte access
  constexpr int D = 256 / RB;            // rows per 256-byte bank period
  constexpr int SUB = 32 * RB;           // bytes of one 32-row sub-block
  constexpr int NSUB = 4 * T::FM * SUB <= Tile<256, BN>::STAGE ? T::FM : 1;
  if constexpr (kWaves != 8 || 4 * SUB > Tile<256, BN>::STAGE) {
    tile_store_direct<BM, BN>(rO, N, m0, n0, acc, padmask);   // the 4-wave variant
  } else {
    static_assert(RPI == 8 || RPI == 16, "read-back rows per access");
    // the lane's offsets are computed here, not hoisted out of the tile loop,
    // where they would hold registers through the K loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / T::WGN, wn = wave % T::WGN;
    const int lr = lane & 31, kh = lane >> 5;
    char* const blk = (wave < 4 ? l0 : l1) + (wave & 3) * (NSUB * SUB);
    const int sw = ((lr / D) & (CPR - 1)) * 16;                   // write: slot permutation of row lr
    char* const wrow = blk + lr * RB + (kh ^ (lr >> 4)) * 8;
    const int rr = lane / CPR, rc = lane % CPR;                   // read: row within the access, chunk
    // read offset of row i * RPI + rr, chunk rc: the row's slot permutation is
    // (rr / D) xor a constant of i ((i * RPI / D) & (CPR - 1))
    const int rslot = rc ^ (rr / D);
    const int rbase = rr * RB;
    const uint32_t row_bytes = (uint32_t)N * 2;
    const uint32_t out_lane = (uint32_t)(m0 + wm * T::WM + rr) * row_bytes + (uint32_t)(n0 + wn * T::WN + rc * 8) * 2;
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm) {
      if constexpr (kMfma16) {
        // group g of lane l: row r = 16 (g & 1) + l % 16 of the sub-block,
        // columns c0 .. c0 + 3 with c0 = 16 (g >> 1) + 4 (l / 16) in each
        // column block: 16-byte chunk fn * 4 + c0 / 8, 8-byte half (c0 / 4) & 1
        // (swapped in rows 16-31), the chunk's slot permuted as in swz. A
        // half-wave writes 16 rows x 16 bytes: all 64 banks once.
        char* const sub = blk + (fm % NSUB) * SUB;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = acc_row(g, lane), c0 = acc_col(g, lane);
          const bool pad = (padmask >> acc_vw(fm, g)) & 1;   // versioned inverse map: stale = padding
          char* const row = sub + r * RB + ((((c0 >> 2) & 1) ^ (r >> 4)) * 8);
          const int rsw = ((r / D) & (CPR - 1)) * 16;
#pragma unroll
          for (int fn = 0; fn < T::FN; ++fn) {
            const f32x4 c = acc_group<BM, BN>(acc, fm, fn, g);
            v2i w;
            w[0] = pad ? 0 : (int)pack_bf16x2(c[0], c[1]);
            w[1] = pad ? 0 : (int)pack_bf16x2(c[2], c[3]);
            *reinterpret_cast<v2i*>(row + (((fn * 4 + (c0 >> 3)) * 16) ^ rsw)) = w;
          }
        }
      } else {
        char* const sub = wrow + (fm % NSUB) * SUB;
        const bool pad = (padmask >> fm) & 1;   // versioned inverse map: stale = padding
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 c = acc_group<BM, BN>(acc, fm, fn, g);
            v2i w;
            w[0] = pad ? 0 : (int)pack_bf16x2(c[0], c[1]);
            w[1] = pad ? 0 : (int)pack_bf16x2(c[2], c[3]);
            *reinterpret_cast<v2i*>(sub + (((fn * 4 + g) * 16) ^ sw)) = w;
          }
        }
      }
      if constexpr (NSUB == T::FM) {
        if (fm + 1 < T::FM) continue;   // all blocks written: read them back below
      }
      constexpr int F0 = NSUB == T::FM ? 0 : -1;   // first fragment row to read back
#pragma unroll
      for (int f = (F0 < 0 ? fm : 0); f <= fm; ++f) {
        v4i x[32 / RPI];
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int k = (i * RPI / D) & (CPR - 1);
          x[i] = *reinterpret_cast<const v4i*>(blk + (f % NSUB) * SUB + i * RPI * RB + rbase + (rslot ^ k) * 16);
        }
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const bool swapped = ((i * RPI) >> 4) & 1;
          const v4i v = swapped ? v4i{x[i][2], x[i][3], x[i][0], x[i][1]} : x[i];
          // the whole offset goes in the VGPR operand, soffset stays 0: a
          // 16-byte store with a register soffset, followed at once by a VALU
          // write of its data registers, stored the new values in some lanes
          // (measured), and the compiler guards that hazard only for a
          // constant soffset
          __builtin_amdgcn_raw_buffer_store_b128(v, rO, out_lane + (uint32_t)(f * 32 + i * RPI) * row_bytes, 0, 0);
        }
      }
    }
  }
}

// --- split-K partial sums ------------------------------------------------
// A tile's partial sum is kept in register order: for wave w and fragment f,
// 16 floats per lane as four 1 KB rows (64 lanes x 16 bytes), so every store
// and load is one fully coalesced 16-byte-per-lane access. One part's block is
// BM * BN * 4 bytes.
template <int BM, int BN>
__device__ __forceinline__ uint32_t partial_off(int wave, int f, int g, int lane) {
  using T = Tile<BM, BN>;
  return (uint32_t)((((wave * (T::FM * T::FN) + f) * 4 + g) * 64 + lane) * 16);
}

// Store all of this part's fragments into its block at byte offset `base`,
// with device-coherent write-through stores (the accumulators are only read).
template <int BM, int BN>
__device__ __forceinline__ void partial_store(__amdgpu_buffer_rsrc_t rW, uint32_t base, const Acc<BM, BN>& acc) {
  using T = Tile<BM, BN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) {
      const int f = fm * T::FN + fn;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // whole-vector bit casts only: a bit cast of a vector element lvalue
        // reads element 0 with this compiler
        const f32x4 x = acc_group<BM, BN>(acc, fm, fn, g);
        store16_coherent(rW, base + partial_off<BM, BN>(wave, f, g, lane), __builtin_bit_cast(v4i, x));
      }
    }
}

// For the fragments this part owns (f % P == part): sum the P partials in
// part order 0..P-1, round to bf16 and store them as tile_store does. The
// order of the fp32 additions is fixed, so the result does not depend on
// which workgroup ran which part. `base` = byte offset of part 0's block;
// blocks are `tile_bytes` apart. Loads use the device-coherent policy: the
// blocks were written by other workgroups, possibly on other XCDs.
template <int BM, int BN>
__device__ __forceinline__ void partial_sum_store(__amdgpu_buffer_rsrc_t rW, uint32_t base, uint32_t tile_bytes,
                                                  int part, int P, __amdgpu_buffer_rsrc_t rO, int N, int m0, int n0,
                                                  const unsigned long long* inv, uint32_t ver) {
  using T = Tile<BM, BN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WGN, wn = wave % T::WGN;
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) {
      const int f = fm * T::FN + fn;
      if (f % P != part) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = m0 + wm * T::WM + fm * 32 + acc_row(g, lane);
        const bool pad = (uint32_t)(inv[m] >> 32) != ver;
        const uint32_t row_off = (uint32_t)m * (uint32_t)N * 2;
        // eight independent loads first (their latencies overlap); those of
        // parts q >= P point past the end of the buffer, where the buffer
        // unit returns zeros; then the sum in part order
        const uint32_t o = partial_off<BM, BN>(wave, f, g, lane);
        f32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          v[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rW, q < P ? base + (uint32_t)q * tile_bytes + o : 0xFFFFFFF0u, 0,
                                               kPolCoherentStore));
        f32x4 sum = v[0];
#pragma unroll
        for (int q = 1; q < 8; ++q) sum += v[q];
        const int n = n0 + wn * T::WN + fn * 32 + acc_col(g, lane);
        v2i w;
        w[0] = pad ? 0 : (int)pack_bf16x2(sum[0], sum[1]);
        w[1] = pad ? 0 : (int)pack_bf16x2(sum[2], sum[3]);
        __builtin_amdgcn_raw_buffer_store_b64(w, rO, row_off + (uint32_t)n * 2, 0, 0);
      }
    }
  }
}

}  // namespace fg
