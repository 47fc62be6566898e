// bf16 x bf16 -> fp32 MFMA tile for gfx950, LDS-staged, two-stage pipeline.
//
// The contraction is the dense GEMM the compute workgroups run once a row
// block's gate opens (the GEMM behind the gate of "PCIe sync protocols" §5):
//   out[m][n] = sum_k A[m][k] * W[k][n],  A = gathered rows (bf16, K contiguous),
//   W stored as [N][K] (K contiguous), fp32 accumulation, bf16 RNE output.
//
// Tile BM x BN, four waves as 2 x 2, each wave (BM/2) x (BN/2) built from
// v_mfma_f32_32x32x16_bf16 fragments. The weight tile is the MFMA "A" operand
// and the gathered tile the "B" operand, so that each lane's four consecutive
// accumulator values are four consecutive output columns of one row (8-byte
// stores). Lane layout (measured on the part): A/B operand lane l holds row/col
// l % 32 and k = 8 * (l / 32) + 0..7; result register v of lane l is
// D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32].
//
// LDS: per stage, each operand tile is stored as rows of 64 k (128 bytes =
// 8 slots of 16 bytes); logical 16-byte chunk c of row r sits in slot
// c ^ (r & 7), so the 8 lanes of a ds_read_b128 phase hit 8 distinct slots.
// Global -> LDS moves use buffer_load ... lds (16 bytes per lane, lane i writes
// base + 16 i), so the swizzle is applied by choosing which chunk a lane fetches.
#pragma once

#include "fg_sync.hpp"

namespace fg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;             // k per LDS stage
constexpr int kRowB = kBK * 2;      // bytes per tile row per stage

template <int BM, int BN>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * kRowB;
  static constexpr int B_BYTES = BN * kRowB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LOADS_A = BM / 32;   // buffer_load_lds per wave per stage for A
  static constexpr int LOADS_B = BN / 32;
  static constexpr int LOADS = LOADS_A + LOADS_B;
};

typedef __attribute__((address_space(3))) void lds_void;

// Issue this wave's share of one stage: `rows` rows starting at byte offset
// `row0_off` of the buffer, k slice [k0, k0 + 64), into LDS at `lds`.
template <int ROWS>
__device__ __forceinline__ void stage_load(__amdgpu_buffer_rsrc_t r, uint32_t row0_off, uint32_t row_stride,
                                           uint32_t k0_bytes, char* lds, int wave, int lane) {
  constexpr int PER_WAVE = ROWS / 32;  // instructions of 8 rows each
  const int sub = lane >> 3;           // row within the 8-row instruction block
  const int slot = lane & 7;
  const int chunk = slot ^ sub;        // (row & 7) == sub
#pragma unroll
  for (int q = 0; q < PER_WAVE; ++q) {
    const int blk = wave * PER_WAVE + q;
    const int row = blk * 8 + sub;
    const uint32_t voff = row0_off + (uint32_t)row * row_stride + k0_bytes + (uint32_t)chunk * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + blk * 1024), 16, voff, 0, 0, 0);
  }
}

// One 16-byte operand fragment: row `row` (multiple-of-32 base + lane % 32), k
// chunk c (0..7) of the stage.
__device__ __forceinline__ bf16x8 frag_read(const char* lds, int row, int c) {
  const int slot = c ^ (row & 7);
  return *reinterpret_cast<const bf16x8*>(lds + row * kRowB + slot * 16);
}

template <int BM, int BN>
struct Acc {
  f32x16 v[Tile<BM, BN>::FM][Tile<BM, BN>::FN];
};

template <int BM, int BN>
struct Frags {
  bf16x8 b[Tile<BM, BN>::FN];
  bf16x8 a[Tile<BM, BN>::FM];
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

// One LDS stage (64 k = 4 MFMA k-steps). The fragments of k-step kk+1 are
// issued before the MFMAs of k-step kk (two fragment sets in registers), with
// scheduling fences so the compiler keeps that order; the MFMAs of one k-step
// write distinct accumulators and pipeline back to back.
template <int BM, int BN>
__device__ __forceinline__ void stage_compute(const char* ldsA, const char* ldsB, Acc<BM, BN>& acc, int wm, int wn,
                                              int lane) {
  Frags<BM, BN> f0, f1;
  frags_read<BM, BN>(ldsA, ldsB, f0, 0, wm, wn, lane);
#pragma unroll
  for (int kk = 0; kk < kBK / 16; kk += 2) {
    frags_read<BM, BN>(ldsA, ldsB, f1, kk + 1, wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
    frags_mfma<BM, BN>(f0, acc);
    __builtin_amdgcn_sched_barrier(0);
    if (kk + 2 < kBK / 16) frags_read<BM, BN>(ldsA, ldsB, f0, kk + 2, wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
    frags_mfma<BM, BN>(f1, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Full K loop for one tile (K a multiple of 128). rA: gathered rows (row stride
// K*2 bytes), a_off = byte offset of the tile's first row; rB: weight rows
// [N][K], b_off likewise. lds0/lds1: the two stage buffers. Each stage is
// loaded one stage ahead; one workgroup barrier per stage both publishes the
// stage just landed and retires the stage just read.
template <int BM, int BN>
__device__ __forceinline__ void tile_mainloop(__amdgpu_buffer_rsrc_t rA, uint32_t a_off,
                                              __amdgpu_buffer_rsrc_t rB, uint32_t b_off, int K,
                                              char* lds0, char* lds1, Acc<BM, BN>& acc) {
  using T = Tile<BM, BN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t stride = (uint32_t)K * 2;
  const int nk = K / kBK;   // even
  stage_load<BM>(rA, a_off, stride, 0, lds0, wave, lane);
  stage_load<BN>(rB, b_off, stride, 0, lds0 + T::A_BYTES, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  stage_load<BM>(rA, a_off, stride, kRowB, lds1, wave, lane);
  stage_load<BN>(rB, b_off, stride, kRowB, lds1 + T::A_BYTES, wave, lane);
  for (int kt = 0; kt < nk; kt += 2) {
    stage_compute<BM, BN>(lds0, lds0 + T::A_BYTES, acc, wm, wn, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 2 < nk) {
      stage_load<BM>(rA, a_off, stride, (uint32_t)(kt + 2) * kRowB, lds0, wave, lane);
      stage_load<BN>(rB, b_off, stride, (uint32_t)(kt + 2) * kRowB, lds0 + T::A_BYTES, wave, lane);
    }
    stage_compute<BM, BN>(lds1, lds1 + T::A_BYTES, acc, wm, wn, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 3 < nk) {
      stage_load<BM>(rA, a_off, stride, (uint32_t)(kt + 3) * kRowB, lds1, wave, lane);
      stage_load<BN>(rB, b_off, stride, (uint32_t)(kt + 3) * kRowB, lds1 + T::A_BYTES, wave, lane);
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 l = (__bf16)lo, h = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// Store the tile: rows whose pad mask bit is set are written as zeros.
// rO: output rows [*, N] (row stride N*2 bytes); m0, n0: tile origin.
template <int BM, int BN>
__device__ __forceinline__ void tile_store(__amdgpu_buffer_rsrc_t rO, int N, int m0, int n0,
                                           const Acc<BM, BN>& acc, const int* pad_rows_info) {
  using T = Tile<BM, BN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm) {
    const int m = m0 + wm * T::WM + fm * 32 + lr;
    const bool pad = pad_rows_info[m] < 0;
    const uint32_t row_off = (uint32_t)m * (uint32_t)N * 2;
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * T::WN + fn * 32 + 8 * g + 4 * kh;
        const f32x16& c = acc.v[fm][fn];
        v2i w;
        w[0] = pad ? 0 : (int)pack_bf16x2(c[4 * g + 0], c[4 * g + 1]);
        w[1] = pad ? 0 : (int)pack_bf16x2(c[4 * g + 2], c[4 * g + 3]);
        __builtin_amdgcn_raw_buffer_store_b64(w, rO, row_off + (uint32_t)n * 2, 0, kPolNT);
      }
    }
  }
}

}  // namespace fg
