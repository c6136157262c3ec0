// qsa_device.h -- constants and device helpers shared by the HIP kernels of
// libqsa.so (gfx950, wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_launch.h"

namespace qsa {

constexpr int kWave = 64;
constexpr int kScoreWaves = 4;        // waves (one 64-group tile each) per scoring workgroup
constexpr int kSelectThreads = 1024;  // one selection workgroup per row
constexpr int kCandCap = 4096;        // candidates kept in LDS before the streaming path
constexpr int kGatherTokens = 8;      // compact rows per gather workgroup

// Residency caps for the streaming kernels.  With fewer wavefronts per SIMD
// than registers would admit, the pooled-key sweep and the pooling read HBM
// faster (measured on this part); a launch caps residency by reserving LDS,
// a 1/wgs_per_cu share of the compute unit's 160 KiB per workgroup, less
// what the kernel declares itself.
constexpr int kLdsPerCu = 160 * 1024;
constexpr int lds_reserve(int wgs_per_cu, int static_bytes) {
  return kLdsPerCu / wgs_per_cu - static_bytes;
}

// Scores are ordered through a monotone unsigned key: -0 is folded onto +0,
// then non-negative floats get their sign bit set and negative floats are
// bit-inverted, so unsigned comparison equals float comparison.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct RowView {
  int64_t n;     // visible tokens
  int64_t g;     // complete groups
  int32_t tail;  // n mod 4
  int32_t b;     // sequence
  bool valid;
};

__device__ __forceinline__ RowView row_view(const int32_t* __restrict__ seq_len, int64_t row,
                                            int32_t queries, int64_t g_max) {
  RowView v;
  v.b = (int32_t)(row / queries);
  const int32_t j = (int32_t)(row - (int64_t)v.b * queries);
  v.n = (int64_t)seq_len[v.b] - queries + 1 + j;
  v.valid = v.n >= 0;
  v.g = v.valid ? (v.n >> 2) : 0;
  v.tail = v.valid ? (int32_t)(v.n & 3) : 0;
  if (v.g > g_max) v.valid = false;
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Index of this wavefront within its workgroup, as a value the compiler knows
// to be uniform (so addresses derived from it use scalar loads).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the wavefront's 64 lanes, on the VALU: steps of
// 1, 2, 4 and 8 lanes inside each 16-lane DPP row (row_shr; a lane shifted in
// from outside the row reads 0), then every row adds the totals of the rows
// below it, read from their last lanes.  Integer sums, exact in any order.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane_id() >> 4;
  return v + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

// Value of `v` in lane `lane` (uniform across the wavefront), on the VALU.
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Wavefront reductions.  Within each 16-lane DPP row, rotations by 1, 2, 4
// and 8 lanes (row_ror) leave every lane holding its row's reduction; lane 0
// of each row is then read into a scalar and the four rows are combined as
// (r0 op r1) op (r2 op r3).  The order is fixed, so a sum is the same bits on
// every run and the result is uniform across the wavefront.  DPP stays in
// the VALU: no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kRowRor1>(v));
  v = fmaxf(v, dpp_f32<kRowRor2>(v));
  v = fmaxf(v, dpp_f32<kRowRor4>(v));
  v = fmaxf(v, dpp_f32<kRowRor8>(v));
  return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}

// Maximum over the 16 lanes of this lane's DPP row (every lane of the row
// receives it; exact, so all agree).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<kRowRor1>(v));
  v = fmaxf(v, dpp_f32<kRowRor2>(v));
  v = fmaxf(v, dpp_f32<kRowRor4>(v));
  v = fmaxf(v, dpp_f32<kRowRor8>(v));
  return v;
}

// Sum over the 16 lanes of this lane's DPP row.  Lanes associate the terms in
// different orders, so only one fixed lane's value is used.
__device__ __forceinline__ float row_sum16(float v) {
  v = v + dpp_f32<kRowRor1>(v);
  v = v + dpp_f32<kRowRor2>(v);
  v = v + dpp_f32<kRowRor4>(v);
  v = v + dpp_f32<kRowRor8>(v);
  return v;
}

// Unsigned maximum over the 16 lanes of this lane's DPP row (every lane of the
// row receives it).
__device__ __forceinline__ uint32_t row_max16_u32(uint32_t v) {
  uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor1, 0xF, 0xF, false);
  v = v > y ? v : y;
  y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor2, 0xF, 0xF, false);
  v = v > y ? v : y;
  y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor4, 0xF, 0xF, false);
  v = v > y ? v : y;
  y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor8, 0xF, 0xF, false);
  return v > y ? v : y;
}

// Unsigned sum and maximum over the wavefront; every lane receives them.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return lane_value(wave_inclusive_sum(v), kWave - 1);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  const uint32_t r = row_max16_u32(v);
  const uint32_t a = lane_value(r, 0), b = lane_value(r, 16), c = lane_value(r, 32),
                 d = lane_value(r, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Butterfly steps across 16-lane rows and 32-lane halves on the VALU (gfx950
// v_permlane16_swap / v_permlane32_swap).  Swapping a value with itself
// leaves, in every lane, the pair (x of the lane, x of the lane 16 -- resp. 32
// -- positions away), lower-row value first in both lanes of the pair, so
// op(first, second) gives both lanes the same bits.
template <class Op>
__device__ __forceinline__ float xor16(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class Op>
__device__ __forceinline__ float xor32(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};

__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_f32<kRowRor1>(v);
  v = v + dpp_f32<kRowRor2>(v);
  v = v + dpp_f32<kRowRor4>(v);
  v = v + dpp_f32<kRowRor8>(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// Exclusive prefix sum over a whole workgroup of NT threads (NT/64 waves);
// `wave_tot` is LDS scratch of NT/64 words.  *total receives the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t x, uint32_t* wave_tot,
                                                        uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int wave = (int)(threadIdx.x / kWave);
  const uint32_t inc = wave_inclusive_sum(x);
  if (lane_id() == kWave - 1) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = wave_tot[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - x;
}

}  // namespace qsa
