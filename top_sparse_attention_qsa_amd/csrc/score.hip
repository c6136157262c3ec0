// score.hip -- step 1: group scores for every complete group of every row.
//
// score(g) = sum over index heads h (ascending, from +0) of ReLU(dot_h), where
// dot_h is a chain of fused multiply-adds over d ascending from +0 (AFN-016 "A
// sparse mask is not sparse attention", §Decision and §Why a sparse mask can
// still be dense: ReLU per head, then the head sum).  The order is fixed so
// scores are bit-reproducible and equal ties stay equal wherever a group
// falls in a tile.
//
// Mapping: one lane owns one group.  A wavefront owns kScoreTilesPerWave
// pooled-key tiles of 64 groups; in the tiled layout, dimension chunk c of a
// tile is 1 KiB contiguous, so each float4 load of the wave is one coalesced
// 1 KiB read.  The index query is uniform across the workgroup and is read
// with scalar loads into SGPRs, so the fma operand costs no LDS or VALU work.
// The workload is HBM-bound: 8 flop per pooled-key byte.
#include "qsa_internal.h"

namespace qsa {
namespace {

template <int HI, int DI, int TPW>
__global__ void __launch_bounds__(kScoreWaves * kWave)
score_kernel(const float* __restrict__ index_q, const float* __restrict__ pooled,
             const int64_t* __restrict__ pooled_off, const int32_t* __restrict__ seq_len,
             int32_t queries, int64_t g_max, int64_t row0, float* __restrict__ scores,
             uint32_t* __restrict__ maxima) {
  const int64_t lrow = blockIdx.y;
  const int64_t row = row0 + lrow;
  const RowView rv = row_view(seq_len, row, queries, g_max);
  if (!rv.valid) return;
  const int wave = (int)(threadIdx.x / kWave);
  const int lane = lane_id();
  const int64_t tiles = (rv.g + 63) >> 6;
  const int64_t t0 = ((int64_t)blockIdx.x * kScoreWaves + wave) * TPW;
  if (t0 >= tiles) return;

  const float* __restrict__ qrow = index_q + row * (int64_t)(HI * DI);
  const float* __restrict__ kbase = pooled + pooled_off[rv.b] + t0 * (64 * DI) + lane * 4;

  bool tile_ok[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) tile_ok[i] = (t0 + i) < tiles;

  float acc[TPW][HI];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int h = 0; h < HI; ++h) acc[i][h] = 0.0f;

  // Register ring of PF dimension chunks per tile: the load of chunk c+PF is
  // issued as soon as chunk c has been taken out of its slot, so PF x TPW
  // KiB per wavefront stay in flight while the fma chains run.
  constexpr int NC = DI / 4;
  constexpr int PF = NC < 4 ? NC : 4;
  float4 ring[PF][TPW];
#pragma unroll
  for (int u = 0; u < PF; ++u)
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      ring[u][i] = tile_ok[i]
                       ? *reinterpret_cast<const float4*>(kbase + (int64_t)i * (64 * DI) + u * 256)
                       : make_float4(0.f, 0.f, 0.f, 0.f);

#pragma unroll 1
  for (int cb = 0; cb < NC; cb += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int c = cb + u;
      float4 kv[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i) kv[i] = ring[u][i];
      if (c + PF < NC) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
          if (tile_ok[i])
            ring[u][i] = *reinterpret_cast<const float4*>(kbase + (int64_t)i * (64 * DI) +
                                                          (c + PF) * 256);
      }
      const float* __restrict__ qc = qrow + 4 * c;
#pragma unroll
      for (int h = 0; h < HI; ++h) {
        const float q0 = qc[h * DI + 0];
        const float q1 = qc[h * DI + 1];
        const float q2 = qc[h * DI + 2];
        const float q3 = qc[h * DI + 3];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          float a = acc[i][h];
          a = __builtin_fmaf(q0, kv[i].x, a);
          a = __builtin_fmaf(q1, kv[i].y, a);
          a = __builtin_fmaf(q2, kv[i].z, a);
          a = __builtin_fmaf(q3, kv[i].w, a);
          acc[i][h] = a;
        }
      }
    }
  }

  float* __restrict__ srow = scores + lrow * g_max;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (!tile_ok[i]) break;
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < HI; ++h) s = s + (acc[i][h] > 0.0f ? acc[i][h] : 0.0f);
    const int64_t g = (t0 + i) * 64 + lane;
    const bool ok = g < rv.g;
    if (ok) srow[g] = s;
    if (maxima) {
      // maximum order key of the 16 consecutive groups sharing this DPP row
      uint32_t m = ok ? order_key(s) : 0u;
#pragma unroll
      for (int o = kSegment / 2; o > 0; o >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)m, o, kWave);
        m = m > y ? m : y;
      }
      if ((lane & (kSegment - 1)) == 0 && ok)
        maxima[lrow * (g_max / kSegment) + g / kSegment] = m;
    }
  }
}

__global__ void __launch_bounds__(256)
segment_maxima_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seq_len,
                      int32_t queries, int64_t g_max, int64_t row0,
                      uint32_t* __restrict__ maxima) {
  const int64_t lrow = blockIdx.y;
  const RowView rv = row_view(seq_len, row0 + lrow, queries, g_max);
  if (!rv.valid) return;
  const int64_t seg = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g0 = seg * kSegment;
  if (g0 >= rv.g) return;
  const float* __restrict__ srow = scores + lrow * g_max;
  uint32_t m = 0;
  for (int e = 0; e < kSegment; ++e) {
    const int64_t g = g0 + e;
    if (g < rv.g) {
      const uint32_t k = order_key(srow[g]);
      m = m > k ? m : k;
    }
  }
  maxima[lrow * (g_max / kSegment) + seg] = m;
}

template <int HI, int DI>
hipError_t launch_score_t(const ScoreArgs& a, hipStream_t s) {
  const int64_t tiles = (a.g_max + 63) / 64;
  const int64_t per_block = (int64_t)kScoreWaves * kScoreTilesPerWave;
  dim3 grid((unsigned)((tiles + per_block - 1) / per_block), (unsigned)a.rows);
  if (grid.x == 0 || a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL((score_kernel<HI, DI, kScoreTilesPerWave>), grid,
                     dim3(kScoreWaves * kWave), 0, s, a.index_q, a.pooled, a.pooled_off,
                     a.seq_len, a.queries, a.g_max, a.row0, a.scores, a.maxima);
  return hipGetLastError();
}

template <int HI>
hipError_t launch_score_h(const ScoreArgs& a, int d_i, hipStream_t s) {
  switch (d_i) {
    case 32: return launch_score_t<HI, 32>(a, s);
    case 64: return launch_score_t<HI, 64>(a, s);
    case 128: return launch_score_t<HI, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int h_i, int d_i, hipStream_t s) {
  switch (h_i) {
    case 1: return launch_score_h<1>(a, d_i, s);
    case 2: return launch_score_h<2>(a, d_i, s);
    case 4: return launch_score_h<4>(a, d_i, s);
    case 8: return launch_score_h<8>(a, d_i, s);
    case 16: return launch_score_h<16>(a, d_i, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_segment_maxima(const float* scores, const int32_t* seq_len, int32_t queries,
                                 int64_t g_max, int64_t row0, int64_t rows, uint32_t* maxima,
                                 hipStream_t s) {
  const int64_t segs = g_max / kSegment;
  dim3 grid((unsigned)((segs + 255) / 256), (unsigned)rows);
  if (grid.x == 0 || rows == 0) return hipSuccess;
  hipLaunchKernelGGL(segment_maxima_kernel, grid, dim3(256), 0, s, scores, seq_len, queries,
                     g_max, row0, maxima);
  return hipGetLastError();
}

}  // namespace qsa
