// score.hip -- step 1: group scores for every complete group of every row.
//
// score(g) = sum over index heads h (ascending, from +0) of ReLU(dot_h), where
// dot_h is a chain of fused multiply-adds over d ascending from +0 (AFN-016 "A
// sparse mask is not sparse attention", §Decision and §Why a sparse mask can
// still be dense: ReLU per head, then the head sum).  The order is fixed so
// scores are bit-reproducible and equal ties stay equal wherever a group
// falls in a tile.
//
// Mapping: one lane owns one group and a wavefront owns one pooled-key tile of
// 64 groups; in the tiled layout, dimension chunk c of a tile is 1 KiB
// contiguous, so each float4 load of the wave is one coalesced 1 KiB read.  The index query is uniform across the workgroup and is read
// with scalar loads into SGPRs, so the fma operand costs no LDS or VALU work.
// The workload is HBM-bound: 8 flop per pooled-key byte.
#include "qsa_internal.h"

namespace qsa {
namespace {

// Pooled keys are read once per step, so they are loaded with the
// nontemporal hint and do not displace the scores or other live data in L2.
__device__ __forceinline__ float4 load_stream(const float* p) {
  typedef float v4 __attribute__((ext_vector_type(4)));
  const v4 v = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

template <int HI, int DI>
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
  const int64_t tile = (int64_t)blockIdx.x * kScoreWaves + wave;  // 64 groups per wavefront
  if (tile * 64 >= rv.g) return;

  const float* __restrict__ qrow = index_q + row * (int64_t)(HI * DI);
  const float* __restrict__ kbase = pooled + pooled_off[rv.b] + tile * (64 * DI) + lane * 4;

  float acc[HI];
#pragma unroll
  for (int h = 0; h < HI; ++h) acc[h] = 0.0f;

  // Register ring of PF dimension chunks: the load of chunk c+PF is issued as
  // soon as chunk c leaves its slot.  A shallow ring keeps the register count
  // low enough for 7-8 resident wavefronts per SIMD, which hides the memory
  // latency better than a deeper ring at lower occupancy (measured).
  constexpr int NC = DI / 4;
  constexpr int PF = 2;
  static_assert(NC % PF == 0, "ring depth must divide the chunk count");
  float4 ring[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) ring[u] = load_stream(kbase + u * 256);

#pragma unroll 1
  for (int cb = 0; cb < NC; cb += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int c = cb + u;
      const float4 kv = ring[u];
      if (c + PF < NC) ring[u] = load_stream(kbase + (c + PF) * 256);
      const float* __restrict__ qc = qrow + 4 * c;
#pragma unroll
      for (int h = 0; h < HI; ++h) {
        float a = acc[h];
        a = __builtin_fmaf(qc[h * DI + 0], kv.x, a);
        a = __builtin_fmaf(qc[h * DI + 1], kv.y, a);
        a = __builtin_fmaf(qc[h * DI + 2], kv.z, a);
        a = __builtin_fmaf(qc[h * DI + 3], kv.w, a);
        acc[h] = a;
      }
    }
  }

  float s = 0.0f;
#pragma unroll
  for (int h = 0; h < HI; ++h) s = s + (acc[h] > 0.0f ? acc[h] : 0.0f);
  const int64_t g = tile * 64 + lane;
  const bool ok = g < rv.g;
  if (ok) scores[lrow * g_max + g] = s;
  if (maxima) {
    // maximum order key of the 16 consecutive groups sharing this DPP row
    static_assert(kSegment == 16, "one DPP row per segment");
    const uint32_t m = row_max16_u32(ok ? order_key(s) : 0u);
    if ((lane & (kSegment - 1)) == 0 && ok) maxima[lrow * (g_max / kSegment) + g / kSegment] = m;
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
  dim3 grid((unsigned)((tiles + kScoreWaves - 1) / kScoreWaves), (unsigned)a.rows);
  if (grid.x == 0 || a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL((score_kernel<HI, DI>), grid,
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

int launch_score(const ScoreArgs& a, int h_i, int d_i, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (h_i) {
    case 1: return launch_score_h<1>(a, d_i, s);
    case 2: return launch_score_h<2>(a, d_i, s);
    case 4: return launch_score_h<4>(a, d_i, s);
    case 8: return launch_score_h<8>(a, d_i, s);
    case 16: return launch_score_h<16>(a, d_i, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_segment_maxima(const float* scores, const int32_t* seq_len, int32_t queries,
                          int64_t g_max, int64_t row0, int64_t rows, uint32_t* maxima,
                          void* stream) {
  const int64_t segs = g_max / kSegment;
  dim3 grid((unsigned)((segs + 255) / 256), (unsigned)rows);
  if (grid.x == 0 || rows == 0) return 0;
  hipLaunchKernelGGL(segment_maxima_kernel, grid, dim3(256), 0,
                     static_cast<hipStream_t>(stream), scores, seq_len, queries, g_max, row0,
                     maxima);
  return hipGetLastError();
}

}  // namespace qsa
