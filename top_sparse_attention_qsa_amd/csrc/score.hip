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
// contiguous, so each float4 load of the wave is one coalesced 1 KiB read,
// issued a few chunks ahead of its use.
// With 4, 8 or 16 index heads the multiply-adds run on the matrix cores
// (score_mfma_kernel: v_mfma_f32_4x4x1_16b_f32 rounds each step once, like
// fmaf, so the bits are those of the chain); the query row is staged in LDS.
// With 1 or 2 heads they run on the VALU (score_kernel), the query in SGPRs.
// The workload is HBM-bound: 8 flop per pooled-key byte.
#include "qsa_internal.h"

namespace qsa {
namespace {

// Cache-policy operand of the buffer intrinsics on this architecture: bit 0
// sc0, bit 1 nt, bit 4 sc1.
constexpr int kPolicyNt = 2;

// A raw buffer resource over `bytes` bytes at p (a uniform address).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Chunk c (dimensions 4c..4c+3) of this lane's group in a wavefront's tile.
// Pooled keys are read once per step, so the loads carry the nontemporal
// hint; every offset lies inside the tile (no SGPR offset: that part of a
// buffer address is not range checked).
struct TileLoader {
  __amdgpu_buffer_rsrc_t rs;
  __device__ float4 operator()(int c, int lane) const {
    typedef float v4 __attribute__((ext_vector_type(4)));
    const v4 v = __builtin_bit_cast(
        v4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + c * 1024, 0, kPolicyNt));
    return make_float4(v.x, v.y, v.z, v.w);
  }
};

// Stores of a wavefront's 64 scores (lane l: group g) and of its tile's four
// 16-group segment maxima (mk: the maximum order key of the lane's DPP row),
// the maxima as one 16-byte store from lane 0; segments past the row's last
// group hold 0 there, and are never read.  The scores are nontemporal: in a
// load-only probe of this kernel's reads, plain 256-byte score stores per
// wavefront added 5-10 us to the 163 us read of 1 GiB, nontemporal ones about
// 1 us (in the decode step the gain is 0-4 us, depending on the device).  The
// maxima (a sixteenth of the bytes) are plain stores, which the selection
// reads first: about 1 us less per decode step than nontemporal ones.
__device__ __forceinline__ void store_scores(float* __restrict__ srow, uint32_t* __restrict__ mrow,
                                             int64_t g_max, int64_t g, bool ok, float s,
                                             uint32_t mk) {
  const int lane = lane_id();
  const auto srs = buffer_over(srow, (uint32_t)(g_max * 4));
  if (ok) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, s), srs, (int)(g * 4), 0,
                                                kPolicyNt);
  if (mrow) {
    const auto mrs = buffer_over(mrow, (uint32_t)((g_max / kSegment) * 4));
    const uint32_t m1 = lane_value(mk, 16), m2 = lane_value(mk, 32), m3 = lane_value(mk, 48);
    typedef int v4i __attribute__((ext_vector_type(4)));
    if (lane == 0 && ok)
      __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)mk, (int)m1, (int)m2, (int)m3}, mrs,
                                             (int)((g / kSegment) * 4), 0, 0);
  }
}

// Residency and load depth of score_mfma_kernel.  Four workgroups (16
// wavefronts) per compute unit, each wavefront with four 1 KiB chunk loads in
// flight, read the pooled keys faster than the eight workgroups with two
// chunks in flight that fit by registers (163.9 against 168.5 us over the
// decode batch's 1 GiB; five per compute unit did as well as four, six,
// eight-chunk rings or eight tiles per wavefront did worse).  The cap is set
// by reserving LDS at launch (lds_reserve).
constexpr int kScoreMfmaRing = 4;
constexpr int kScoreWgsPerCu = 4;

// Matrix-core form of score_kernel for HI a multiple of 4: the same lanes,
// loads and fused multiply-adds in the same order, issued as
// v_mfma_f32_4x4x1_16b_f32.  With one product per step, block b of that
// instruction (lanes 4b..4b+3) adds A[i] * B[j] to D[i][j] with one
// rounding, A[i] from lane 4b+i and B[j] from lane 4b+j, D[i][j] in
// register i of lane 4b+j: with B = the key value of group l in lane l and
// A = the query value of head 4m + (l mod 4), register i of lane l
// accumulates head 4m+i of group l exactly as the fmaf chain does.
template <int HI, int DI>
__global__ void __launch_bounds__(kScoreWaves * kWave)
score_mfma_kernel(const float* __restrict__ index_q, const float* __restrict__ pooled,
                  const int64_t* __restrict__ pooled_off, const int32_t* __restrict__ seq_len,
                  int32_t queries, int64_t g_max, int64_t row0, float* __restrict__ scores,
                  uint32_t* __restrict__ maxima) {
  static_assert(HI % 4 == 0, "head quads");
  constexpr int HQ = HI / 4;
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef float vqf __attribute__((ext_vector_type(HQ)));
  const int64_t lrow = blockIdx.y;
  const int64_t row = row0 + lrow;
  const RowView rv = row_view(seq_len, row, queries, g_max);
  if (!rv.valid) return;
  const int wave = (int)(threadIdx.x / kWave);
  const int lane = lane_id();
  const int64_t tile = (int64_t)blockIdx.x * kScoreWaves + wave;  // 64 groups per wavefront
  const bool active = tile * 64 < rv.g;

  const float* __restrict__ qrow = index_q + row * (int64_t)(HI * DI);
  const float* tbase = pooled + pooled_off[rv.b] + tile * (64 * DI);
  const TileLoader ld{buffer_over(tbase, 64 * DI * 4)};

  constexpr int NC = DI / 4;
  constexpr int PF = kScoreMfmaRing;
  static_assert(NC % PF == 0, "ring depth must divide the chunk count");
  float4 ring[PF];
  if (active) {
#pragma unroll
    for (int u = 0; u < PF; ++u) ring[u] = ld(u, lane);
  }
  // the row's query, dimension-major: qs[d][i] holds heads i, 4+i, 8+i, ...
  __shared__ __attribute__((aligned(16))) float qs[DI][4][HQ];
  {
    // thread t fills entry t = (d, i) of qs with heads i, 4+i, ...: its HQ
    // values are gathered from the query rows, and consecutive threads write
    // consecutive entries (no LDS bank conflicts)
    constexpr int NT = kScoreWaves * kWave;
    constexpr int NE = DI * 4;  // (d, i) entries
    constexpr int PER = (NE + NT - 1) / NT;
    float qv[PER][HQ];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = (int)threadIdx.x + p * NT;
      const int d = e >> 2, i = e & 3;
#pragma unroll
      for (int m = 0; m < HQ; ++m)
        if (NE % NT == 0 || e < NE) qv[p][m] = qrow[(4 * m + i) * DI + d];
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = (int)threadIdx.x + p * NT;
      if (NE % NT == 0 || e < NE) {
        vqf v;
#pragma unroll
        for (int m = 0; m < HQ; ++m) v[m] = qv[p][m];
        *reinterpret_cast<vqf*>(&qs[e >> 2][e & 3][0]) = v;
      }
    }
  }
  __syncthreads();
  if (!active) return;

  v4f acc[HQ];
#pragma unroll
  for (int m = 0; m < HQ; ++m) acc[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const int qi = lane & 3;

#pragma unroll 1
  for (int cb = 0; cb < NC; cb += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int c = cb + u;
      const float4 kv = ring[u];
      if (c + PF < NC) ring[u] = ld(c + PF, lane);
      const vqf a0 = *reinterpret_cast<const vqf*>(&qs[4 * c + 0][qi][0]);
      const vqf a1 = *reinterpret_cast<const vqf*>(&qs[4 * c + 1][qi][0]);
      const vqf a2 = *reinterpret_cast<const vqf*>(&qs[4 * c + 2][qi][0]);
      const vqf a3 = *reinterpret_cast<const vqf*>(&qs[4 * c + 3][qi][0]);
#pragma unroll
      for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a0[m], kv.x, acc[m], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a1[m], kv.y, acc[m], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a2[m], kv.z, acc[m], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a3[m], kv.w, acc[m], 0, 0, 0);
    }
  }

  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < HQ; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) s = s + (acc[m][i] > 0.0f ? acc[m][i] : 0.0f);
  const int64_t g = tile * 64 + lane;
  const bool ok = g < rv.g;
  static_assert(kSegment == 16, "one DPP row per segment");
  const uint32_t mk = maxima ? row_max16_u32(ok ? order_key(s) : 0u) : 0u;
  store_scores(scores + lrow * g_max, maxima ? maxima + lrow * (g_max / kSegment) : nullptr,
               g_max, g, ok, s, mk);
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
  const float* tbase = pooled + pooled_off[rv.b] + tile * (64 * DI);
  const TileLoader ld{buffer_over(tbase, 64 * DI * 4)};

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
  for (int u = 0; u < PF; ++u) ring[u] = ld(u, lane);

#pragma unroll 1
  for (int cb = 0; cb < NC; cb += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int c = cb + u;
      const float4 kv = ring[u];
      if (c + PF < NC) ring[u] = ld(c + PF, lane);
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
  // maximum order key of the 16 consecutive groups sharing this DPP row
  static_assert(kSegment == 16, "one DPP row per segment");
  const uint32_t mk = maxima ? row_max16_u32(ok ? order_key(s) : 0u) : 0u;
  store_scores(scores + lrow * g_max, maxima ? maxima + lrow * (g_max / kSegment) : nullptr,
               g_max, g, ok, s, mk);
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
  if constexpr (HI % 4 == 0) {
    // the query staging (qs) is the kernel's only LDS; the rest of the
    // workgroup's share is reserved to cap residency
    constexpr int staged = DI * HI * 4;
    constexpr int reserve = lds_reserve(kScoreWgsPerCu, staged);
    static_assert(reserve >= 0, "query staging exceeds the workgroup's LDS share");
    hipLaunchKernelGGL((score_mfma_kernel<HI, DI>), grid, dim3(kScoreWaves * kWave), reserve, s,
                       a.index_q, a.pooled, a.pooled_off, a.seq_len, a.queries, a.g_max, a.row0,
                       a.scores, a.maxima);
  }
  else
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
