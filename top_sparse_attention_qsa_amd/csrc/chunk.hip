// chunk.hip -- step 1 for a causal chunk of query rows (prefill), on MFMA.
//
// With Q query rows per sequence every pooled key is used by Q x H_I dot
// products, so the row scores form a dense contraction
//   X[(row, head), g] = q_(row, head) . k_g,   score(row, g) = sum_h ReLU(X)
// and run on v_mfma_f32_16x16x4_f32 (AFN-016 "A sparse mask is not sparse
// attention", §Why a sparse mask can still be dense, for the score; AFN-017
// "Top-k chooses the set; time chooses the order", capsule evidence:
// chunk/decode equality, for what the chunk path must reproduce).
//
// MFMA's internal summation order is not the documented fused-multiply-add
// chain, so these scores are approximations s~ with a certified bound:
//   |s~ - s| <= E = 2 * ((2*g(D+2) + g(D)) * |k_g| * sum_h |q_h| + 2*g(H)*|s~|) / (1 - g(H))
// where s is the chain score, g(n) = n*u/(1-n*u), u = 2^-24 (the standard
// rounding-error bound of an n-term sum, once for the MFMA order, allowing an
// extra rounding per product, and once for the chain; sum_d |q_d k_d| is
// bounded by Cauchy-Schwarz; ReLU is 1-Lipschitz; the final 2 absorbs the
// rounding of E itself).  The kernel writes hi = s~ + E as the row's score and
// the per-16-group maxima of the order key of lo = s~ - E.  The selection
// kernel then keeps every group whose hi reaches a lower bound of the k-th
// largest lo, rescores those exactly with the chain, and selects among them,
// so the chosen set equals the one the chain scores give (see select.hip).
//
// Mapping: a workgroup owns 4 M-tiles of 16 (row, head) pairs (16/H_I rows
// each) and 4 wavefronts; each wavefront owns one 64-group pooled-key tile
// (4 N-subtiles of 16 groups).  A fragments are staged in LDS once per
// workgroup; B fragments are single dword loads that read 256 contiguous
// bytes of the tiled layout per wavefront.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int HI, int DI>
__global__ void __launch_bounds__(4 * kWave)
chunk_score_kernel(const float* __restrict__ index_q, const float* __restrict__ pooled,
                   const int64_t* __restrict__ pooled_off, const int32_t* __restrict__ seq_len,
                   int32_t queries, int64_t g_max, int64_t row0, float* __restrict__ approx,
                   float* __restrict__ bound, float* __restrict__ hi,
                   uint32_t* __restrict__ lo_maxima) {
  constexpr int RPM = 16 / HI;    // query rows per M-tile
  constexpr int RB = 4 * RPM;     // query rows per workgroup
  constexpr int NK = DI / 4;      // k-steps
  __shared__ float qa[NK * 4 * kWave];  // A fragments [k-step][M-tile][lane]
  __shared__ float hnorm[RB * HI];      // |q_(row, head)|
  __shared__ float qnorm[RB];           // sum over heads of |q_h| per row

  const int tid = (int)threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  const int64_t lrow0 = (int64_t)blockIdx.x * RB;  // first local row of this workgroup
  const int64_t grow0 = row0 + lrow0;
  const int b = (int)(grow0 / queries);            // all RB rows share this sequence

  // stage A fragments: A[i][k] of M-tile m, k-step c = q[row][head][4c + k]
  // with M-row i -> (row m*RPM + i/HI, head i%HI), i = lane%16, k = lane/16
  for (int e = tid; e < NK * 4 * kWave; e += 4 * kWave) {
    const int l = e & (kWave - 1);
    const int m = (e / kWave) & 3;
    const int c = e / (4 * kWave);
    const int i = l & 15;
    const int r = m * RPM + i / HI;
    qa[e] = index_q[((grow0 + r) * HI + (i % HI)) * DI + 4 * c + (l >> 4)];
  }
  if (tid < RB * HI) {  // RB * HI == 64: one (row, head) per lane of wavefront 0
    const float* qh = index_q + (grow0 * HI + tid) * DI;
    float ss = 0.0f;
    for (int d = 0; d < DI; ++d) ss = __builtin_fmaf(qh[d], qh[d], ss);
    hnorm[tid] = sqrtf(ss);
  }
  __syncthreads();
  if (tid < RB) {
    float sn = 0.0f;
    for (int h = 0; h < HI; ++h) sn += hnorm[tid * HI + h];
    qnorm[tid] = sn;
  }
  __syncthreads();

  // the longest row of the workgroup sets the tile range; shorter rows mask
  int64_t g_rows[RB];
  int64_t g_max_rows = 0;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const RowView rv = row_view(seq_len, grow0 + r, queries, g_max);
    g_rows[r] = rv.valid ? rv.g : -1;
    g_max_rows = rv.g > g_max_rows && rv.valid ? rv.g : g_max_rows;
  }
  const int64_t tile = (int64_t)blockIdx.y * 4 + wave;
  if (tile * 64 >= g_max_rows) return;

  const float* __restrict__ kt = pooled + pooled_off[b] + tile * (64 * DI);
  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ksq[4] = {0.f, 0.f, 0.f, 0.f};
  // B[k][j] of N-subtile t, k-step c = key[group 16t + j][4c + k], j = lane%16, k = lane/16
  const int boff = (lane & 15) * 4 + (lane >> 4);
  float bcur[4], bnext[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) bcur[t] = kt[t * 64 + boff];
#pragma unroll 2
  for (int c = 0; c < NK; ++c) {
    if (c + 1 < NK) {
#pragma unroll
      for (int t = 0; t < 4; ++t) bnext[t] = kt[(c + 1) * 256 + t * 64 + boff];
    }
    float a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = qa[(c * 4 + m) * kWave + lane];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      ksq[t] = __builtin_fmaf(bcur[t], bcur[t], ksq[t]);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], bcur[t], acc[m][t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) bcur[t] = bnext[t];
  }

  constexpr float u = 5.9604644775390625e-8f;  // 2^-24
  constexpr float gD = DI * u / (1.0f - DI * u);
  constexpr float gD2 = (DI + 2) * u / (1.0f - (DI + 2) * u);
  constexpr float gH = HI * u / (1.0f - HI * u);
  const int sub_row = (4 * (lane >> 4)) / HI;  // row within the M-tile held by this lane
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // |k_g|^2: lanes l, l^16, l^32, l^48 hold the four k-lanes of group l%16
    float kk = ksq[t];
    kk += __shfl_xor(kk, 16, kWave);
    kk += __shfl_xor(kk, 32, kWave);
    const float knorm = sqrtf(kk);
    const int64_t g = tile * 64 + t * 16 + (lane & 15);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // D[4*(l/16) + r][l%16]: this lane's four M-rows, all of one query row
      const f32x4 d = acc[m][t];
      float s = (d.x > 0.f ? d.x : 0.f) + (d.y > 0.f ? d.y : 0.f) + (d.z > 0.f ? d.z : 0.f) +
                (d.w > 0.f ? d.w : 0.f);
#pragma unroll
      for (int o = 16; o < 4 * HI; o <<= 1) s += __shfl_xor(s, o, kWave);
      const int r = m * RPM + sub_row;
      int64_t g_row = g_rows[m * RPM];  // select, not a lane-dependent register index
#pragma unroll
      for (int q2 = 1; q2 < RPM; ++q2)
        if (sub_row == q2) g_row = g_rows[m * RPM + q2];
      const float e = 2.0f * (((2.0f * gD2 + gD) * knorm * qnorm[r] + 2.0f * gH * fabsf(s)) /
                              (1.0f - gH)) + 1e-30f;
      const bool ok = g < g_row;
      // one lane group per query row writes (the others hold copies)
      const bool writer = ((lane >> 4) % (HI / 4)) == 0;
      const int64_t lr = lrow0 + r;
      if (ok && writer) {
        if (approx) approx[lr * g_max + g] = s;
        if (bound) bound[lr * g_max + g] = e;
        if (hi) hi[lr * g_max + g] = s + e;
      }
      if (lo_maxima) {
        uint32_t mk = ok ? order_key(s - e) : 0u;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const uint32_t y = (uint32_t)__shfl_xor((int)mk, o, kWave);
          mk = mk > y ? mk : y;
        }
        if (writer && (lane & 15) == 0 && ok)
          lo_maxima[lr * (g_max / kSegment) + g / kSegment] = mk;
      }
    }
  }
}

template <int HI, int DI>
hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t s) {
  constexpr int RB = 4 * (16 / HI);
  const int64_t tiles = (a.g_max + 63) / 64;
  dim3 grid((unsigned)(a.rows / RB), (unsigned)((tiles + 3) / 4));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_score_kernel<HI, DI>), grid, dim3(4 * kWave), 0, s, a.index_q,
                     a.pooled, a.pooled_off, a.seq_len, a.queries, a.g_max, a.row0, a.approx,
                     a.bound, a.hi, a.lo_maxima);
  return hipGetLastError();
}

template <int HI>
hipError_t launch_chunk_h(const ChunkArgs& a, int d_i, hipStream_t s) {
  switch (d_i) {
    case 32: return launch_chunk_t<HI, 32>(a, s);
    case 64: return launch_chunk_t<HI, 64>(a, s);
    case 128: return launch_chunk_t<HI, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool chunk_supported(int h_i, int queries, int64_t rows_per_launch) {
  if (h_i != 4 && h_i != 8 && h_i != 16) return false;
  const int rb = 4 * (16 / h_i);
  return queries % rb == 0 && rows_per_launch % rb == 0;
}

hipError_t launch_chunk(const ChunkArgs& a, int h_i, int d_i, hipStream_t s) {
  switch (h_i) {
    case 4: return launch_chunk_h<4>(a, d_i, s);
    case 8: return launch_chunk_h<8>(a, d_i, s);
    case 16: return launch_chunk_h<16>(a, d_i, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa
