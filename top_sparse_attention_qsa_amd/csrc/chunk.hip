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
// rounding of E itself: a few operations of at most an ulp each, the square
// roots on the hardware's v_sqrt_f32 and 1/(1 - g(H)) a rounded constant).  The kernel writes hi = s~ + E as the row's score,
// the per-16-group maxima of the order key of lo = s~ - E, and per 64-group
// tile a width W >= hi - s.  The selection kernel keeps every group whose hi
// reaches a lower bound of the k-th largest lo, settles by their bounds which
// of those are certainly in or out, rescores the rest exactly with the chain
// and selects among them, so the chosen set equals the one the chain scores
// give (see select.hip).
//
// Mapping: a workgroup owns 4 M-tiles of 16 (row, head) pairs (16/H_I rows
// each) and 4 wavefronts; each wavefront owns one 64-group pooled-key tile
// (4 N-subtiles of 16 groups).  The contraction over d may take the dimensions
// in any order (the bound does not depend on it), so k-slot kk of k-step
// 4q + i carries dimension 16q + 4kk + i: a lane then reads the B operands of
// four consecutive k-steps as one float4 of its group's key (dimension chunk
// 4q + kk of the tiled layout), and 16 lanes read 256 contiguous bytes.  A
// fragments are staged in LDS once per workgroup in the same order, one
// float4 per (quad, M-tile, lane).  The B loads of quad q + 1 are in flight
// while quad q runs on MFMA.  The output set is a template parameter (CERT):
// approximate scores and bounds, or hi, lo maxima and tile widths for the
// certified selection.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// v_sqrt_f32 is within an ulp for arguments from 2^-96 up; smaller sums of
// squares are raised to 2^-96 first, which can only enlarge a norm, so the
// bound stays an upper bound.
constexpr float kSqrtFloor = 0x1p-96f;

// At least three wavefronts per SIMD: without the register limit this sets,
// the compiler takes enough registers that only two fit, and the MFMA pipes
// idle while they wait for B (measured 25% slower at 16 heads x 128).
// Smaller index shapes hold more rows per workgroup and keep the default.
template <int HI, int DI, bool CERT>
__global__ void __launch_bounds__(4 * kWave)
__attribute__((amdgpu_waves_per_eu(HI * DI >= 512 ? 3 : 2)))
chunk_score_kernel(const float* __restrict__ index_q, const float* __restrict__ pooled,
                   const int64_t* __restrict__ pooled_off, const int32_t* __restrict__ seq_len,
                   int32_t queries, int64_t g_max, int64_t row0, float* __restrict__ approx,
                   float* __restrict__ bound, float* __restrict__ hi,
                   uint32_t* __restrict__ lo_maxima, float* __restrict__ widths) {
  constexpr int RPM = 16 / HI;    // query rows per M-tile
  constexpr int RB = 4 * RPM;     // query rows per workgroup
  constexpr int NQ = DI / 16;     // quads of four k-steps
  __shared__ f32x4 qa[NQ * 4 * kWave];  // A fragments [quad][M-tile][lane], 4 k-steps each
  __shared__ float qnorm[RB];           // sum over heads of |q_h| per row

  const int tid = (int)threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  const int64_t lrow0 = (int64_t)blockIdx.x * RB;  // first local row of this workgroup
  const int64_t grow0 = row0 + lrow0;
  // all RB rows share one sequence (RB divides the queries per sequence and
  // the first row); rows fit in 32 bits (at most 65,535), so one 32-bit
  // division finds it
  const int32_t b = (int32_t)grow0 / queries;
  const int32_t j0 = (int32_t)grow0 - b * queries;  // query index of the first row
  const int64_t n0 = (int64_t)seq_len[b] - queries + 1 + j0;  // visible tokens of the first row

  // the longest row of the workgroup sets the tile range; shorter rows mask.
  // A workgroup whose four tiles all lie past it leaves before staging
  // anything (with rows of very different lengths, most of the grid).
  // Row r sees n0 + r tokens (a row with none or more than g_max groups has
  // no groups to score).
  int64_t g_rows[RB];
  int64_t g_max_rows = 0;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int64_t n = n0 + r;
    const bool valid = n >= 0 && (n >> 2) <= g_max;
    g_rows[r] = valid ? (n >> 2) : -1;
    g_max_rows = valid && (n >> 2) > g_max_rows ? (n >> 2) : g_max_rows;
  }
  if ((int64_t)blockIdx.y * 4 * 64 >= g_max_rows) return;

  // this wavefront's pooled-key tile; a wavefront whose tile lies past the
  // rows reads tile 0 (which exists: the workgroup has a tile inside) until
  // it leaves after the barrier, so no load sits behind a branch
  const int64_t tile = (int64_t)blockIdx.y * 4 + wave;
  const bool active = tile * 64 < g_max_rows;
  const float* __restrict__ kt = pooled + pooled_off[b] + (active ? tile : 0) * (64 * DI);
  // lane (kk, j) of N-subtile t, quad q reads dimensions 16q + 4kk .. +3 of group 16t + j
  const float* __restrict__ kl = kt + (lane >> 4) * 256 + (lane & 15) * 4;
  auto load_quad = [&](f32x4 (&dst)[4], int q) {
#pragma unroll
    for (int t = 0; t < 4; ++t) dst[t] = *reinterpret_cast<const f32x4*>(kl + q * 1024 + t * 64);
  };
  f32x4 b0[4], b1[4];

  // stage A fragments: A[i][kk] of M-tile m, k-step 4q + s = q[row][head][16q + 4kk + s]
  // with M-row i -> (row m*RPM + i/HI, head i%HI), i = lane%16, kk = lane/16.
  // Each thread moves NQ float4s (four consecutive dimensions each), all
  // loads issued before the first store.  Thread (wavefront m, lane l) moves
  // quad n's float4 of M-tile m, lane l: its NQ float4s are a quarter of one
  // (row, head) pair's dimensions, the lanes l, l^16, l^32, l^48 hold the
  // rest, so the norms come from the same registers.
  {
    f32x4 st[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int i = lane & 15;
      const int r = wave * RPM + i / HI;
      st[n] = *reinterpret_cast<const f32x4*>(
          index_q + ((grow0 + r) * HI + (i % HI)) * DI + 16 * n + 4 * (lane >> 4));
    }
    // the first quad of B is issued after the A loads, so that waiting for
    // A does not wait for it, and arrives while A is staged
    __builtin_amdgcn_sched_barrier(0);
    load_quad(b0, 0);
    __builtin_amdgcn_sched_barrier(0);
    float ss = 0.0f;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      qa[tid + n * 4 * kWave] = st[n];
      ss = __builtin_fmaf(st[n].x, st[n].x, ss);
      ss = __builtin_fmaf(st[n].y, st[n].y, ss);
      ss = __builtin_fmaf(st[n].z, st[n].z, ss);
      ss = __builtin_fmaf(st[n].w, st[n].w, ss);
    }
    ss = xor16(ss, AddOp{});  // the pair's four quarters
    ss = xor32(ss, AddOp{});
    // |q_(row, head)| summed over the row's HI heads: aligned groups of HI
    // lanes of a DPP row, by quad swaps and row mirrors (each step adds two
    // partial sums whose order does not matter, so all lanes agree)
    float sn = __builtin_amdgcn_sqrtf(fmaxf(ss, kSqrtFloor));
    if constexpr (HI >= 2) sn = sn + dpp_f32<0xB1>(sn);   // quad_perm [1,0,3,2]
    if constexpr (HI >= 4) sn = sn + dpp_f32<0x4E>(sn);   // quad_perm [2,3,0,1]
    if constexpr (HI >= 8) sn = sn + dpp_f32<0x141>(sn);  // row_half_mirror
    if constexpr (HI >= 16) sn = sn + dpp_f32<0x140>(sn); // row_mirror
    if (lane < 16 && lane % HI == 0) qnorm[wave * RPM + lane / HI] = sn;
  }
  __syncthreads();

  if (!active) return;

  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ksq[4] = {0.f, 0.f, 0.f, 0.f};
  auto run_quad = [&](const f32x4 (&bv)[4], int q) {
    f32x4 a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = qa[(q * 4 + m) * kWave + lane];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float kk = ksq[t];
      kk = __builtin_fmaf(bv[t].x, bv[t].x, kk);
      kk = __builtin_fmaf(bv[t].y, bv[t].y, kk);
      kk = __builtin_fmaf(bv[t].z, bv[t].z, kk);
      kk = __builtin_fmaf(bv[t].w, bv[t].w, kk);
      ksq[t] = kk;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m][s], bv[t][s], acc[m][t], 0, 0, 0);
  };
  // two-deep ring over quads (NQ is even); the last refill re-reads the last
  // quad instead of being conditional, so every wait is for the older quad only
#pragma unroll 1
  for (int q = 0; q < NQ; q += 2) {
    load_quad(b1, q + 1);
    __builtin_amdgcn_sched_barrier(0);
    run_quad(b0, q);
    __builtin_amdgcn_sched_barrier(0);
    load_quad(b0, q + 2 < NQ ? q + 2 : NQ - 1);
    __builtin_amdgcn_sched_barrier(0);
    run_quad(b1, q + 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  constexpr float u = 5.9604644775390625e-8f;  // 2^-24
  constexpr float gD = DI * u / (1.0f - DI * u);
  constexpr float gD2 = (DI + 2) * u / (1.0f - (DI + 2) * u);
  constexpr float gH = HI * u / (1.0f - HI * u);
  constexpr float kInvOneMinusGH = 1.0f / (1.0f - gH);
  // After the head sum, lane (li, lq) holds for every N-subtile t the score
  // of group 16t + li for query row m * RPM + sub_row; the CPR lane groups
  // of one row hold copies.  The stores give each copy its own subtiles:
  // store v of M-tile m writes subtile t = v * CPR + lq % CPR, so every lane
  // writes a distinct group and a DPP row holds one 16-group segment
  // (4 / CPR stores per M-tile, all lanes active; at 16 heads one store
  // writes the tile's 64 groups as 256 contiguous bytes).
  constexpr int CPR = HI / 4;
  const int sub_row = (4 * (lane >> 4)) / HI;  // row within the M-tile held by this lane
  const int copy = (lane >> 4) % CPR;
  float knorm[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // |k_g|^2: lanes l, l^16, l^32, l^48 hold the four k-lanes of group l%16
    // (VALU cross-lane swaps: both lanes of a pair add the same two values)
    float kk = ksq[t];
    kk = xor16(kk, AddOp{});
    kk = xor32(kk, AddOp{});
    knorm[t] = __builtin_amdgcn_sqrtf(fmaxf(kk, kSqrtFloor));
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = m * RPM + sub_row;
    int64_t g_row = g_rows[m * RPM];  // select, not a lane-dependent register index
#pragma unroll
    for (int q2 = 1; q2 < RPM; ++q2)
      if (sub_row == q2) g_row = g_rows[m * RPM + q2];
    const int64_t lr = lrow0 + r;
    float sv[4], ev[4];
    float wt = 0.0f;  // the widest group of this lane's four (row, tile) groups
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // D[4*(l/16) + r][l%16]: this lane's four M-rows, all of one query row
      const f32x4 d = acc[m][t];
      float s = (d.x > 0.f ? d.x : 0.f) + (d.y > 0.f ? d.y : 0.f) + (d.z > 0.f ? d.z : 0.f) +
                (d.w > 0.f ? d.w : 0.f);
      if constexpr (HI >= 8) s = xor16(s, AddOp{});  // the head sum across lane rows
      if constexpr (HI >= 16) s = xor32(s, AddOp{});
      const float e = 2.0f * (((2.0f * gD2 + gD) * knorm[t] * qnorm[r] + 2.0f * gH * fabsf(s)) *
                              kInvOneMinusGH) + 1e-30f;
      sv[t] = s;
      ev[t] = e;
      const int64_t g = tile * 64 + t * 16 + (lane & 15);
      // hi - s <= (s~ + e)(1 + u) - (s~ - e/2) < 1.5e + u|hi|; the width adds
      // margin for its own rounding and for the subtraction hi - W the
      // selection makes, so that fl(hi - W) <= s (select.hip, certified band)
      if (CERT && g < g_row) wt = fmaxf(wt, 2.02f * e + 4.0f * u * fabsf(s + e));
    }
#pragma unroll
    for (int v = 0; v < 4 / CPR; ++v) {
      const int t = v * CPR + copy;
      float s = sv[v * CPR], e = ev[v * CPR];
#pragma unroll
      for (int c = 1; c < CPR; ++c)
        if (copy == c) {
          s = sv[v * CPR + c];
          e = ev[v * CPR + c];
        }
      const int64_t g = tile * 64 + t * 16 + (lane & 15);
      const bool ok = g < g_row;
      if constexpr (CERT) {
        if (ok) hi[lr * g_max + g] = s + e;
        // segment = the 16 lanes of a DPP row
        const uint32_t mk = row_max16_u32(ok ? order_key(s - e) : 0u);
        if ((lane & 15) == 0 && ok) lo_maxima[lr * (g_max / kSegment) + g / kSegment] = mk;
      } else if (ok) {
        approx[lr * g_max + g] = s;
        bound[lr * g_max + g] = e;
      }
    }
    if constexpr (CERT) {
      // one width per (row, 64-group tile): the maximum over the DPP row of the
      // lanes' maxima over the four N-subtiles (all 64 groups of the tile)
      const float w = row_max16(wt);
      if (copy == 0 && (lane & 15) == 0 && tile * 64 < g_row)
        widths[lr * (g_max / 64) + tile] = w;
    }
  }
}

template <int HI, int DI>
hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t s) {
  constexpr int RB = 4 * (16 / HI);
  const bool cert = a.hi != nullptr;
  if (cert ? (!a.lo_maxima || !a.widths || a.approx || a.bound)
           : (!a.approx || !a.bound || a.lo_maxima || a.widths))
    return hipErrorInvalidValue;
  const int64_t tiles = (a.g_max + 63) / 64;
  dim3 grid((unsigned)(a.rows / RB), (unsigned)((tiles + 3) / 4));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (cert)
    hipLaunchKernelGGL((chunk_score_kernel<HI, DI, true>), grid, dim3(4 * kWave), 0, s,
                       a.index_q, a.pooled, a.pooled_off, a.seq_len, a.queries, a.g_max, a.row0,
                       a.approx, a.bound, a.hi, a.lo_maxima, a.widths);
  else
    hipLaunchKernelGGL((chunk_score_kernel<HI, DI, false>), grid, dim3(4 * kWave), 0, s,
                       a.index_q, a.pooled, a.pooled_off, a.seq_len, a.queries, a.g_max, a.row0,
                       a.approx, a.bound, a.hi, a.lo_maxima, a.widths);
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

int launch_chunk(const ChunkArgs& a, int h_i, int d_i, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (h_i) {
    case 4: return launch_chunk_h<4>(a, d_i, s);
    case 8: return launch_chunk_h<8>(a, d_i, s);
    case 16: return launch_chunk_h<16>(a, d_i, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa
