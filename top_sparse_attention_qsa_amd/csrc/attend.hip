// attend.hip -- step 8: F32 online-softmax attention over the compact row.
//
// Attention over the same rows is permutation invariant only in exact
// arithmetic; in F32 the visit order shows in the last bits, so one canonical
// order is fixed (AFN-017 "Top-k chooses the set; time chooses the order",
// §Floating point makes order observable).  The order used here depends on
// the width alone: the compact row is cut into chunks of kAttnChunk
// consecutive rows; each chunk produces a partial (max m_c, denominator l_c,
// accumulator acc_c) with a fixed butterfly for the denominator and a
// chronological accumulation over the chunk's rows; the partials are merged
// in ascending chunk order (running maximum, rescale, denominator and
// accumulator updates).  No float atomics: results are run-to-run identical.
//
// attend_chunk_kernel: one workgroup per (chunk, KV head, row) stages the
// chunk's K and V rows of that KV head in LDS (K rows padded by 16 bytes so
// lane-per-row float4 reads are bank-conflict free) and serves every query
// head of its GQA group (query head hq reads KV head hq / (H_q/H_kv)).
// Scores: lane = compact row, query from scalar loads.  P.V: lane = output
// dimension.  merge_kernel: one wavefront per (query head, row).
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int C = kAttnChunk;

template <int D, int GQ>
__global__ void __launch_bounds__((GQ < 4 ? GQ : 4) * kWave)
attend_chunk_kernel(const float* __restrict__ q, const float* __restrict__ k_compact,
                    const float* __restrict__ v_compact, const int32_t* __restrict__ width,
                    int32_t q_heads, int32_t kv_heads, int32_t stride, int32_t n_chunks,
                    float scale, int64_t row0, float* __restrict__ part_acc,
                    float* __restrict__ part_ml) {
  constexpr int NW = GQ < 4 ? GQ : 4;
  constexpr int HPW = GQ / NW;   // query heads per wavefront
  constexpr int KP = D + 4;      // padded K row, floats
  constexpr int DPL = D / kWave; // output dims per lane
  __shared__ float4 ks4[C * KP / 4];
  __shared__ float4 vs4[C * D / 4];
  __shared__ float ps[GQ * C];
  const float* ks = reinterpret_cast<const float*>(ks4);
  const float* vs = reinterpret_cast<const float*>(vs4);

  const int tid = (int)threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int chunk = (int)blockIdx.x;
  const int hk = (int)blockIdx.y;
  const int64_t lrow = blockIdx.z;
  const int64_t row = row0 + lrow;
  const int32_t w = width[row];
  const int32_t c0 = chunk * C;
  if (w <= 0 || w > stride - 1 || c0 >= w) return;  // widths above 4k+3 are invalid
  const int cn = (w - c0) < C ? (w - c0) : C;

  // stage K and V of this chunk (rows past the width are zero)
  const int64_t rstride = (int64_t)kv_heads * D;  // floats between compact rows
  const float* kb = k_compact + ((lrow * stride + c0) * kv_heads + hk) * (int64_t)D;
  const float* vb = v_compact + ((lrow * stride + c0) * kv_heads + hk) * (int64_t)D;
  for (int e = tid; e < C * D / 4; e += NW * kWave) {
    const int i = e / (D / 4);
    const int c = e - i * (D / 4);
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
    if (i < cn) {
      kv = *reinterpret_cast<const float4*>(kb + i * rstride + 4 * c);
      vv = *reinterpret_cast<const float4*>(vb + i * rstride + 4 * c);
    }
    ks4[(i * KP) / 4 + c] = kv;
    vs4[e] = vv;
  }
  __syncthreads();

  // scores for this wavefront's query heads: lane = compact row
  const float* qrow[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    qrow[hh] = q + (row * q_heads + (int64_t)hk * GQ + wave * HPW + hh) * D;
  float dot[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) dot[hh] = 0.0f;
#pragma unroll 8
  for (int d = 0; d < D; d += 4) {
    const float4 k4 = *reinterpret_cast<const float4*>(ks + lane * KP + d);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float a = dot[hh];
      a = __builtin_fmaf(qrow[hh][d + 0], k4.x, a);
      a = __builtin_fmaf(qrow[hh][d + 1], k4.y, a);
      a = __builtin_fmaf(qrow[hh][d + 2], k4.z, a);
      a = __builtin_fmaf(qrow[hh][d + 3], k4.w, a);
      dot[hh] = a;
    }
  }
  float m_h[HPW], l_h[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float s = (lane < cn) ? dot[hh] * scale : -INFINITY;
    const float m = wave_max(s);
    const float p = (lane < cn) ? expf(s - m) : 0.0f;
    m_h[hh] = m;
    l_h[hh] = wave_sum(p);
    ps[(wave * HPW + hh) * C + lane] = p;
  }
  __syncthreads();

  // P.V: lane owns dims lane*DPL .. lane*DPL+DPL-1; rows in chronological order
  float acc[HPW][DPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[hh][j] = 0.0f;
#pragma unroll 4
  for (int i = 0; i < C; ++i) {
    float v[DPL];
    if constexpr (DPL == 2) {
      const float2 v2 = *reinterpret_cast<const float2*>(vs + i * D + 2 * lane);
      v[0] = v2.x;
      v[1] = v2.y;
    } else {
      v[0] = vs[i * D + lane];
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float p = ps[(wave * HPW + hh) * C + i];
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[hh][j] = __builtin_fmaf(p, v[j], acc[hh][j]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int64_t hq = (int64_t)hk * GQ + wave * HPW + hh;
    const int64_t slot = (lrow * q_heads + hq) * n_chunks + chunk;
    float* pa = part_acc + slot * D;
    if constexpr (DPL == 2)
      *reinterpret_cast<float2*>(pa + 2 * lane) = make_float2(acc[hh][0], acc[hh][1]);
    else
      pa[lane] = acc[hh][0];
    if (lane == 0) *reinterpret_cast<float2*>(part_ml + slot * 2) = make_float2(m_h[hh], l_h[hh]);
  }
}

template <int D>
__global__ void __launch_bounds__(kWave)
merge_kernel(const float* __restrict__ part_acc, const float* __restrict__ part_ml,
             const int32_t* __restrict__ width, int32_t q_heads, int32_t n_chunks,
             int32_t stride, int64_t row0, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int DPL = D / kWave;
  const int lane = lane_id();
  const int64_t hq = blockIdx.x;
  const int64_t lrow = blockIdx.y;
  const int64_t row = row0 + lrow;
  const int32_t w = width[row];
  float* o = out + (row * q_heads + hq) * D;
  if (w <= 0 || w > stride - 1) {
    const float fill = (w == 0) ? 0.0f : __int_as_float(0x7fc00000);
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[lane * DPL + j] = fill;
    if (lse && lane == 0) lse[row * q_heads + hq] = (w == 0) ? -INFINITY : fill;
    return;
  }
  const int nc = (w + C - 1) / C;
  const int64_t base = (lrow * q_heads + hq) * n_chunks;
  float m = -INFINITY;
  for (int c = 0; c < nc; ++c) m = fmaxf(m, part_ml[(base + c) * 2]);
  float l = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.0f;
  for (int c = 0; c < nc; ++c) {
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + (base + c) * 2);
    const float a = expf(ml.x - m);
    l = __builtin_fmaf(ml.y, a, l);
    const float* pa = part_acc + (base + c) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = __builtin_fmaf(pa[j], a, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[lane * DPL + j] = acc[j] / l;
  if (lse && lane == 0) lse[row * q_heads + hq] = m + logf(l);
}

template <int D, int GQ>
hipError_t launch_attend_t(const AttendArgs& a, hipStream_t s) {
  constexpr int NW = GQ < 4 ? GQ : 4;
  dim3 grid((unsigned)a.n_chunks, (unsigned)a.kv_heads, (unsigned)a.rows);
  hipLaunchKernelGGL((attend_chunk_kernel<D, GQ>), grid, dim3(NW * kWave), 0, s, a.q,
                     a.k_compact, a.v_compact, a.width, a.q_heads, a.kv_heads, a.stride,
                     a.n_chunks, a.scale, a.row0, a.part_acc, a.part_ml);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attend_d(const AttendArgs& a, hipStream_t s) {
  switch (a.q_heads / a.kv_heads) {
    case 1: return launch_attend_t<D, 1>(a, s);
    case 2: return launch_attend_t<D, 2>(a, s);
    case 4: return launch_attend_t<D, 4>(a, s);
    case 8: return launch_attend_t<D, 8>(a, s);
    case 16: return launch_attend_t<D, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  switch (a.head_dim) {
    case 64: return launch_attend_d<64>(a, s);
    case 128: return launch_attend_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const AttendArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  dim3 grid((unsigned)a.q_heads, (unsigned)a.rows);
  switch (a.head_dim) {
    case 64:
      hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kWave), 0, s, a.part_acc, a.part_ml,
                         a.width, a.q_heads, a.n_chunks, a.stride, a.row0, a.out, a.lse);
      break;
    case 128:
      hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kWave), 0, s, a.part_acc, a.part_ml,
                         a.width, a.q_heads, a.n_chunks, a.stride, a.row0, a.out, a.lse);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
