// pool.hip -- group pooling into the tiled pooled-key buffer.
//
// One pooled index key per complete four-token group, the group mean of the
// four raw index keys evaluated as (((r0 + r1) + r2) + r3) * 0.25; the raw
// cache itself is left untouched (AFN-016 "A sparse mask is not sparse
// attention", §Why a sparse mask can still be dense).  A launch pools groups
// [first_group[b], floor(seq_len[b]/4)) of every sequence, so pooling a whole
// history and appending the groups completed since the last call produce the
// same bits (AFN-017 "Top-k chooses the set; time chooses the order", capsule
// evidence: full-raw/incremental identity).
//
// A thread owns one float4 of one group: it reads the four raw rows and
// writes the 16-byte slot of the tiled layout.  Lanes are laid out as
// kGroups consecutive groups by dimension chunk, so that each load of a
// wavefront reads 128-byte runs of raw rows and each store writes 128-byte
// runs of the tiled layout (consecutive groups of one chunk are adjacent
// there).
#include "qsa_internal.h"

namespace qsa {
namespace {

template <int DI>
__global__ void __launch_bounds__(256)
pool_kernel(const float* __restrict__ raw, const int64_t* __restrict__ raw_off,
            const int32_t* __restrict__ seq_len, const int32_t* __restrict__ first_group,
            float* __restrict__ pooled, const int64_t* __restrict__ pooled_off, int64_t g_max) {
  constexpr int NC = DI / 4;
  constexpr int kGroups = 8;  // divides every max_groups (a multiple of 64)
  const int b = (int)blockIdx.y;
  const int64_t n = seq_len[b];
  int64_t G = n > 0 ? n / 4 : 0;
  if (G > g_max) G = g_max;
  int64_t g_from = first_group ? (int64_t)first_group[b] : 0;
  if (g_from < 0) g_from = 0;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = e / (kGroups * NC);
  const int u = (int)(e - blk * (kGroups * NC));
  const int c = u / kGroups;
  const int64_t g = blk * kGroups + (u - c * kGroups);
  if (g < g_from || g >= G) return;
  const float* r = raw + (raw_off[b] + 4 * g) * DI + 4 * c;
  const float4 r0 = *reinterpret_cast<const float4*>(r);
  const float4 r1 = *reinterpret_cast<const float4*>(r + DI);
  const float4 r2 = *reinterpret_cast<const float4*>(r + 2 * DI);
  const float4 r3 = *reinterpret_cast<const float4*>(r + 3 * DI);
  float4 s;
  s.x = (((r0.x + r1.x) + r2.x) + r3.x) * 0.25f;
  s.y = (((r0.y + r1.y) + r2.y) + r3.y) * 0.25f;
  s.z = (((r0.z + r1.z) + r2.z) + r3.z) * 0.25f;
  s.w = (((r0.w + r1.w) + r2.w) + r3.w) * 0.25f;
  float* dst = pooled + pooled_off[b] + (g >> 6) * (64 * DI) + c * 256 + (g & 63) * 4;
  *reinterpret_cast<float4*>(dst) = s;
}

constexpr int kPoolWgsPerCu = 4;

template <int DI>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t s) {
  const int64_t elems = a.g_max * (DI / 4);
  dim3 grid((unsigned)((elems + 255) / 256), (unsigned)a.batch);
  if (grid.x == 0 || a.batch == 0) return hipSuccess;
  // four workgroups per compute unit: 0.941 ms against 0.982 ms for the eight
  // that fit by threads (4 GiB read, 1 GiB written; three to five per compute
  // unit did about as well, six or more no better than eight)
  hipLaunchKernelGGL(pool_kernel<DI>, grid, dim3(256), lds_reserve(kPoolWgsPerCu, 0), s,
                     a.raw_keys, a.raw_off, a.seq_len, a.first_group, a.pooled, a.pooled_off,
                     a.g_max);
  return hipGetLastError();
}

}  // namespace

int launch_pool(const PoolArgs& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.index_dim) {
    case 32: return launch_pool_t<32>(a, s);
    case 64: return launch_pool_t<64>(a, s);
    case 128: return launch_pool_t<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa
