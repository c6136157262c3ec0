// bench_stream_read.hip -- a plain streaming read of a device buffer, for the
// "achievable bandwidth" context line of bench.py.  Not part of libqsa: it
// computes nothing of the attention path and is built into its own small
// library next to bench.py (bench_stream_read.so).
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

// Grid-stride float4 loads over the whole buffer; the sum is stored only if
// it equals a value it never takes, which keeps every load live.
__global__ void __launch_bounds__(256)
stream_read_kernel(const float4* __restrict__ p, int64_t n4, float* __restrict__ sink) {
  float acc = 0.0f;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += step) {
    const float4 v = p[i];
    acc += (v.x + v.y) + (v.z + v.w);
  }
  if (acc == -1.2345e-30f) sink[0] = acc;
}

// Tiled read in the scoring kernel's shape: each wavefront streams one
// 32 KiB tile as 1 KiB chunks, four chunks in flight (nontemporal), and the
// launch reserves LDS so that at most five 256-thread workgroups share a
// compute unit (the fastest of the shapes measured on this part).
__global__ void __launch_bounds__(256)
tiled_read_kernel(const float* __restrict__ p, int64_t tiles, float* __restrict__ sink) {
  typedef float v4 __attribute__((ext_vector_type(4)));
  constexpr int kChunks = 32, kRing = 4;
  const int wave = (int)threadIdx.x / 64, lane = (int)threadIdx.x % 64;
  const int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  if (tile >= tiles) return;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p + tile * 8192), (short)0,
                                                    32768, 0x00020000);
  v4 ring[kRing];
#pragma unroll
  for (int u = 0; u < kRing; ++u)
    ring[u] = __builtin_bit_cast(v4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + u * 1024, 0, 2));
  float acc = 0.0f;
#pragma unroll 1
  for (int cb = 0; cb < kChunks; cb += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const v4 v = ring[u];
      if (cb + u + kRing < kChunks)
        ring[u] = __builtin_bit_cast(
            v4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + (cb + u + kRing) * 1024, 0, 2));
      acc += (v.x + v.y) + (v.z + v.w);
    }
  }
  if (acc == -1.2345e-30f) sink[0] = acc;
}

}  // namespace

// The tiled read over `bytes` (a multiple of 32 KiB) at `p`; same contract as
// bw_stream_read below.
extern "C" __attribute__((visibility("default"))) int bw_tiled_read(const void* p, int64_t bytes,
                                                                    float* sink, void* stream) {
  if (!p || !sink || bytes <= 0 || bytes % 32768 != 0) return 1;
  const int64_t tiles = bytes / 32768;
  hipLaunchKernelGGL(tiled_read_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 160 * 1024 / 5,
                     (hipStream_t)stream, reinterpret_cast<const float*>(p), tiles, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads `bytes` (a multiple of 16) from device pointer `p` once, on `stream`.
// `sink` is a device float that is written only in the impossible case above.
// Returns 0, 1 for a bad argument, 2 for a launch error.
extern "C" __attribute__((visibility("default"))) int bw_stream_read(const void* p, int64_t bytes,
                                                                     float* sink, void* stream) {
  if (!p || !sink || bytes <= 0 || bytes % 16 != 0) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const float4*>(p), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
