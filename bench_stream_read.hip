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

}  // namespace

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
