// noalloc.hip -- qsa_decode_noalloc: qsa_decode over the library's own
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The workspace is the file-scope array `scratch` below: every device the
// library runs on holds its own copy, of QSA_NOALLOC_WORKSPACE_BYTES, until
// the process ends.  In host code the array's name is only a host-side
// stand-in, so its device address is looked up once per device (with that
// device current) through hipGetSymbolAddress and kept in a per-device table;
// host code uses that address, never the name.  The decode kernels write every
// workspace byte they later read within the same call, so nothing has to start
// at zero; calls that overlap on one device share the array and race.
#include <atomic>
#include <mutex>

#include "qsa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_lookup;

// The current device's address of `scratch`, looked up on the first call on
// that device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QSA_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QSA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QSA_OK;
}

}  // namespace

extern "C" int qsa_decode_noalloc(const qsa_shape* s, const float* index_q, const float* pooled,
                                  const int64_t* pooled_off, const int32_t* seq_len,
                                  const int32_t* slot_map, const int64_t* slot_off,
                                  const float* k_cache, const float* v_cache, const float* q,
                                  float softmax_scale, int32_t* token_ids, int32_t* width,
                                  float* out, float* lse, qsa_timer* timer, qsa_stream stream) {
  if (!s) return QSA_ERR_NULL;
  // 0 means an invalid shape: qsa_decode then reports which check failed
  // before it looks at the workspace
  const size_t need = qsa_workspace_bytes(s);
  if (need > (size_t)QSA_NOALLOC_WORKSPACE_BYTES) return QSA_ERR_STATIC_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc != QSA_OK) return rc;
  }
  return qsa_decode(s, index_q, pooled, pooled_off, seq_len, slot_map, slot_off, k_cache, v_cache,
                    q, softmax_scale, token_ids, width, out, lse, ws,
                    (size_t)QSA_NOALLOC_WORKSPACE_BYTES, timer, stream);
}
