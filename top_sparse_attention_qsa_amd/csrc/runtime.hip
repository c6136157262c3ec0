// runtime.hip -- the HIP runtime calls the host side of libqsa.so makes
// outside kernel launches: the device's compute-unit count (persistent grids)
// and the events of the stage timer.
#include "qsa_internal.h"

namespace qsa {

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

int event_create(void** ev) {
  hipEvent_t e = nullptr;
  const hipError_t rc = hipEventCreate(&e);
  *ev = rc == hipSuccess ? static_cast<void*>(e) : nullptr;
  return rc;
}

int event_destroy(void* ev) { return hipEventDestroy(static_cast<hipEvent_t>(ev)); }

int event_record(void* ev, void* stream) {
  return hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(stream));
}

int event_synchronize(void* ev) { return hipEventSynchronize(static_cast<hipEvent_t>(ev)); }

int event_elapsed_ms(float* ms, void* start, void* stop) {
  return hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
}

}  // namespace qsa
