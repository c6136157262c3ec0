// stub.h -- a recording stand-in for the kernel launchers of libqsa.so, so
// that the host side (api.cpp) can be built and exercised under the host
// sanitizers on a machine without a GPU.  No launcher touches memory.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

namespace stub {

struct Call {
  std::string name;
  int64_t row0 = 0, rows = 0;
  std::vector<const void*> ptrs;  // pointer arguments, in declaration order
  void* stream = nullptr;
};

extern std::vector<Call> calls;  // launches and event records since the last reset
extern int fail_at;              // index of the launch that reports a HIP error (-1: none)
extern int events_live;          // events created and not yet destroyed

void reset();
int count(const std::string& name);

}  // namespace stub
