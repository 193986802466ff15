// Opt-in per-kernel timing: when enabled, each kernel launch is bracketed by
// a pair of HIP events recorded on the launch stream; records are reduced to
// (kernel name, launches, total milliseconds) when read back.
#pragma once

#include <hip/hip_runtime.h>

namespace dsa {

bool profiling_enabled();

class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t stream);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
  bool on_ = false;
};

}  // namespace dsa
