// RAII bracket for one kernel launch: records HIP events around it when the
// library's timing diagnostics are enabled (see rmm_timing_enable).
#pragma once

#include <hip/hip_runtime.h>

#include <string>

namespace rmm {

bool timing_on();

class KernelTimer {
 public:
  KernelTimer(const char *kernel, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer &) = delete;
  KernelTimer &operator=(const KernelTimer &) = delete;

 private:
  hipStream_t stream_;
  void *a_ = nullptr;
  void *b_ = nullptr;
  std::string key_;
};

}  // namespace rmm
