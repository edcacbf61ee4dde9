// Opt-in per-kernel timing: when enabled on a thread, every kernel the library
// launches from that thread is bracketed by HIP events on its own stream.
#pragma once

#include <hip/hip_runtime.h>

namespace vca {

// RAII bracket around one launch; a no-op unless timing is enabled.
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t stream);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  int slot_ = -1;
  hipStream_t stream_;
};

}  // namespace vca
