// Per-kernel event timing (see attn.h: attn_timing_enable / attn_timing_read).
#include <cstring>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "attn_error.hpp"
#include "attn_timing.hpp"

namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

struct TimingState {
  bool enabled = false;
  std::vector<Record> records;
  std::vector<hipEvent_t> pool;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

thread_local TimingState g_timing;

}  // namespace

namespace vca {

TimedLaunch::TimedLaunch(const char* name, hipStream_t stream) : stream_(stream) {
  if (!g_timing.enabled) return;
  Record r{name, g_timing.get(), g_timing.get()};
  if (!r.start || !r.stop || hipEventRecord(r.start, stream) != hipSuccess) return;
  slot_ = (int)g_timing.records.size();
  g_timing.records.push_back(r);
}

TimedLaunch::~TimedLaunch() {
  if (slot_ < 0) return;
  (void)hipEventRecord(g_timing.records[slot_].stop, stream_);
}

}  // namespace vca

extern "C" {

int attn_timing_enable(int enable) {
  const int prev = g_timing.enabled ? 1 : 0;
  g_timing.enabled = enable != 0;
  return prev;
}

int attn_timing_read(int max_records, char* names, int name_len, float* ms, int* count) {
  if (!count || max_records < 0 || (max_records > 0 && (!ms || !names || name_len < 2))) {
    vca::set_last_error("attn_timing_read: invalid arguments");
    return ATTN_E_INVALID;
  }
  const int n = (int)g_timing.records.size();
  *count = n;
  int status = ATTN_OK;
  for (int i = 0; i < n; ++i) {
    Record& r = g_timing.records[i];
    float t = -1.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      status = ATTN_E_HIP;
    if (i < max_records) {
      ms[i] = t;
      std::strncpy(names + (size_t)i * name_len, r.name, name_len - 1);
      names[(size_t)i * name_len + name_len - 1] = '\0';
    }
    g_timing.pool.push_back(r.start);
    g_timing.pool.push_back(r.stop);
  }
  g_timing.records.clear();
  if (status != ATTN_OK) vca::set_last_error("attn_timing_read: event query failed");
  return status;
}

}  // extern "C"
