// Event-based kernel timing used by the benchmark (diagnostics only).
#include "timing.hpp"

#include <cstring>
#include <string>
#include <vector>

#include "../../include/spatten.h"

namespace spatten {

bool g_timing = false;

namespace {

struct Mark {
  const char* name;
  hipEvent_t start, stop;
};

std::vector<Mark> g_marks;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void timing_mark(const char* name, hipStream_t stream, bool begin) {
  if (begin) {
    Mark m{name, take_event(), nullptr};
    if (m.start && hipEventRecord(m.start, stream) != hipSuccess) m.start = nullptr;
    g_marks.push_back(m);
  } else if (!g_marks.empty()) {
    Mark& m = g_marks.back();
    m.stop = take_event();
    if (m.stop && hipEventRecord(m.stop, stream) != hipSuccess) m.stop = nullptr;
  }
}

}  // namespace spatten

using namespace spatten;

extern "C" {

int spatten_debug_timing(int enable) {
  g_timing = enable != 0;
  return SPATTEN_OK;
}

int spatten_debug_kernel_times(int max_kernels, char* names, int name_len, double* total_ms,
                               int* launches, int* n_kernels) {
  if (max_kernels < 0 || name_len < 1 || !n_kernels) return SPATTEN_EINVAL;
  std::vector<std::string> keys;
  std::vector<double> ms;
  std::vector<int> cnt;
  int status = SPATTEN_OK;
  for (Mark& m : g_marks) {
    float t = 0.0f;
    if (!m.start || !m.stop) {
      status = SPATTEN_EHIP;
    } else if (hipEventSynchronize(m.stop) != hipSuccess ||
               hipEventElapsedTime(&t, m.start, m.stop) != hipSuccess) {
      status = SPATTEN_EHIP;
    }
    size_t i = 0;
    while (i < keys.size() && keys[i] != m.name) ++i;
    if (i == keys.size()) {
      keys.emplace_back(m.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
    if (m.start) g_pool.push_back(m.start);
    if (m.stop) g_pool.push_back(m.stop);
  }
  g_marks.clear();
  const int n = int(keys.size()) < max_kernels ? int(keys.size()) : max_kernels;
  for (int i = 0; i < n; ++i) {
    if (names) {
      std::strncpy(names + size_t(i) * name_len, keys[i].c_str(), size_t(name_len) - 1);
      names[size_t(i) * name_len + name_len - 1] = 0;
    }
    if (total_ms) total_ms[i] = ms[i];
    if (launches) launches[i] = cnt[i];
  }
  *n_kernels = n;
  return status;
}

}  // extern "C"
