// Per-kernel event timing for libdsa (see profile.h and dsa_profile_* in dsa.h).
#include "profile.h"

#include <atomic>
#include <map>
#include <mutex>
#include <string.h>
#include <string>
#include <vector>

#include "../../include/dsa.h"

namespace dsa {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  std::lock_guard<std::mutex> lk(g_mu);
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

bool profiling_enabled() { return g_on.load(std::memory_order_relaxed); }

ProfScope::ProfScope(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  if (!profiling_enabled()) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, stream_) == hipSuccess) on_ = true;
}

ProfScope::~ProfScope() {
  if (!on_) return;
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, stream_) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_records.push_back({name_, start_, stop});
}

}  // namespace dsa

extern "C" {

int dsa_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(dsa::g_mu);
  for (auto& r : dsa::g_records) {
    dsa::g_pool.push_back(r.start);
    dsa::g_pool.push_back(r.stop);
  }
  dsa::g_records.clear();
  dsa::g_on.store(on != 0);
  return DSA_OK;
}

int dsa_profile_read(int max_kernels, char* names, int name_len, int* launches,
                     double* total_ms, int* n_kernels) {
  if (max_kernels < 0 || name_len < 1 || !n_kernels) return DSA_ERR_INVALID_ARG;
  std::vector<dsa::Record> recs;
  {
    std::lock_guard<std::mutex> lk(dsa::g_mu);
    recs.swap(dsa::g_records);
  }
  std::map<std::string, std::pair<int, double>> agg;
  std::vector<std::string> order;
  int status = DSA_OK;
  for (auto& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      status = DSA_ERR_HIP;
      continue;
    }
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {1, (double)ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
  }
  {
    std::lock_guard<std::mutex> lk(dsa::g_mu);
    for (auto& r : recs) {
      dsa::g_pool.push_back(r.start);
      dsa::g_pool.push_back(r.stop);
    }
  }
  int n = 0;
  for (auto& name : order) {
    if (n >= max_kernels) break;
    if (names) {
      strncpy(names + (size_t)n * name_len, name.c_str(), name_len - 1);
      names[(size_t)n * name_len + name_len - 1] = '\0';
    }
    if (launches) launches[n] = agg[name].first;
    if (total_ms) total_ms[n] = agg[name].second;
    ++n;
  }
  *n_kernels = n;
  return status;
}

}  // extern "C"
