// trace.cpp -- event bracketing of kernel launches for measurement.
#include "trace.hpp"

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "attn.h"

namespace lcattn {
namespace {

struct Record {
  const char* name;  // static string of the launcher
  hipEvent_t start, stop;
};

constexpr size_t kMaxRecords = 8192;

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
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

bool trace_on() { return g_on.load(std::memory_order_relaxed); }

int trace_begin(const char* name, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_records.size() >= kMaxRecords) return -1;
  Record r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return -1;
  if (hipEventRecord(r.start, stream) != hipSuccess) return -1;
  g_records.push_back(r);
  return (int)g_records.size() - 1;
}

void trace_end(int slot, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (slot >= 0 && (size_t)slot < g_records.size()) (void)hipEventRecord(g_records[slot].stop, stream);
}

}  // namespace lcattn

extern "C" {

int attn_trace_enable(int on) {
  lcattn::g_on.store(on != 0, std::memory_order_relaxed);
  return ATTN_OK;
}

int attn_trace_collect(char* names, int name_len, double* total_ms, int* calls, int max_kernels) {
  using namespace lcattn;
  std::lock_guard<std::mutex> lock(g_mu);
  int n = 0;
  int status = 0;
  for (const Record& r : g_records) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      status = -ATTN_ERR_HIP;
    }
    int k = 0;
    while (k < n && std::strncmp(names + (size_t)k * name_len, r.name, name_len - 1) != 0) ++k;
    if (k == n) {
      if (n == max_kernels) continue;
      std::strncpy(names + (size_t)k * name_len, r.name, name_len - 1);
      names[(size_t)k * name_len + name_len - 1] = '\0';
      total_ms[k] = 0.0;
      calls[k] = 0;
      ++n;
    }
    total_ms[k] += ms;
    calls[k] += 1;
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
  return status ? status : n;
}

}  // extern "C"
