// Kernel timing: HIP event pairs around each launch, on the launch stream.
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "trace.hpp"

namespace lora {
namespace {

struct Rec {
  std::string name;
  hipEvent_t start, stop;
};

// g_on is read without the lock on every launch, so a launch with tracing off
// touches no lock; the records and the event pool are guarded by g_mu.
std::mutex g_mu;
std::atomic<bool> g_on{false};
std::string g_prefix;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
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

bool trace_on() { return g_on.load(std::memory_order_acquire); }

void* trace_start(const char* name, hipStream_t st) {
  if (!g_on.load(std::memory_order_acquire)) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on.load(std::memory_order_relaxed)) return nullptr;
  if (!g_prefix.empty() && std::strncmp(name, g_prefix.c_str(), g_prefix.size()) != 0) return nullptr;
  Rec r{name, get_event(), get_event()};
  if (!r.start || !r.stop) return nullptr;
  if (hipEventRecord(r.start, st) != hipSuccess) return nullptr;
  g_recs.push_back(r);
  return reinterpret_cast<void*>(g_recs.size());  // 1-based handle
}

void trace_stop(void* handle, hipStream_t st) {
  if (!handle) return;
  std::lock_guard<std::mutex> lk(g_mu);
  const size_t i = reinterpret_cast<size_t>(handle) - 1;
  if (i < g_recs.size()) (void)hipEventRecord(g_recs[i].stop, st);
}

}  // namespace lora

using namespace lora;

extern "C" {

lora_status lora_trace_begin(const char* prefix) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prefix = prefix ? prefix : "";
  for (auto& r : g_recs) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  g_on.store(true, std::memory_order_release);
  return LORA_OK;
}

lora_status lora_trace_end(lora_trace_entry* out, int32_t max, int32_t* count) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on.store(false, std::memory_order_release);
  std::vector<lora_trace_entry> agg;
  lora_status st = LORA_OK;
  for (auto& r : g_recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = LORA_EDEVICE;
      continue;
    }
    size_t j = 0;
    while (j < agg.size() && std::strncmp(agg[j].name, r.name.c_str(), sizeof(agg[j].name)) != 0) ++j;
    if (j == agg.size()) {
      lora_trace_entry e{};
      std::strncpy(e.name, r.name.c_str(), sizeof(e.name) - 1);
      agg.push_back(e);
    }
    agg[j].launches += 1;
    agg[j].total_ms += ms;
  }
  for (auto& r : g_recs) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  if (count) *count = (int32_t)agg.size();
  for (size_t j = 0; out && j < agg.size() && (int32_t)j < max; ++j) out[j] = agg[j];
  return st;
}

}  // extern "C"
