// Launch bracketing for lora_trace_begin / lora_trace_end.
#pragma once
#include <hip/hip_runtime.h>

#include "lora_mi355x.h"

namespace lora {
bool trace_on();
void* trace_start(const char* name, hipStream_t st);  // nullptr when tracing is off
void trace_stop(void* handle, hipStream_t st);

// Brackets one launch on `st` with an event pair when tracing is on.
struct TraceScope {
  void* h;
  hipStream_t st;
  TraceScope(const char* name, hipStream_t s) : h(trace_start(name, s)), st(s) {}
  ~TraceScope() { trace_stop(h, st); }
};
}  // namespace lora
