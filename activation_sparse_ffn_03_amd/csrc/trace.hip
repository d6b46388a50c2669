// Per-kernel tracing with HIP events (diagnostics for timing individual
// kernels on the stream they run on). Events are created up front by
// twell_trace_start, so recording allocates nothing.
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/twell.h"
#include "twell_trace.h"

namespace twell {
namespace {

struct Rec {
  const char* name;
  hipEvent_t beg, end;
};

struct State {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<Rec> recs;  // pre-created events
  int used = 0;
  int dropped = 0;
  bool open = false;
};

State& st() {
  static State s;
  return s;
}

}  // namespace

bool trace_on() { return st().on.load(std::memory_order_relaxed); }

void trace_begin(hipStream_t s, const char* name) {
  if (!trace_on()) return;
  State& S = st();
  std::lock_guard<std::mutex> g(S.mu);
  if (S.used >= (int)S.recs.size()) {
    ++S.dropped;
    S.open = false;
    return;
  }
  Rec& r = S.recs[S.used];
  r.name = name;
  (void)hipEventRecord(r.beg, s);
  S.open = true;
}

void trace_end(hipStream_t s) {
  if (!trace_on()) return;
  State& S = st();
  std::lock_guard<std::mutex> g(S.mu);
  if (!S.open) return;
  (void)hipEventRecord(S.recs[S.used].end, s);
  ++S.used;
  S.open = false;
}

}  // namespace twell

extern "C" {

twell_status twell_trace_start(int32_t capacity) {
  if (capacity <= 0 || capacity > (1 << 20)) return TWELL_ERR_INVALID_ARG;
  twell::State& S = twell::st();
  std::lock_guard<std::mutex> g(S.mu);
  S.on.store(false);
  while ((int)S.recs.size() < capacity) {
    twell::Rec r{nullptr, nullptr, nullptr};
    if (hipEventCreate(&r.beg) != hipSuccess) return TWELL_ERR_HIP;
    if (hipEventCreate(&r.end) != hipSuccess) {
      (void)hipEventDestroy(r.beg);
      return TWELL_ERR_HIP;
    }
    S.recs.push_back(r);
  }
  S.used = 0;
  S.dropped = 0;
  S.open = false;
  S.on.store(true);
  return TWELL_OK;
}

twell_status twell_trace_stop(void) {
  twell::st().on.store(false);
  return TWELL_OK;
}

int32_t twell_trace_count(void) { return twell::st().used; }

int32_t twell_trace_dropped(void) { return twell::st().dropped; }

twell_status twell_trace_get(int32_t i, const char** name, float* ms) {
  twell::State& S = twell::st();
  std::lock_guard<std::mutex> g(S.mu);
  if (i < 0 || i >= S.used || name == nullptr || ms == nullptr) return TWELL_ERR_INVALID_ARG;
  const twell::Rec& r = S.recs[i];
  if (hipEventSynchronize(r.end) != hipSuccess) return TWELL_ERR_HIP;
  if (hipEventElapsedTime(ms, r.beg, r.end) != hipSuccess) return TWELL_ERR_HIP;
  *name = r.name;
  return TWELL_OK;
}

}  // extern "C"
