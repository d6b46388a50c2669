// A second stream per device for the independent branch of a call: work that
// neither reads nor writes what the main chain of the same call touches runs
// beside it (on MI355X small, latency-bound launches then overlap the
// bandwidth-bound gathers instead of queueing behind them).
//
// fork_side: the side stream waits for everything enqueued on the caller's
// stream so far. join_side: the caller's stream waits for everything enqueued
// on the side stream so far. Both only enqueue; neither blocks the host. The
// streams (default priority, non-blocking) and their two events are created
// on a device's first fork and kept until the process ends.
#include <mutex>

#include "twell_kernels.h"

namespace twell {
namespace {

constexpr int kMaxDevices = 64;

struct Side {
  bool tried = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

std::mutex g_mu;  // one record + wait pair at a time (the events are shared)
Side g_side[kMaxDevices];

}  // namespace

hipError_t fork_side(hipStream_t main, hipStream_t* side) {
  *side = main;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipSuccess;  // no side stream: everything stays on `main`
  std::lock_guard<std::mutex> g(g_mu);
  Side& S = g_side[dev];
  if (!S.tried) {
    S.tried = true;
    if (hipStreamCreateWithFlags(&S.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&S.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&S.join, hipEventDisableTiming) != hipSuccess) {
      S.s = nullptr;
      (void)hipGetLastError();
      return hipSuccess;
    }
  }
  if (S.s == nullptr) return hipSuccess;
  if ((err = hipEventRecord(S.fork, main)) != hipSuccess) return err;
  if ((err = hipStreamWaitEvent(S.s, S.fork, 0)) != hipSuccess) return err;
  *side = S.s;
  return hipSuccess;
}

hipError_t join_side(hipStream_t main, hipStream_t side) {
  if (side == main) return hipSuccess;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> g(g_mu);
  Side& S = g_side[dev];
  if ((err = hipEventRecord(S.join, side)) != hipSuccess) return err;
  return hipStreamWaitEvent(main, S.join, 0);
}

}  // namespace twell
