// A second stream for the independent branch of a call: work that neither
// reads nor writes what the main chain of the same call touches runs beside
// it (on MI355X small, latency-bound launches then overlap the
// bandwidth-bound gathers instead of queueing behind them).
//
// Each caller stream (per device) gets its own side stream and its own pair of
// fork / join events, created on its first fork and kept until the process
// ends, so calls on different caller streams neither serialise through a
// shared stream nor share events. At most kMaxPerDevice caller streams per
// device get one; further ones, and a caller stream that is being captured
// into a graph before it has a side stream (no stream is created during a
// capture), run the branch in order on the caller's stream instead.
//
// fork_side: the side stream waits for everything enqueued on the caller's
// stream so far. join_side: the caller's stream waits for everything enqueued
// on the side stream so far. mark_side / wait_mark split a join in two: the
// mark is taken on the side stream (everything enqueued there so far), and the
// caller's stream waits for it later, so work enqueued on the side stream in
// between runs on past that point. All only enqueue; none blocks the host.
// All streams have the default priority and are non-blocking.
#include <mutex>

#include "twell_kernels.h"

namespace twell {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxPerDevice = 16;

struct Side {
  hipStream_t caller = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, mark = nullptr;
};

struct DeviceSides {
  Side e[kMaxPerDevice];
  int n = 0;
};

std::mutex g_mu;  // guards the tables and each record + wait pair
DeviceSides g_dev[kMaxDevices];

Side* find_caller(DeviceSides& d, hipStream_t caller) {
  for (int k = 0; k < d.n; ++k)
    if (d.e[k].caller == caller) return &d.e[k];
  return nullptr;
}

Side* find_side(DeviceSides& d, hipStream_t side) {
  for (int k = 0; k < d.n; ++k)
    if (d.e[k].s == side) return &d.e[k];
  return nullptr;
}

}  // namespace

hipError_t fork_side(hipStream_t main, hipStream_t* side) {
  *side = main;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipSuccess;  // no side stream: everything stays on `main`
  std::lock_guard<std::mutex> g(g_mu);
  DeviceSides& d = g_dev[dev];
  Side* S = find_caller(d, main);
  if (S == nullptr) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(main, &cs) != hipSuccess) {
      (void)hipGetLastError();
      return hipSuccess;
    }
    if (cs != hipStreamCaptureStatusNone || d.n >= kMaxPerDevice) return hipSuccess;
    Side n;
    n.caller = main;
    if (hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) != hipSuccess) {
      (void)hipGetLastError();
      return hipSuccess;
    }
    if (hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.join, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.mark, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipStreamDestroy(n.s);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.join) (void)hipEventDestroy(n.join);
      return hipSuccess;
    }
    d.e[d.n] = n;
    S = &d.e[d.n++];
  }
  if ((err = hipEventRecord(S->fork, main)) != hipSuccess) return err;
  if ((err = hipStreamWaitEvent(S->s, S->fork, 0)) != hipSuccess) return err;
  *side = S->s;
  return hipSuccess;
}

hipError_t join_side(hipStream_t main, hipStream_t side) {
  if (side == main) return hipSuccess;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> g(g_mu);
  Side* S = find_side(g_dev[dev], side);
  if (S == nullptr) return hipErrorInvalidValue;  // not a side stream this library forked
  if ((err = hipEventRecord(S->join, side)) != hipSuccess) return err;
  return hipStreamWaitEvent(main, S->join, 0);
}

hipError_t mark_side(hipStream_t main, hipStream_t side) {
  if (side == main) return hipSuccess;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> g(g_mu);
  Side* S = find_side(g_dev[dev], side);
  if (S == nullptr) return hipErrorInvalidValue;
  return hipEventRecord(S->mark, side);
}

hipError_t wait_mark(hipStream_t main, hipStream_t side) {
  if (side == main) return hipSuccess;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> g(g_mu);
  Side* S = find_side(g_dev[dev], side);
  if (S == nullptr) return hipErrorInvalidValue;
  return hipStreamWaitEvent(main, S->mark, 0);
}

}  // namespace twell
