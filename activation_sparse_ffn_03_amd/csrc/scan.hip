// Deterministic single-workgroup compaction used for the overflow-row list
// (TwELL) and the dense-backup row list (hybrid format). Both lists are in
// ascending row order, the reading taken for the pages' row routing (no
// order is stated there).
#include "block_scan.h"
#include "twell_device.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

// 1 in byte k of the result iff byte k of w is nonzero (bit 0 of each byte
// gathers the byte's 8 bits; bits that fold in from the next byte land above
// bit 0 and are masked off).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
  w |= w >> 4;
  w |= w >> 2;
  w |= w >> 1;
  return w & 0x01010101u;
}

// One workgroup of 1024 threads: thread t owns the flags [t*chunk, t*chunk +
// chunk), read as 32-bit words when chunk is a multiple of 4 (all of a
// thread's loads in flight together), and the workgroup's exclusive sum of
// the per-thread counts is the list position of its first flagged row; only
// threads with a flagged row read their flags a second time.
__global__ __launch_bounds__(1024) void compact_flags(const uint8_t* __restrict__ flag, int64_t N, int32_t* rows,
                                                      int cap, int32_t* n_out, uint32_t* status, uint32_t bit) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x;
  const int64_t chunk = (N + 1023) / 1024;
  const int64_t b = min(N, (int64_t)tid * chunk), en = min(N, b + chunk);
  int32_t c = 0;
  int64_t i = b;
  if ((chunk & 3) == 0 && (reinterpret_cast<uintptr_t>(flag) & 3) == 0) {
#pragma unroll 4
    for (; i + 4 <= en; i += 4) c += __popc(nonzero_bytes(*reinterpret_cast<const uint32_t*>(flag + i)));
  }
  for (; i < en; ++i) c += flag[i] != 0;
  int32_t total;
  int32_t pos = block_excl_1024(c, wsum, &total);
  if (c > 0)
    for (int64_t k = b; k < en; ++k)
      if (flag[k]) {
        if (pos < cap) rows[pos] = (int32_t)k;
        ++pos;
      }
  if (tid == 1023) {
    *n_out = total;
    *status = total > cap ? bit : 0u;
  }
}

}  // namespace

hipError_t launch_compact(const uint8_t* flag, int64_t N, int32_t* rows, int cap, int32_t* n_out,
                          uint32_t* status, uint32_t bit, hipStream_t s) {
  TWELL_LAUNCH("compact_flags", compact_flags, 1, 1024, 0, s, flag, N, rows, cap, n_out, status, bit);
  return hipGetLastError();
}

}  // namespace twell
