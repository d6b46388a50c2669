// Deterministic single-workgroup compaction used for the overflow-row list
// (TwELL) and the dense-backup row list (hybrid format). Both lists are in
// ascending row order, the reading taken for the pages' "routes rows" (no
// order is stated there).
#include "twell_device.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

__global__ __launch_bounds__(1024) void compact_flags(const uint8_t* __restrict__ flag, int64_t N, int32_t* rows,
                                                      int cap, int32_t* n_out, uint32_t* status, uint32_t bit) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t chunk = (N + 1023) / 1024;
  const int64_t b = min(N, (int64_t)tid * chunk), en = min(N, b + chunk);
  int32_t c = 0;
  for (int64_t i = b; i < en; ++i) c += flag[i] != 0;
  part[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t pos = part[tid] - c;
  for (int64_t i = b; i < en; ++i)
    if (flag[i]) {
      if (pos < cap) rows[pos] = (int32_t)i;
      ++pos;
    }
  if (tid == 1023) {
    *n_out = part[1023];
    *status = part[1023] > cap ? bit : 0u;
  }
}

}  // namespace

hipError_t launch_compact(const uint8_t* flag, int64_t N, int32_t* rows, int cap, int32_t* n_out,
                          uint32_t* status, uint32_t bit, hipStream_t s) {
  TWELL_LAUNCH("compact_flags", compact_flags, 1, 1024, 0, s, flag, N, rows, cap, n_out, status, bit);
  return hipGetLastError();
}

}  // namespace twell
