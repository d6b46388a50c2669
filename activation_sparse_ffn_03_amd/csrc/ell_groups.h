// Per-row group positions of the row-ELL, for the blocked dz (bwd_blocked.hip):
// the ELL position of each ELL row's first entry in every group of
// blk::kGroupCols columns (its columns ascend).
#pragma once

#include "blocked_sddmm.h"
#include "twell_kernels.h"

namespace twell {

// One wave, row i (lane = ELL position): egrp[g][i] = ELL position of the
// first entry of row i with column >= g * kGroupCols, for g = 0 .. n_groups
// (0 everywhere for dense rows). Entry k writes the groups after its
// predecessor's up to its own; the first position past the row's end writes
// the rest, so every egrp value is written exactly once.
__device__ __forceinline__ void ell_groups_row(const BwdArgs& a, int n_groups, int64_t i) {
  const int lane = threadIdx.x & 63;
  const int64_t N = a.N;
  const int n = a.is_dense[i] ? 0 : min(a.row_nnz[i], a.row_cap);
  int32_t* eg = a.ws.egrp + i;  // row g at eg[g * N]
  int prev_last = -1;           // group of position kb - 1
  for (int kb = 0; kb <= n; kb += 64) {
    const int k = kb + lane;
    // group of position k; positions at or past the end count as group n_groups
    const int cur = k < n ? (int)min((unsigned)a.ell_cols[(size_t)k * N + i] / blk::kGroupCols,
                                     (unsigned)n_groups - 1)
                          : n_groups;
    int prev = __shfl_up(cur, 1, 64);
    if (lane == 0) prev = prev_last;
    if (k <= n)
      for (int g = prev + 1; g <= cur; ++g) eg[(size_t)g * N] = k;
    prev_last = __shfl(cur, 63, 64);
  }
}

}  // namespace twell
