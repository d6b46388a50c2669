// Heaviest-first order of 4-row blocks for the down projection (fused_fwd.hip).
//
// Its kernel gives a wave one row and one d_model slice, four rows to a
// workgroup, and walks the row's whole list; with skewed rows (lists several
// times the mean) a heavy block dispatched near the end of the grid leaves
// the GPU waiting on it. Dispatching blocks in descending weight class (the
// bit length of the block's longest list) lets the short ones fill in behind
// the long ones. The order only permutes which workgroup takes which block,
// so every result is the same bit for bit.
//
//   block_classes  called by a 256-thread workgroup owning 256 consecutive
//                  rows: each 4-row block's class and its rank among the
//                  workgroup's blocks of that class (rb_code), and the
//                  workgroup's count per class (rb_hist)
//   order_blocks   one workgroup: class bases (heavier first), per-workgroup
//                  offsets by a scan, then every block's position
#pragma once

#include "twell_device.h"

namespace twell {
namespace blkord {

constexpr int kClasses = 16;
constexpr int kOrderWgs = 1024;  // 256-row workgroups one ordering workgroup handles

inline bool order_fits(int64_t N) { return (N + 255) / 256 <= kOrderWgs; }

// Every thread of the workgroup calls this with the work of its row
// blockIdx.x * 256 + threadIdx.x (0 past the batch).
__device__ __forceinline__ void block_classes(int len, int64_t N, int32_t* __restrict__ rb_code,
                                              int32_t* __restrict__ rb_hist) {
  __shared__ int cls[64];
  len = max(len, __shfl_xor(len, 1, 64));
  len = max(len, __shfl_xor(len, 2, 64));
  if ((threadIdx.x & 3) == 0) cls[threadIdx.x >> 2] = min(len == 0 ? 0 : 32 - __clz(len), kClasses - 1);
  __syncthreads();
  const int64_t n_rb = (N + 3) / 4;
  const int t = threadIdx.x;
  if (t < 64 && (int64_t)blockIdx.x * 64 + t < n_rb) {
    const int c = cls[t];
    int r = 0;
    for (int u = 0; u < t; ++u) r += cls[u] == c;
    rb_code[(size_t)blockIdx.x * 64 + t] = (c << 16) | r;
  }
  if (t < kClasses) {
    int n = 0;
    for (int u = 0; u < 64 && (int64_t)blockIdx.x * 64 + u < n_rb; ++u) n += cls[u] == t;
    rb_hist[(size_t)blockIdx.x * kClasses + t] = n;
  }
}

namespace {

// One workgroup of 1024 threads (order_fits(N)): heavier classes first,
// within a class by workgroup, then by rank (deterministic).
__global__ __launch_bounds__(1024) void order_blocks(int64_t N, const int32_t* __restrict__ rb_code,
                                                     const int32_t* __restrict__ rb_hist,
                                                     int32_t* __restrict__ rb_order) {
  __shared__ int wtot[16][kClasses];
  __shared__ int base[kClasses];
  __shared__ int woff[kOrderWgs][kClasses];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t n_rb = (N + 3) / 4;
  const int n_wg = (int)((N + 255) / 256);
  int h[kClasses], x[kClasses];
#pragma unroll
  for (int c = 0; c < kClasses; ++c) {
    h[c] = t < n_wg ? rb_hist[(size_t)t * kClasses + c] : 0;
    x[c] = h[c];
  }
  // inclusive scan over the threads, per class: within the wave, then over waves
#pragma unroll
  for (int off = 1; off < 64; off <<= 1)
#pragma unroll
    for (int c = 0; c < kClasses; ++c) {
      const int y = __shfl_up(x[c], off, 64);
      if (lane >= off) x[c] += y;
    }
  if (lane == 63)
#pragma unroll
    for (int c = 0; c < kClasses; ++c) wtot[wave][c] = x[c];
  __syncthreads();
  if (t < kClasses) {  // blocks of heavier classes come first
    int tot = 0;
    for (int c2 = kClasses - 1; c2 > t; --c2)
      for (int w = 0; w < 16; ++w) tot += wtot[w][c2];
    base[t] = tot;
  }
  __syncthreads();
  if (t < n_wg) {
#pragma unroll
    for (int c = 0; c < kClasses; ++c) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wtot[w][c];
      woff[t][c] = base[c] + before + x[c] - h[c];
    }
  }
  __syncthreads();
  constexpr int U = 4;  // blocks whose codes are loaded together
  for (int64_t rb0 = t; rb0 < n_rb; rb0 += (int64_t)U * 1024) {
    int code[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rb = rb0 + (int64_t)u * 1024;
      code[u] = rb < n_rb ? rb_code[rb] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rb = rb0 + (int64_t)u * 1024;
      if (rb < n_rb) {
        const int64_t dst = (int64_t)woff[rb / 64][code[u] >> 16] + (code[u] & 0xffff);
        if (dst < n_rb) rb_order[dst] = (int32_t)rb;  // a permutation: every position written once
      }
    }
  }
}

}  // namespace
}  // namespace blkord
}  // namespace twell
