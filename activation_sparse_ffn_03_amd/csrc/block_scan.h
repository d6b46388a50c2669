// Workgroup-wide exclusive sum for 1024-thread workgroups (wave64), shared by
// the single-workgroup passes: the row offsets of the backward and the
// ascending row lists.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

// Exclusive sum over the 1024 threads of the block of v (wave scans, then the
// 16 wave totals through LDS); *total gets the block's sum. wsum is a
// __shared__ int32_t[16]; every thread of the block must call this (it holds
// two barriers), and wsum may be reused by a following call.
__device__ __forceinline__ int32_t block_excl_1024(int32_t v, int32_t* wsum, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int32_t t = wsum[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

}  // namespace twell
