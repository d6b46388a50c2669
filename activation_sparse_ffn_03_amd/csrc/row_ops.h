// Register-resident row helpers for the wave-per-row sparse kernels.
//
// A row of D elements is held by one wave as 16-byte chunks: chunk q covers
// elements [q*E, q*E+E) (E = 8 for bf16, 4 for fp32) and lane l owns chunks
// q = m*64 + l for m < M. Loads of one row are therefore fully coalesced.
#pragma once

#include "twell_device.h"

namespace twell {

template <typename TS> struct ChunkElems;
template <> struct ChunkElems<uint16_t> { static constexpr int E = 8; };
template <> struct ChunkElems<float> { static constexpr int E = 4; };

template <typename TS, int M>
__device__ __forceinline__ void load_row(u32x4_t (&r)[M], const TS* __restrict__ base, int nch, int lane) {
  constexpr int E = ChunkElems<TS>::E;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int q = m * 64 + lane;
    r[m] = q < nch ? *reinterpret_cast<const u32x4_t*>(base + (size_t)q * E) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Per-lane partial dot product of two register rows (4 independent chains).
template <typename TS, int M>
__device__ __forceinline__ float dot_rows(const u32x4_t (&a)[M], const u32x4_t (&b)[M]) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if constexpr (ChunkElems<TS>::E == 8) {
      s0 = dot2_bf16(a[m].x, b[m].x, s0);
      s1 = dot2_bf16(a[m].y, b[m].y, s1);
      s2 = dot2_bf16(a[m].z, b[m].z, s2);
      s3 = dot2_bf16(a[m].w, b[m].w, s3);
    } else {
      s0 = fmaf(__uint_as_float(a[m].x), __uint_as_float(b[m].x), s0);
      s1 = fmaf(__uint_as_float(a[m].y), __uint_as_float(b[m].y), s1);
      s2 = fmaf(__uint_as_float(a[m].z), __uint_as_float(b[m].z), s2);
      s3 = fmaf(__uint_as_float(a[m].w), __uint_as_float(b[m].w), s3);
    }
  }
  return (s0 + s1) + (s2 + s3);
}

// acc += z * row  (acc[m][e] is element m-chunk, position e)
template <typename TS, int M>
__device__ __forceinline__ void axpy_row(float (&acc)[M][8], float z, const u32x4_t (&w)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if constexpr (ChunkElems<TS>::E == 8) {
      acc[m][0] = fmaf(z, bf16lo_to_f32(w[m].x), acc[m][0]);
      acc[m][1] = fmaf(z, bf16hi_to_f32(w[m].x), acc[m][1]);
      acc[m][2] = fmaf(z, bf16lo_to_f32(w[m].y), acc[m][2]);
      acc[m][3] = fmaf(z, bf16hi_to_f32(w[m].y), acc[m][3]);
      acc[m][4] = fmaf(z, bf16lo_to_f32(w[m].z), acc[m][4]);
      acc[m][5] = fmaf(z, bf16hi_to_f32(w[m].z), acc[m][5]);
      acc[m][6] = fmaf(z, bf16lo_to_f32(w[m].w), acc[m][6]);
      acc[m][7] = fmaf(z, bf16hi_to_f32(w[m].w), acc[m][7]);
    } else {
      acc[m][0] = fmaf(z, __uint_as_float(w[m].x), acc[m][0]);
      acc[m][1] = fmaf(z, __uint_as_float(w[m].y), acc[m][1]);
      acc[m][2] = fmaf(z, __uint_as_float(w[m].z), acc[m][2]);
      acc[m][3] = fmaf(z, __uint_as_float(w[m].w), acc[m][3]);
    }
  }
}

template <int M>
__device__ __forceinline__ void zero_acc(float (&acc)[M][8]) {
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
}

template <typename TS, int M>
__device__ __forceinline__ void store_row(float* __restrict__ dst, const float (&acc)[M][8], int nch, int lane) {
  constexpr int E = ChunkElems<TS>::E;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int q = m * 64 + lane;
    if (q < nch) {
      float4* d = reinterpret_cast<float4*>(dst + (size_t)q * E);
      d[0] = make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
      if constexpr (E == 8) d[1] = make_float4(acc[m][4], acc[m][5], acc[m][6], acc[m][7]);
    }
  }
}

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Dispatch helper: smallest M in {1,2,4,8,16} with M*64 chunks covering nch.
inline int pick_m(int nch) {
  int m = 1;
  while (m * 64 < nch) m *= 2;
  return m;
}

}  // namespace twell
