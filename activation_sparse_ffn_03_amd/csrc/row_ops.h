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

// EPL consecutive storage elements per lane, loaded with one or two vector
// loads and widened to fp32.
template <typename TS, int EPL> struct Slice;
template <int EPL> struct Slice<uint16_t, EPL> {
  static constexpr int W = EPL >= 2 ? EPL / 2 : 1;  // 32-bit words (EPL == 1 uses the low half)
  uint32_t w[W];
  __device__ __forceinline__ void load(const uint16_t* p) {
    if constexpr (EPL == 1) {
      w[0] = *p;
    } else if constexpr (EPL == 2) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (EPL == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < EPL / 8; ++q) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p + q * 8);
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
    }
  }
  __device__ __forceinline__ void fma(float z, float (&acc)[EPL]) const {
    if constexpr (EPL == 1) {
      acc[0] = fmaf(z, bf16lo_to_f32(w[0]), acc[0]);
    } else {
#pragma unroll
      for (int q = 0; q < W; ++q) {
        acc[2 * q] = fmaf(z, bf16lo_to_f32(w[q]), acc[2 * q]);
        acc[2 * q + 1] = fmaf(z, bf16hi_to_f32(w[q]), acc[2 * q + 1]);
      }
    }
  }
};
template <int EPL> struct Slice<float, EPL> {
  float w[EPL];
  __device__ __forceinline__ void load(const float* p) {
    if constexpr (EPL == 1) {
      w[0] = *p;
    } else if constexpr (EPL == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < EPL / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(p + q * 4);
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
    }
  }
  __device__ __forceinline__ void fma(float z, float (&acc)[EPL]) const {
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(z, w[e], acc[e]);
  }
};

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// d_model slicing of the sliced gather kernels. d_model is cut into P slices
// (P = 8, one per XCD, whenever the slice length is then a power of two); a
// row's slice is read by LPR lanes with EPL elements each, 16 bytes per lane
// wherever the slice allows, so one wave load instruction covers RPI = 64/LPR
// rows. Load instructions, not bytes, bound these gathers on MI355X: 16-byte
// lanes move twice the data per instruction of 8-byte lanes.
struct SliceGeom {
  int P, EPL, RPI;
};
inline SliceGeom pick_slices(int D, int esz) {
  const int e16 = 16 / esz;
  int P = 0, slice = 0;
  for (int p = 8; p >= 1; p >>= 1) {
    const int sl = D / p;
    if (D % p == 0 && (sl & (sl - 1)) == 0 && sl >= e16) {
      P = p;
      slice = sl;
      break;
    }
  }
  if (P == 0) {  // d_model is not a power of two times <= 8: 64-element slices
    P = D / 64;
    slice = 64;
  }
  const int lpr = slice / e16 >= 64 ? 64 : slice / e16;
  return {P, slice / lpr, 64 / lpr};
}

// Slicing for a pass that gathers slices of the rows of one [rows x D] matrix:
// the slice is the widest power of two (down to 64 elements, and never wider
// than pick_slices gives) whose column of the matrix, rows x slice, fits the
// budget: by default 3.75 MB of an XCD's 4 MB L2 (dx of the training step:
// 4.2 MB slices measured slower there); the down projection passes its own. geom.P is then the total number of slices; they
// are processed 8 at a time (one per XCD), in P/8 successive passes.
inline SliceGeom pick_l2_slices(int D, int esz, int64_t rows, int64_t budget = 15ll << 18) {
  SliceGeom g = pick_slices(D, esz);
  const int e16 = 16 / esz;
  int slice = D / g.P;
  while (slice > 64 && slice % 2 == 0 && (int64_t)slice / 2 >= e16 && rows * slice * esz > budget) slice /= 2;
  const int lpr = slice / e16 >= 64 ? 64 : slice / e16;
  return {D / slice, slice / lpr, 64 / lpr};
}

// Workgroup b of a sliced launch over `blocks` row blocks and P slices that go
// G8 at a time (slice_group): slice pass * G8 + b % G8 and row block
// (b / G8) % blocks, passes in grid order. Workgroups are dealt to the 8 XCDs
// round-robin, so with G8 = 8 each XCD holds one slice at a time.
__device__ __forceinline__ void slice_block(int64_t b, int G8, int64_t blocks, int& p, int64_t& rb) {
  const int64_t r = b / G8;
  p = (int)(r / blocks) * G8 + (int)(b % G8);
  rb = r % blocks;
}
// Slices per pass: 8 (one per XCD) when they divide P, else all P in one pass.
inline int slice_group(int P) { return P % 8 == 0 ? 8 : P; }

// Load instructions a sliced gather keeps in flight per wave: 4 KB per wave
// whatever the slice width (RPI = 1 loads one row per instruction), but no
// more rows than one 64-entry list holds.
template <int RPI>
constexpr int sliced_inflight() { return RPI == 1 ? 8 : (64 / RPI < 4 ? 64 / RPI : 4); }

// acc += sum over the list entries k < n of z_k * row(c_k)[slice], where lane
// k of (c_l, z_l) holds entry k and `base` already points at this lane's slice
// elements. Lane group g = lane / (64/RPI) takes entries g, g+RPI, ...; U load
// instructions (U*RPI rows) are in flight at a time. Entries whose column is
// outside [0, F) contribute nothing.
template <typename TS, int EPL, int RPI, int U>
__device__ __forceinline__ void sliced_axpy(const TS* __restrict__ base, int D, int F, int c_l, float z_l, int n,
                                            int lane, float (&acc)[EPL]) {
  constexpr int LPR = 64 / RPI;
  const int g = lane / LPR;
  for (int k = 0; k < n; k += U * RPI) {
    Slice<TS, EPL> w[U];
    float z[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + u * RPI + g;
      const int ks = kk < n ? kk : n - 1;
      int c;
      float zz;
      if constexpr (RPI == 1) {  // ks is wave-uniform
        c = __builtin_amdgcn_readlane(c_l, ks);
        zz = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z_l), ks));
      } else {
        c = __shfl(c_l, ks, 64);
        zz = __shfl(z_l, ks, 64);
      }
      const bool ok = kk < n && (unsigned)c < (unsigned)F;
      z[u] = ok ? zz : 0.f;
      w[u].load(base + (size_t)(ok ? c : 0) * D);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) w[u].fma(z[u], acc);
  }
}

// Add up the partial slices of the RPI lane groups (lanes l, l + 64/RPI, ...
// hold the same slice elements); afterwards group 0 holds the total.
template <int EPL, int RPI>
__device__ __forceinline__ void combine_groups(float (&acc)[EPL]) {
#pragma unroll
  for (int off = 32; off >= 64 / RPI; off >>= 1)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
}

// Dispatch a sliced kernel template K<EPL, RPI> for the runtime geometry.
#define TWELL_SLICED_CASES(E16, CALL)                                                       \
  switch (geom.EPL == E16 ? geom.RPI : (geom.EPL == 2 * E16 ? 100 + geom.RPI : -1)) {      \
    case 1: CALL(E16, 1); break;                                                            \
    case 2: CALL(E16, 2); break;                                                            \
    case 4: CALL(E16, 4); break;                                                            \
    case 8: CALL(E16, 8); break;                                                            \
    case 16: CALL(E16, 16); break;                                                          \
    case 32: CALL(E16, 32); break;                                                          \
    case 64: CALL(E16, 64); break;                                                          \
    case 101: CALL(2 * E16, 1); break;                                                      \
    default: return hipErrorInvalidValue;                                                   \
  }

// Dispatch helper: smallest M in {1,2,4,8,16} with M*64 chunks covering nch.
inline int pick_m(int nch) {
  int m = 1;
  while (m * 64 < nch) m *= 2;
  return m;
}

}  // namespace twell
