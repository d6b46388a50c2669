// Device-side helpers shared by the libtwell kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// bf16 <-> fp32 on raw 16-bit storage.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 for finite inputs.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Full-wave sum; every lane receives the result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// One DPP step: v + (the value the DPP pattern routes to this lane), lanes
// outside row_mask adding 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Full-wave sum with DPP (GFX9 row broadcasts), returned in every lane:
// quad swaps, half-row and row mirrors give every lane its 16-lane row sum;
// row_bcast:15 and row_bcast:31 fold rows 0..3 into lane 63, read back with
// readlane. Six VALU ops instead of six LDS-crossbar shuffles.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_lane() { return threadIdx.x & (kWave - 1); }

// Maximum of v over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t lanemask_lt_popc(uint64_t m, int lane) {
  return __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}

// Workgroup barrier that orders LDS accesses only (waits for this wave's
// outstanding LDS operations, not for its global loads or stores).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's bytes land at lds_byte + 16 * l, where
// lds_byte is the wave's base address (wave-uniform by construction).
__device__ __forceinline__ void dma_16B(const void* g, uint32_t lds_byte) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory");
}
// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block index of workgroup b of nb such that the workgroups of each XCD (b
// runs on XCD b % 8) take one contiguous run of blocks.
__device__ __forceinline__ int64_t xcd_run_block(int64_t b, int64_t nb) {
  const int x = (int)(b % 8);
  const int64_t q = nb / 8, r = nb % 8;
  return x * q + (x < r ? x : r) + b / 8;
}

// Storage types: raw bf16 bits or fp32.
template <typename T> struct Store;
template <> struct Store<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ uint16_t from_f32(float f) { return f32_to_bf16(f); }
};
template <> struct Store<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ float from_f32(float f) { return f; }
};

}  // namespace twell
