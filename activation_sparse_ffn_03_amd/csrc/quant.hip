// Per-row FP8 E4M3 quantisation of the gate projection's operands.
//
// "How TwELL by Sakana AI and NVIDIA Accelerates LLMs by 20% Using
// Unstructured Sparsity", "Long-term Impact", names TwELL combined with 8-bit
// quantisation as a direction; the scheme here (one fp32 scale per row equal
// to the row's largest magnitude / 448, elements rounded to the nearest E4M3
// value with ties to even) is this library's reading.
//
// One workgroup per row: the row's largest magnitude (exact), scale =
// max / 448 in fp32 (1 for an all-zero row), then every element x / scale
// (IEEE fp32 division) encoded to E4M3: sign bit, 4 exponent bits with bias
// 7, 3 mantissa bits, subnormals m * 2^-9, magnitudes of 448 and above
// saturated to 448, NaN to 0x7F. Memory-bound: reads the row once from L2
// after the reduction pass.
#include "twell_device.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

// Nearest E4M3 code of v, ties to the even code (integer arithmetic on the
// fp32 encoding).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;              // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;      // |v| >= 448: saturate
  const int e = (int)(a >> 23) - 127;             // floor(log2 |v|) for normals
  if (e < -6) {                                   // below 2^-6: quantum 2^-9
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, then ties-to-even
    return sign | (uint32_t)m;                    // m = 8 is the code of 2^-6
  }
  const uint32_t mant = a & 0x7FFFFFu;
  uint32_t q = mant >> 20;                        // 3 kept bits
  const uint32_t rem = mant & 0xFFFFFu, half = 0x80000u;
  if (rem > half || (rem == half && (q & 1u))) ++q;  // may carry into the exponent
  uint32_t code = ((uint32_t)(e + 7) << 3) + q;
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

template <typename TS>
__global__ __launch_bounds__(256) void quantize_rows_e4m3(const TS* __restrict__ in, int64_t rows, int cols,
                                                          uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float wmax[4];
  const int64_t r = blockIdx.x;
  if (r >= rows) return;
  const TS* row = in + (size_t)r * cols;
  float m = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) m = fmaxf(m, fabsf(Store<TS>::load(row, c)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float sc = m > 0.f ? m / 448.0f : 1.0f;
  if (threadIdx.x == 0) scale[r] = sc;
  uint8_t* qrow = q + (size_t)r * cols;
  // four codes per 32-bit store where the row allows it
  if ((cols & 3) == 0) {
    for (int c4 = threadIdx.x; c4 < cols / 4; c4 += 256) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) w |= e4m3_code(Store<TS>::load(row, 4 * c4 + k) / sc) << (8 * k);
      reinterpret_cast<uint32_t*>(qrow)[c4] = w;
    }
  } else {
    for (int c = threadIdx.x; c < cols; c += 256) qrow[c] = (uint8_t)e4m3_code(Store<TS>::load(row, c) / sc);
  }
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* in, int is_bf16, int64_t rows, int cols, uint8_t* q, float* scale,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (is_bf16)
    TWELL_LAUNCH("quantize_e4m3", quantize_rows_e4m3<uint16_t>, dim3((unsigned)rows), 256, 0, s,
                 (const uint16_t*)in, rows, cols, q, scale);
  else
    TWELL_LAUNCH("quantize_e4m3", quantize_rows_e4m3<float>, dim3((unsigned)rows), 256, 0, s, (const float*)in,
                 rows, cols, q, scale);
  return hipGetLastError();
}

}  // namespace twell
