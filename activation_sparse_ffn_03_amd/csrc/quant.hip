// Per-row FP8 E4M3 quantisation of the gate projection's operands.
//
// "How TwELL by Sakana AI and NVIDIA Accelerates LLMs by 20% Using
// Unstructured Sparsity", "Long-term Impact", names TwELL combined with 8-bit
// quantisation as a direction; the scheme here (one fp32 scale per row equal
// to the row's largest magnitude / 448, elements rounded to the nearest E4M3
// value with ties to even) is this library's reading.
//
// One wavefront per row (four rows per workgroup): the row is read once with
// 16-byte loads and kept in registers (rows longer than 64 * 16 * kRegChunks
// bytes re-read the rest from L2), its largest magnitude is reduced across
// the wave, scale = max / 448 in fp32 (1 when that is not > 0: an all-zero
// row, a row whose maximum underflows, and a row holding NaN, since the
// maximum is taken on the magnitudes' bit patterns and NaN wins it), then
// every element x / scale (IEEE fp32
// division) is encoded: sign bit, 4 exponent bits with bias 7, 3 mantissa
// bits, subnormals m * 2^-9, magnitudes of 448 and above saturated to 448,
// NaN to 0x7F (rows with a finite maximum use the hardware conversion, which
// gives the same codes there). Rows whose width or base address does not
// allow 16-byte loads take a scalar path with the same arithmetic.
// HBM-bound: 2 (bf16) or 4 (fp32) bytes read and 1 written per element.
#include "twell_device.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kRegChunks = 8;  // 16-byte chunks per lane held in registers

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

// Element access on raw 32-bit words: bf16 packs two elements per word.
template <typename TS>
struct Words;
template <>
struct Words<uint16_t> {
  static constexpr int kPerWord = 2;
  // largest |x| bit pattern of the word, as an fp32 bit pattern
  __device__ static uint32_t mag_bits(uint32_t w) { return max((w & 0x7FFFu) << 16, w & 0x7FFF0000u); }
  __device__ static float elem(uint32_t w, int k) { return __uint_as_float(k ? (w & 0xFFFF0000u) : (w << 16)); }
  __device__ static uint32_t mag_scalar(uint16_t h) { return ((uint32_t)h & 0x7FFFu) << 16; }
  __device__ static float scalar(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
};
template <>
struct Words<float> {
  static constexpr int kPerWord = 1;
  __device__ static uint32_t mag_bits(uint32_t w) { return w & 0x7FFFFFFFu; }
  __device__ static float elem(uint32_t w, int) { return __uint_as_float(w); }
  __device__ static uint32_t mag_scalar(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }
  __device__ static float scalar(float f) { return f; }
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  return m;
}

// scale of a row from the bit pattern of its largest magnitude: m / 448 in
// fp32, or 1 when that is not > 0 (an all-zero row, a row holding NaN, or a
// maximum so small that the quotient underflows to 0)
__device__ __forceinline__ float row_scale(uint32_t mbits) {
  const float s = __uint_as_float(mbits) / 448.0f;
  return s > 0.f ? s : 1.0f;  // NaN fails the test
}

// Bit pattern of 448 * 2^-126: rows whose largest magnitude is at least this
// have a normal scale, so every quotient stays below 448.001.
constexpr uint32_t kHwMinMaxBits = 0x04E00000u;

// Codes of four quotients with the hardware conversion (v_cvt_pk_fp8_f32,
// round to nearest even). A sweep of all 2^32 fp32 bit patterns on gfx950
// found it equal to e4m3_code for every |v| <= 448, subnormals and -0
// included; it differs only above 464 and on NaN and infinities. A row whose
// largest magnitude m is finite and at least 448 * 2^-126 has a normal scale
// fl(m / 448) and every quotient |x / scale| <= m / fl(m / 448) < 448.001, so
// such rows may take it. (A smaller m gives a subnormal scale, rounded by up
// to half of 2^-149, and quotients up to 512 and beyond.)
__device__ __forceinline__ uint32_t e4m3_codes_hw(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <typename TS, bool HW>
__device__ __forceinline__ void encode_chunk(const u32x4_t& v, float sc, uint8_t* dst) {
  using W = Words<TS>;
  if constexpr (HW) {
    if constexpr (W::kPerWord == 2) {
      const uint32_t lo = e4m3_codes_hw(W::elem(v[0], 0) / sc, W::elem(v[0], 1) / sc, W::elem(v[1], 0) / sc,
                                        W::elem(v[1], 1) / sc);
      const uint32_t hi = e4m3_codes_hw(W::elem(v[2], 0) / sc, W::elem(v[2], 1) / sc, W::elem(v[3], 0) / sc,
                                        W::elem(v[3], 1) / sc);
      *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
    } else {
      *reinterpret_cast<uint32_t*>(dst) = e4m3_codes_hw(W::elem(v[0], 0) / sc, W::elem(v[1], 0) / sc,
                                                        W::elem(v[2], 0) / sc, W::elem(v[3], 0) / sc);
    }
  } else if constexpr (W::kPerWord == 2) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= e4m3_code(W::elem(v[k >> 1], k & 1) / sc) << (8 * k);
      hi |= e4m3_code(W::elem(v[2 + (k >> 1)], k & 1) / sc) << (8 * k);
    }
    *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) w |= e4m3_code(W::elem(v[k], 0) / sc) << (8 * k);
    *reinterpret_cast<uint32_t*>(dst) = w;
  }
}

// 16-byte path: cols * sizeof(TS) % 16 == 0 and 16-byte aligned rows.
template <typename TS>
__global__ __launch_bounds__(64 * kRowsPerBlock) void quantize_rows_vec(const TS* __restrict__ in, int64_t rows,
                                                                         int cols, uint8_t* __restrict__ q,
                                                                         float* __restrict__ scale) {
  using W = Words<TS>;
  constexpr int EPC = 16 / (int)sizeof(TS);  // elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  const u32x4_t* row = reinterpret_cast<const u32x4_t*>(in + r * cols);
  const int nch = cols / EPC;
  u32x4_t v[kRegChunks];
  uint32_t mb = 0;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int i = lane + 64 * c;
    v[c] = i < nch ? row[i] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) mb = max(mb, W::mag_bits(v[c][k]));
  }
  for (int i = lane + 64 * kRegChunks; i < nch; i += 64) {
    const u32x4_t t = row[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) mb = max(mb, W::mag_bits(t[k]));
  }
  const uint32_t mbits = wave_max_u32(mb);
  const float sc = row_scale(mbits);
  if (lane == 0) scale[r] = sc;
  uint8_t* qrow = q + r * cols;
  auto encode = [&](auto hw) {
    constexpr bool HW = decltype(hw)::value;
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
      const int i = lane + 64 * c;
      if (i < nch) encode_chunk<TS, HW>(v[c], sc, qrow + (size_t)i * EPC);
    }
    for (int i = lane + 64 * kRegChunks; i < nch; i += 64) encode_chunk<TS, HW>(row[i], sc, qrow + (size_t)i * EPC);
  };
  // finite largest magnitude with a normal scale (wave-uniform): every
  // quotient is within the hardware conversion's exact range; NaN or infinity
  // in the row, or a subnormal scale: software
  if (mbits < 0x7F800000u && mbits >= kHwMinMaxBits)
    encode(std::true_type{});
  else
    encode(std::false_type{});
}

// Any width and alignment: one element per lane per step, read twice.
template <typename TS>
__global__ __launch_bounds__(64 * kRowsPerBlock) void quantize_rows_scalar(const TS* __restrict__ in, int64_t rows,
                                                                            int cols, uint8_t* __restrict__ q,
                                                                            float* __restrict__ scale) {
  using W = Words<TS>;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  const TS* row = in + r * cols;
  uint32_t mb = 0;
  for (int c = lane; c < cols; c += 64) mb = max(mb, W::mag_scalar(row[c]));
  const float sc = row_scale(wave_max_u32(mb));
  if (lane == 0) scale[r] = sc;
  uint8_t* qrow = q + r * cols;
  for (int c = lane; c < cols; c += 64) qrow[c] = (uint8_t)e4m3_code(W::scalar(row[c]) / sc);
}

template <typename TS>
hipError_t launch_typed(const void* in, int64_t rows, int cols, uint8_t* q, float* scale, hipStream_t s) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const int epc = 16 / (int)sizeof(TS);
  const bool vec = cols % epc == 0 && (uintptr_t)in % 16 == 0 && (uintptr_t)q % 8 == 0;
  if (vec)
    TWELL_LAUNCH("quantize_e4m3", quantize_rows_vec<TS>, grid, 64 * kRowsPerBlock, 0, s, (const TS*)in, rows, cols, q,
                 scale);
  else
    TWELL_LAUNCH("quantize_e4m3", quantize_rows_scalar<TS>, grid, 64 * kRowsPerBlock, 0, s, (const TS*)in, rows, cols,
                 q, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* in, int is_bf16, int64_t rows, int cols, uint8_t* q, float* scale,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  return is_bf16 ? launch_typed<uint16_t>(in, rows, cols, q, scale, s)
                 : launch_typed<float>(in, rows, cols, q, scale, s);
}

}  // namespace twell
