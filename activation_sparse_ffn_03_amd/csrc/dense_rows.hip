// Overflow rows of the forward on the matrix cores.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// a row whose activations do not fit the ELL slots is kept in a dense form
// instead. Its share of the up / down projection is then an ordinary dense
// product, and all overflow rows together make two skinny products:
//
//   a = X_o . W_up^T        X_o: the overflow rows of x, gathered (rows x d_model)
//   z = h * a               h: their dense activation rows (ovf_h)
//   y_o = z . W_down        (rows x d_model)
//
// With a few dozen rows these are bound by streaming the two weights, so each
// weight is read once per block of 64 overflow rows and the arithmetic runs on
// v_mfma_f32_16x16x32_bf16:
//
//   dense_up_mfma    a wave owns 16 columns of W_up and runs over all of
//                    d_model in 32-element steps (both operands are
//                    d_model-contiguous, so each lane loads 16 bytes of a row
//                    straight into its MFMA operand). No LDS, no barrier and
//                    few registers, so it runs beside the up projection, which
//                    holds all of a CU's LDS (measured on the 8192 x 4096 x
//                    14336 forward with 64 overflow rows: 2.13-2.17 ms per
//                    forward against 2.23-2.32 with 16 or 32 columns and
//                    4 or 8 steps per batch of loads, and 2.26 with the
//                    overflow branch in order on one stream). z = h*a
//                    (fp32) is stored as two bf16 numbers, z_hi = RNE(z) and
//                    z_lo = RNE(z - z_hi), which together carry 16 significant
//                    bits.
//   dense_down_mfma  W_down is [d_ff][d_model]: the contraction index is its
//                    row, so the 8 consecutive k an MFMA B operand takes from
//                    one lane are 8 different rows. Each lane loads an 8 x 8
//                    block (8 rows, 16 bytes each; 16 lanes cover 128
//                    contiguous columns of a row) and regroups it in registers
//                    into 8 B operands, one per column of its 8. z_hi and z_lo
//                    go through the same B operand (two MFMAs, fp32
//                    accumulation). d_ff is split into kDenseChunk chunks; each
//                    chunk's partial y goes to part[o][chunk][:] and
//                    dense_reduce adds the chunks in order (deterministic).
//
// gate_rows_skinny computes the overflow rows' dense activations h for the
// gate itself in the same way; its chain of MFMAs per output is the gate
// GEMM's, so h is bit-identical to what the pack epilogue saw.
//
// Rows past the overflow count load zeros and are not stored; so are columns
// past d_ff. Rows beyond the first 64 take further passes (the weights are
// streamed again per 64 rows).
#include "skinny_mfma.h"
#include "twell_device.h"
#include "twell_host.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

using namespace skinny;

// Dense activation rows of the overflow rows: h = Q(ReLU(g - t)) with g from
// the same instruction chain as the gate GEMM's pack epilogue (bit-identical
// g, so h is what the pack saw).
template <int UW, int B>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gate_rows_skinny(const uint16_t* __restrict__ x,
                                                                        const uint16_t* __restrict__ w, int D, int F,
                                                                        const int32_t* __restrict__ rows,
                                                                        const int32_t* __restrict__ n_ptr, int cap,
                                                                        const float* __restrict__ t,
                                                                        uint16_t* __restrict__ ovf_h) {
  const int lane = threadIdx.x & 63;
  int c0;
  const uint16_t* wrow[UW];
  if (!skinny_columns<UW>(w, D, F, c0, wrow)) return;
  const int n = min(*n_ptr, cap);
  for (int m0 = blockIdx.z * kRowsPerPass; m0 < n; m0 += gridDim.z * kRowsPerPass) {
    f32x4_t acc[NF][UW];
    skinny_nt<UW, B>(x, rows, n, m0, wrow, D, acc);
    // 16x16 MFMA result: lane l holds rows 4*(l>>4)+r of column l&15
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = m0 + 16 * f + 4 * (lane >> 4) + r;
        if (o >= n) continue;
        const float tv = t[rows[o]];
#pragma unroll
        for (int u = 0; u < UW; ++u) {
          const int col = c0 + 16 * u + (lane & 15);
          const float g = acc[f][u][r];
          if (col < F) ovf_h[(size_t)o * F + col] = g > tv ? f32_to_bf16(g - tv) : uint16_t(0);
        }
      }
  }
}

// z = h * (X_o . W_up^T) of the overflow rows, stored as bf16 high and low
// parts (rows of stride Fz).
template <int UW, int B>
__global__ __launch_bounds__(64 * kSkinnyWaves) void dense_up_mfma(const uint16_t* __restrict__ x,
                                                                     const int32_t* __restrict__ rows,
                                                                     const int32_t* __restrict__ n_ptr, int cap,
                                                                     const uint16_t* __restrict__ w,
                                                                     const uint16_t* __restrict__ h, int D, int F,
                                                                     int Fz, uint16_t* __restrict__ zhi,
                                                                     uint16_t* __restrict__ zlo) {
  const int lane = threadIdx.x & 63;
  int c0;
  const uint16_t* wrow[UW];
  if (!skinny_columns<UW>(w, D, F, c0, wrow)) return;
  const int n = min(*n_ptr, cap);
  for (int m0 = blockIdx.z * kRowsPerPass; m0 < n; m0 += gridDim.z * kRowsPerPass) {
    f32x4_t acc[NF][UW];
    skinny_nt<UW, B>(x, rows, n, m0, wrow, D, acc);
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = m0 + 16 * f + 4 * (lane >> 4) + r;
        if (o >= n) continue;
#pragma unroll
        for (int u = 0; u < UW; ++u) {
          const int col = c0 + 16 * u + (lane & 15);
          if (col < F) {
            const float z = bf16_to_f32(h[(size_t)o * F + col]) * acc[f][u][r];
            const uint16_t hi = f32_to_bf16(z);
            zhi[(size_t)o * Fz + col] = hi;
            zlo[(size_t)o * Fz + col] = f32_to_bf16(z - bf16_to_f32(hi));
          }
        }
      }
  }
}

// Wave (d_model tile of 128 columns, d_ff chunk g): partial y of the chunk.
__global__ __launch_bounds__(64 * kDownWaves) void dense_down_mfma(const uint16_t* __restrict__ zhi,
                                                                     const uint16_t* __restrict__ zlo,
                                                                     const uint16_t* __restrict__ w,
                                                                     const int32_t* __restrict__ n_ptr, int cap, int D,
                                                                     int F, int Fz, int G, float* __restrict__ part) {
  NnOperands<1> p;
  p.hi[0] = zhi;
  p.lo[0] = zlo;
  p.w[0] = w;
  skinny_nn<1>(p, min(*n_ptr, cap), D, F, Fz, G, part);
}

}  // namespace

bool dense_mfma_applies(const FwdArgs& a) { return a.is_bf16 && a.D % kDownCols == 0 && a.zov != nullptr; }

bool gate_rows_skinny_applies(int D) { return D % 32 == 0; }

hipError_t launch_gate_rows_skinny(const uint16_t* x, const uint16_t* w, int D, int F, const int32_t* rows,
                                   const int32_t* n_ovf, int cap, const float* t, uint16_t* ovf_h, hipStream_t s) {
  if (!gate_rows_skinny_applies(D)) return hipErrorInvalidValue;
  TWELL_LAUNCH("gate_rows_skinny", (gate_rows_skinny<kSkinnyUW, kSkinnyB>),
               dim3(skinny_blocks(F, kSkinnyUW), 1, kPassSplit),
               64 * kSkinnyWaves, 0, s, x, w, D, F, rows, n_ovf, cap, t, ovf_h);
  return hipGetLastError();
}

hipError_t launch_dense_mfma(const FwdArgs& a, hipStream_t s) {
  if (!dense_mfma_applies(a)) return hipErrorInvalidValue;
  const int Fz = dense_z_stride(a.F);
  const int G = (a.F + kDenseChunk - 1) / kDenseChunk;
  uint16_t* zhi = a.zov;
  uint16_t* zlo = a.zov + (size_t)a.ovf_cap * Fz;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);
  TWELL_LAUNCH("dense_up_mfma", (dense_up_mfma<kSkinnyUW, kSkinnyB>),
               dim3(skinny_blocks(a.F, kSkinnyUW), 1, kPassSplit),
               64 * kSkinnyWaves, 0, s, x, a.ovf_rows, a.n_ovf, a.ovf_cap, reinterpret_cast<const uint16_t*>(a.w_up),
               reinterpret_cast<const uint16_t*>(a.ovf_h), a.D, a.F, Fz, zhi, zlo);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  TWELL_LAUNCH("dense_down_mfma", dense_down_mfma, skinny_nn_grid(a.D, G),
               64 * kDownWaves, 0, s, zhi, zlo, reinterpret_cast<const uint16_t*>(a.w_down), a.n_ovf, a.ovf_cap, a.D,
               a.F, Fz, G, a.part);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_dense_reduce(a.part, a.ovf_rows, a.n_ovf, a.ovf_cap, G, a.D, a.y, s);
}

}  // namespace twell
