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
#include "twell_device.h"
#include "twell_host.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int kRowsPerPass = 64;  // 4 MFMA row fragments
constexpr int NF = kRowsPerPass / 16;
constexpr int kSkinnyWaves = 4;   // waves per workgroup of the skinny NT kernels (independent)
constexpr int kSkinnyUW = 1;      // 16-column groups per wave
constexpr int kSkinnyB = 2;       // 32-element steps per batch of loads

// One wave: acc[f][u] = rows m0 + 16f + (0..15) (gathered through `rows`, zero
// past n) times columns c0 + 16u + (0..15) of w, over all of d_model in
// ascending 32-element steps, one v_mfma_f32_16x16x32_bf16 per step and
// fragment pair. Lane l supplies row l & 15 and elements 8*(l >> 4) .. +7 of
// each step for both operands, exactly as the gate GEMM's LDS fragments do, so
// every output is accumulated by the same chain of instructions as there.
template <int UW, int B>
__device__ __forceinline__ void skinny_nt(const uint16_t* __restrict__ x, const int32_t* __restrict__ rows, int n,
                                          int m0, const uint16_t* const (&wrow)[UW], int D, f32x4_t (&acc)[NF][UW]) {
  const int lane = threadIdx.x & 63;
  const int ko = (lane >> 4) * 8;
  const uint16_t* xrow[NF];
  bool xok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int o = m0 + 16 * f + (lane & 15);
    xok[f] = o < n;
    xrow[f] = x + (size_t)(xok[f] ? rows[o] : 0) * D + ko;
  }
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int u = 0; u < UW; ++u) acc[f][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero{0u, 0u, 0u, 0u};
  const int S = D / 32;
  for (int s0 = 0; s0 < S; s0 += B) {
    u32x4_t bv[B][UW], av[B][NF];
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int u = 0; u < UW; ++u)
        bv[j][u] = s0 + j < S ? *reinterpret_cast<const u32x4_t*>(wrow[u] + (size_t)(s0 + j) * 32) : zero;
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        av[j][f] = (s0 + j < S && xok[f]) ? *reinterpret_cast<const u32x4_t*>(xrow[f] + (size_t)(s0 + j) * 32) : zero;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (s0 + j >= S) break;  // wave-uniform
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int u = 0; u < UW; ++u)
          acc[f][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[j][f]),
                                                              __builtin_bit_cast(bf16x8_t, bv[j][u]), acc[f][u], 0, 0,
                                                              0);
    }
  }
}

// Wave w of the grid owns columns [16*UW*w, 16*UW*(w+1)); past d_ff it exits
// (no barriers). Columns past d_ff read row F - 1 and are never stored.
template <int UW>
__device__ __forceinline__ bool skinny_columns(const uint16_t* __restrict__ w, int D, int F, int& c0,
                                               const uint16_t* (&wrow)[UW]) {
  const int lane = threadIdx.x & 63;
  c0 = (blockIdx.x * kSkinnyWaves + (threadIdx.x >> 6)) * 16 * UW;
  if (c0 >= F) return false;
#pragma unroll
  for (int u = 0; u < UW; ++u) {
    const int col = c0 + 16 * u + (lane & 15);
    wrow[u] = w + (size_t)(col < F ? col : F - 1) * D + (lane >> 4) * 8;
  }
  return true;
}

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
  for (int m0 = 0; m0 < n; m0 += kRowsPerPass) {
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
  for (int m0 = 0; m0 < n; m0 += kRowsPerPass) {
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

unsigned skinny_blocks(int F, int UW) {
  const int waves = (F + 16 * UW - 1) / (16 * UW);
  return (unsigned)((waves + kSkinnyWaves - 1) / kSkinnyWaves);
}

// Column j of an 8x8 block of bf16 held as 8 rows v[0..7] (row i = 8 values in
// 4 dwords): the 8 values v[0][j] .. v[7][j], packed two per dword.
template <int J>
__device__ __forceinline__ bf16x8_t block_column(const u32x4_t (&v)[8]) {
  u32x4_t c;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t a = v[2 * p][J >> 1], b = v[2 * p + 1][J >> 1];
    c[p] = (J & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
  }
  return __builtin_bit_cast(bf16x8_t, c);
}

constexpr int kDownWaves = 4;
constexpr int kDownCols = 128;  // d_model columns per wave: 16 lanes x 8

template <int J>
__device__ __forceinline__ void down_column(const u32x4_t (&v)[8], const u32x4_t (&ah)[NF],
                                            const u32x4_t (&al)[NF], f32x4_t (&acc)[NF][8]) {
  const bf16x8_t b = block_column<J>(v);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    acc[f][J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah[f]), b, acc[f][J], 0, 0, 0);
    acc[f][J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al[f]), b, acc[f][J], 0, 0, 0);
  }
}

// Wave (d_model tile of 128 columns, d_ff chunk g): partial y of the chunk.
__global__ __launch_bounds__(64 * kDownWaves) void dense_down_mfma(const uint16_t* __restrict__ zhi,
                                                                     const uint16_t* __restrict__ zlo,
                                                                     const uint16_t* __restrict__ w,
                                                                     const int32_t* __restrict__ n_ptr, int cap, int D,
                                                                     int F, int Fz, int G, float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int dt = blockIdx.x * kDownWaves + (threadIdx.x >> 6);
  if (dt * kDownCols >= D) return;  // no barriers below
  const int n = min(*n_ptr, cap);
  const int g = blockIdx.y;
  const int dl = dt * kDownCols + 8 * (lane & 15);  // this lane's 8 columns
  const int kq = 8 * (lane >> 4);                   // this lane's 8 rows of a 32-row block
  const int c_lo = g * kDenseChunk, c_hi = min(F, c_lo + kDenseChunk);
  const u32x4_t zero{0u, 0u, 0u, 0u};
  for (int m0 = 0; m0 < n; m0 += kRowsPerPass) {
    const uint16_t* ahp[NF];
    const uint16_t* alp[NF];
    bool aok[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int o = m0 + 16 * f + (lane & 15);
      aok[f] = o < n;
      const size_t ro = (size_t)(aok[f] ? o : 0) * Fz;
      ahp[f] = zhi + ro;
      alp[f] = zlo + ro;
    }
    f32x4_t acc[NF][8];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int cb = c_lo; cb < c_hi; cb += 32) {
      const int k0 = cb + kq;  // first of this lane's 8 rows (k0 + 8 <= Fz)
      u32x4_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = k0 + i < c_hi ? *reinterpret_cast<const u32x4_t*>(w + (size_t)(k0 + i) * D + dl) : zero;
      u32x4_t ah[NF], al[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        ah[f] = aok[f] ? *reinterpret_cast<const u32x4_t*>(ahp[f] + k0) : zero;
        al[f] = aok[f] ? *reinterpret_cast<const u32x4_t*>(alp[f] + k0) : zero;
      }
      if (k0 + 8 > c_hi) {  // the chunk's last, partial block: zero the z of rows past its end
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t keep = (k0 + 2 * q < c_hi ? 0xffffu : 0u) | (k0 + 2 * q + 1 < c_hi ? 0xffff0000u : 0u);
            ah[f][q] &= keep;
            al[f][q] &= keep;
          }
      }
      down_column<0>(v, ah, al, acc);
      down_column<1>(v, ah, al, acc);
      down_column<2>(v, ah, al, acc);
      down_column<3>(v, ah, al, acc);
      down_column<4>(v, ah, al, acc);
      down_column<5>(v, ah, al, acc);
      down_column<6>(v, ah, al, acc);
      down_column<7>(v, ah, al, acc);
    }
    // acc[f][j][r] = partial y[m0 + 16f + 4(lane>>4) + r][dl + j]
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = m0 + 16 * f + 4 * (lane >> 4) + r;
        if (o < n) {
          float4* dst = reinterpret_cast<float4*>(part + ((size_t)o * G + g) * D + dl);
          dst[0] = make_float4(acc[f][0][r], acc[f][1][r], acc[f][2][r], acc[f][3][r]);
          dst[1] = make_float4(acc[f][4][r], acc[f][5][r], acc[f][6][r], acc[f][7][r]);
        }
      }
  }
}

}  // namespace

bool dense_mfma_applies(const FwdArgs& a) { return a.is_bf16 && a.D % kDownCols == 0 && a.zov != nullptr; }

bool gate_rows_skinny_applies(int D) { return D % 32 == 0; }

hipError_t launch_gate_rows_skinny(const uint16_t* x, const uint16_t* w, int D, int F, const int32_t* rows,
                                   const int32_t* n_ovf, int cap, const float* t, uint16_t* ovf_h, hipStream_t s) {
  if (!gate_rows_skinny_applies(D)) return hipErrorInvalidValue;
  TWELL_LAUNCH("gate_rows_skinny", (gate_rows_skinny<kSkinnyUW, kSkinnyB>), dim3(skinny_blocks(F, kSkinnyUW)),
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
  TWELL_LAUNCH("dense_up_mfma", (dense_up_mfma<kSkinnyUW, kSkinnyB>), dim3(skinny_blocks(a.F, kSkinnyUW)),
               64 * kSkinnyWaves, 0, s, x, a.ovf_rows, a.n_ovf, a.ovf_cap, reinterpret_cast<const uint16_t*>(a.w_up),
               reinterpret_cast<const uint16_t*>(a.ovf_h), a.D, a.F, Fz, zhi, zlo);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int dtiles = a.D / kDownCols;
  TWELL_LAUNCH("dense_down_mfma", dense_down_mfma, dim3((unsigned)((dtiles + kDownWaves - 1) / kDownWaves), (unsigned)G),
               64 * kDownWaves, 0, s, zhi, zlo, reinterpret_cast<const uint16_t*>(a.w_down), a.n_ovf, a.ovf_cap, a.D,
               a.F, Fz, G, a.part);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_dense_reduce(a.part, a.ovf_rows, a.n_ovf, a.ovf_cap, G, a.D, a.y, s);
}

}  // namespace twell
