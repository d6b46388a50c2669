// Skinny MFMA products of a few dozen gathered rows against a whole weight
// matrix (the dense overflow / backup rows), shared by the forward's and the
// backward's dense-row paths. Operands are bf16; results are fp32.
#pragma once

#include "twell_device.h"
#include "twell_kernels.h"

namespace twell {
namespace skinny {

constexpr int kRowsPerPass = 64;  // 4 MFMA row fragments
constexpr int NF = kRowsPerPass / 16;
constexpr int kSkinnyWaves = 4;   // waves per workgroup of the skinny NT kernels (independent)
constexpr int kSkinnyUW = 1;      // 16-column groups per wave
constexpr int kSkinnyB = 2;       // 32-element steps per batch of loads
// Passes of kRowsPerPass rows go to kPassSplit workgroups per column group
// (grid z; pass p to workgroup p % kPassSplit), so that above 64 rows the
// passes stream their weights at the same time: a pass is bound by the
// latency of its loads (one wave per SIMD), not by bandwidth.
constexpr int kPassSplit = 2;

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

inline unsigned skinny_blocks(int F, int UW) {
  const int waves = (F + 16 * UW - 1) / (16 * UW);
  return (unsigned)((waves + kSkinnyWaves - 1) / kSkinnyWaves);
}

constexpr int kDownWaves = 4;
constexpr int kDownCols = 128;  // d_model columns per wave: 16 lanes x 8

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

// Skinny NN product in d_ff chunks: for the wave's 128 d_model columns
// [dt*128, dt*128 + 128) and chunk g of d_ff, part[o][g][:] = sum over the
// chunk's columns c and the NP pairs q of A_q[o][c] * W_q[c][:], with A_q held
// as bf16 high and low parts (rows of stride Fz, zero past the row count n)
// and W_q [d_ff][d_model]. W_q's contraction index is its row, so each lane
// loads an 8 x 8 block (8 rows, 16 bytes each; 16 lanes cover 128 contiguous
// columns of a row) and regroups it in registers into 8 B operands, one per
// column of its 8; high and low part go through the same B operand (two
// MFMAs, fp32 accumulation).
template <int NP>
struct NnOperands {
  const uint16_t* hi[NP];
  const uint16_t* lo[NP];
  const uint16_t* w[NP];
};

template <int NP>
__device__ __forceinline__ void skinny_nn(const NnOperands<NP>& p, int n, int D, int F, int Fz, int G,
                                          float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int dt = blockIdx.x * kDownWaves + (threadIdx.x >> 6);
  if (dt * kDownCols >= D) return;  // no barriers below
  const int g = blockIdx.y;
  const int dl = dt * kDownCols + 8 * (lane & 15);  // this lane's 8 columns
  const int kq = 8 * (lane >> 4);                   // this lane's 8 rows of a 32-row block
  const int c_lo = g * kDenseChunk, c_hi = min(F, c_lo + kDenseChunk);
  const u32x4_t zero{0u, 0u, 0u, 0u};
  for (int m0 = blockIdx.z * kRowsPerPass; m0 < n; m0 += gridDim.z * kRowsPerPass) {
    size_t ro[NF];
    bool aok[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int o = m0 + 16 * f + (lane & 15);
      aok[f] = o < n;
      ro[f] = (size_t)(aok[f] ? o : 0) * Fz;
    }
    f32x4_t acc[NF][8];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int cb = c_lo; cb < c_hi; cb += 32) {
      const int k0 = cb + kq;  // first of this lane's 8 rows (k0 + 8 <= Fz)
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        u32x4_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[i] = k0 + i < c_hi ? *reinterpret_cast<const u32x4_t*>(p.w[q] + (size_t)(k0 + i) * D + dl) : zero;
        u32x4_t ah[NF], al[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          ah[f] = aok[f] ? *reinterpret_cast<const u32x4_t*>(p.hi[q] + ro[f] + k0) : zero;
          al[f] = aok[f] ? *reinterpret_cast<const u32x4_t*>(p.lo[q] + ro[f] + k0) : zero;
        }
        if (k0 + 8 > c_hi) {  // the chunk's last, partial block: zero A past its end
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t keep = (k0 + 2 * e < c_hi ? 0xffffu : 0u) | (k0 + 2 * e + 1 < c_hi ? 0xffff0000u : 0u);
              ah[f][e] &= keep;
              al[f][e] &= keep;
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
    }
    // acc[f][j][r] = partial row m0 + 16f + 4(lane>>4) + r, column dl + j
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

// (workgroups of 4 waves over the 128-column tiles of d_model) x d_ff chunks
// x the row-pass split
inline dim3 skinny_nn_grid(int D, int G) {
  const int dtiles = D / kDownCols;
  return dim3((unsigned)((dtiles + kDownWaves - 1) / kDownWaves), (unsigned)G, (unsigned)kPassSplit);
}

}  // namespace skinny
}  // namespace twell
