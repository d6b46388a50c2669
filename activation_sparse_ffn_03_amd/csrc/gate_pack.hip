// Stage 1: gate projection with the TwELL pack formed in the GEMM epilogue.
//
// Follows "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second
// paragraph: d_ff is cut into horizontal tiles of width T_n matched to the
// matmul tile, nonzeros are packed locally inside each tile, and the format is
// produced directly in the epilogue of the gate-projection kernel (no separate
// conversion pass, no extra round trip through global memory).
//
// Kernels
//   gate_mfma_bf16   256x128 output tile per 256-thread workgroup, 4 waves of
//                    128x64, v_mfma_f32_16x16x32_bf16, K-loop of 64 with two
//                    LDS stages; epilogue stages the fp32 tile in LDS (two
//                    passes of 128 rows) and packs it.
//   gate_simt_f32    64x128 fp32 tile, plain FMA (fp32 storage only).
//   pack_from_g      64x128 tile of a given pre-activation (test entry).
//   ovf_flags        overflow flag of every row from its true tile counts
//                    (the ascending list is built by launch_compact).
// The same kernels, with MODE_DENSE, recompute the dense activation rows of
// the overflow rows with identical arithmetic (gathered A rows).
#include "twell_device.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int AS = BK + 8;   // LDS row stride in bf16 (144 B: 16 consecutive rows hit 16 distinct bank groups)
constexpr int GS = BN + 4;   // LDS row stride of the fp32 epilogue tile (floats)
constexpr int EPI_ROWS = 128;
constexpr int LDS_MFMA_BYTES = (2 * BM * AS + 2 * BN * AS) * 2;
static_assert(EPI_ROWS * GS * 4 <= LDS_MFMA_BYTES, "epilogue tile must fit in the GEMM buffers");

constexpr int SBM = 64;      // rows of the fp32 / pack_from_g tiles
constexpr int SBK = 16;

enum { MODE_PACK = 0, MODE_DENSE = 1 };

struct Epi {
  int mode;
  int64_t N;
  int F, tile_n, slots;
  const float* t;
  void* vals;
  uint16_t* cols;
  uint16_t* counts;
  float* g_dump;
  const int32_t* rows;   // MODE_DENSE: overflow row list
  const int32_t* n_ovf;  // MODE_DENSE: true count (device)
  int cap;               // MODE_DENSE: capacity
  void* ovf_h;           // MODE_DENSE: [cap][F]
};

__device__ __forceinline__ uint64_t mask_below(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1ull); }

// popcount of bits [a, b) of the 128-bit value (m1:m0), 0 <= a <= b <= 128
__device__ __forceinline__ int popc_range128(uint64_t m0, uint64_t m1, int a, int b) {
  int lo0 = min(a, 64), hi0 = min(b, 64);
  int lo1 = max(a, 64) - 64, hi1 = max(b, 64) - 64;
  int r = 0;
  if (hi0 > lo0) r += __popcll(m0 & mask_below(hi0) & ~mask_below(lo0));
  if (hi1 > lo1) r += __popcll(m1 & mask_below(hi1) & ~mask_below(lo1));
  return r;
}

__device__ __forceinline__ int dense_valid(const Epi& e) { return min(*e.n_ovf, e.cap); }

// Pack `rows` rows of the fp32 tile Gs (row stride GS) whose first logical row
// is row0 and first column n0. Logical rows are tokens (MODE_PACK) or
// positions in the overflow list (MODE_DENSE). One wave per row: lane l owns
// columns n0+l and n0+64+l; two ballots give the row's 128-bit active mask and
// a masked popcount gives every active column its slot inside its tile.
template <typename TS>
__device__ void pack_epilogue(const float* Gs, int rows, int64_t row0, int n0, const Epi& e) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int tn = e.tile_n;
  const int tpb = BN / tn;
  const int nvalid = (e.mode == MODE_DENSE) ? dense_valid(e) : 0;
  for (int r = wave; r < rows; r += nw) {
    const int64_t lr = row0 + r;
    int64_t tok;
    if (e.mode == MODE_PACK) {
      if (lr >= e.N) break;
      tok = lr;
    } else {
      if (lr >= nvalid) break;
      tok = e.rows[lr];
    }
    const float tv = e.t[tok];
    const float g0 = Gs[r * GS + lane], g1 = Gs[r * GS + 64 + lane];
    const int c0 = n0 + lane, c1 = n0 + 64 + lane;
    const bool a0 = (c0 < e.F) && (g0 > tv);
    const bool a1 = (c1 < e.F) && (g1 > tv);
    if (e.mode == MODE_DENSE) {
      TS* oh = reinterpret_cast<TS*>(e.ovf_h) + (size_t)lr * e.F;
      if (c0 < e.F) oh[c0] = a0 ? Store<TS>::from_f32(g0 - tv) : TS(0);
      if (c1 < e.F) oh[c1] = a1 ? Store<TS>::from_f32(g1 - tv) : TS(0);
      continue;
    }
    if (e.g_dump) {
      float* gd = e.g_dump + (size_t)tok * e.F;
      if (c0 < e.F) gd[c0] = g0;
      if (c1 < e.F) gd[c1] = g1;
    }
    const uint64_t m0 = ballot(a0), m1 = ballot(a1);
    const int ts0 = (lane / tn) * tn, ts1 = ((64 + lane) / tn) * tn;
    TS* vals = reinterpret_cast<TS*>(e.vals);
    if (a0) {
      const int p = popc_range128(m0, m1, ts0, lane);
      if (p < e.slots) {
        const size_t off = ((size_t)((n0 + ts0) / tn) * e.slots + p) * (size_t)e.N + tok;
        vals[off] = Store<TS>::from_f32(g0 - tv);
        e.cols[off] = uint16_t(lane - ts0);
      }
    }
    if (a1) {
      const int p = popc_range128(m0, m1, ts1, 64 + lane);
      if (p < e.slots) {
        const size_t off = ((size_t)((n0 + ts1) / tn) * e.slots + p) * (size_t)e.N + tok;
        vals[off] = Store<TS>::from_f32(g1 - tv);
        e.cols[off] = uint16_t(64 + lane - ts1);
      }
    }
    if (lane < tpb) {
      const int jt = n0 / tn + lane;
      if (jt * tn < e.F) e.counts[(size_t)jt * e.N + tok] = uint16_t(popc_range128(m0, m1, lane * tn, lane * tn + tn));
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA GEMM

// g tile = x[m0:m0+256, :] . w[n0:n0+128, :]^T. In MODE_DENSE, A rows are
// gathered through the overflow list. Both operands are K-contiguous; each
// thread moves 16-byte chunks global -> registers -> LDS.
template <int MODE>
__global__ __launch_bounds__(256, 1) void gate_mfma_bf16(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w, int D,
                                                        int n_col_blocks, Epi e) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_MFMA_BYTES];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * BM * AS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nb_id = blockIdx.x % n_col_blocks;
  const int mb_id = blockIdx.x / n_col_blocks;
  const int64_t m0 = (int64_t)mb_id * BM;
  const int n0 = nb_id * BN;

  int64_t mlimit;
  if (MODE == MODE_DENSE) {
    mlimit = dense_valid(e);
    if (m0 >= mlimit) return;
  } else {
    mlimit = e.N;
  }

  // Global source rows for this thread's A chunks (8) and B chunks (4).
  const uint16_t* a_src[8];
  bool a_ok[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int q = tid + 256 * r;
    const int row = q >> 3, kc = q & 7;
    const int64_t lr = m0 + row;
    a_ok[r] = lr < mlimit;
    int64_t tok = lr;
    if (MODE == MODE_DENSE) tok = a_ok[r] ? (int64_t)e.rows[lr] : 0;
    a_src[r] = x + (a_ok[r] ? tok : 0) * (int64_t)D + kc * 8;
  }
  const uint16_t* b_src[4];
  bool b_ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = tid + 256 * r;
    const int row = q >> 3, kc = q & 7;
    b_ok[r] = (n0 + row) < e.F;
    b_src[r] = w + (int64_t)(b_ok[r] ? n0 + row : 0) * D + kc * 8;
  }

  u32x4_t ra[8], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      ra[r] = a_ok[r] ? *reinterpret_cast<const u32x4_t*>(a_src[r] + k0) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r)
      rb[r] = b_ok[r] ? *reinterpret_cast<const u32x4_t*>(b_src[r] + k0) : u32x4_t{0, 0, 0, 0};
  };
  auto lstore = [&](int buf) {
    uint16_t* A = As + buf * BM * AS;
    uint16_t* B = Bs + buf * BN * AS;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int q = tid + 256 * r;
      *reinterpret_cast<u32x4_t*>(A + (q >> 3) * AS + (q & 7) * 8) = ra[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = tid + 256 * r;
      *reinterpret_cast<u32x4_t*>(B + (q >> 3) * AS + (q & 7) * 8) = rb[r];
    }
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = D / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const uint16_t* A = As + buf * BM * AS;
    const uint16_t* B = Bs + buf * BN * AS;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = ks * 4 + (lane >> 4);
      bf16x8_t af[8], bfr[4];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(A + (wm * 128 + i * 16 + (lane & 15)) * AS + kc * 8));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(B + (wn * 64 + j * 16 + (lane & 15)) * AS + kc * 8));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: two passes of 128 rows through an fp32 LDS tile.
  float* Gs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (wm == pass) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // 16x16 MFMA result: lane l holds rows 4*(l>>4)+r of column l&15
            const int row = i * 16 + 4 * (lane >> 4) + r;
            const int col = wn * 64 + j * 16 + (lane & 15);
            Gs[row * GS + col] = acc[i][j][r];
          }
    }
    __syncthreads();
    pack_epilogue<uint16_t>(Gs, EPI_ROWS, m0 + pass * EPI_ROWS, n0, e);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- fp32 SIMT GEMM

template <int MODE>
__global__ __launch_bounds__(256) void gate_simt_f32(const float* __restrict__ x, const float* __restrict__ w,
                                                     int D, int n_col_blocks, Epi e) {
  __shared__ float Ak[SBK][SBM + 4];
  __shared__ float Bk[SBK][BN + 4];
  __shared__ float Gs[SBM * GS];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int nb_id = blockIdx.x % n_col_blocks;
  const int64_t m0 = (int64_t)(blockIdx.x / n_col_blocks) * SBM;
  const int n0 = nb_id * BN;
  int64_t mlimit = e.N;
  if (MODE == MODE_DENSE) {
    mlimit = dense_valid(e);
    if (m0 >= mlimit) return;
  }
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < D; k0 += SBK) {
    // A: 64 rows x 16 k = 1024 values, 4 per thread
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = tid + 256 * r, row = q >> 4, k = q & 15;
      const int64_t lr = m0 + row;
      float v = 0.f;
      if (lr < mlimit) {
        const int64_t tok = (MODE == MODE_DENSE) ? (int64_t)e.rows[lr] : lr;
        v = x[tok * D + k0 + k];
      }
      Ak[k][row] = v;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int q = tid + 256 * r, row = q >> 4, k = q & 15;
      Bk[k][row] = (n0 + row < e.F) ? w[(int64_t)(n0 + row) * D + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SBK; ++k) {
      float av[4], bv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = Ak[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[j] = Bk[k][tx * 8 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) Gs[(ty * 4 + i) * GS + tx * 8 + j] = acc[i][j];
  __syncthreads();
  pack_epilogue<float>(Gs, SBM, m0, n0, e);
}

// ---------------------------------------------------------------- pack from a given g

template <typename TS, int MODE>
__global__ __launch_bounds__(256) void pack_from_g(const float* __restrict__ g, int n_col_blocks, Epi e) {
  __shared__ float Gs[SBM * GS];
  const int tid = threadIdx.x;
  const int n0 = (blockIdx.x % n_col_blocks) * BN;
  const int64_t m0 = (int64_t)(blockIdx.x / n_col_blocks) * SBM;
  int64_t mlimit = e.N;
  if (MODE == MODE_DENSE) {
    mlimit = dense_valid(e);
    if (m0 >= mlimit) return;
  }
  for (int q = tid; q < SBM * BN; q += 256) {
    const int row = q / BN, col = q % BN;
    const int64_t lr = m0 + row;
    float v = 0.f;
    if (lr < mlimit && n0 + col < e.F) {
      const int64_t tok = (MODE == MODE_DENSE) ? (int64_t)e.rows[lr] : lr;
      v = g[tok * e.F + n0 + col];
    }
    Gs[row * GS + col] = v;
  }
  __syncthreads();
  pack_epilogue<TS>(Gs, SBM, m0, n0, e);
}

// ---------------------------------------------------------------- overflow rows

__global__ __launch_bounds__(256) void ovf_flags(const uint16_t* __restrict__ counts, int64_t N, int n_tiles,
                                                 int slots, uint8_t* __restrict__ flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  uint8_t f = 0;
  for (int j = 0; j < n_tiles; ++j) f |= counts[(size_t)j * N + i] > slots;
  flag[i] = f;
}

}  // namespace

hipError_t launch_gate_pack(const GateArgs& a, hipStream_t s) {
  Epi e{};
  e.N = a.N;
  e.F = a.F;
  e.tile_n = a.tile_n;
  e.slots = a.slots;
  e.t = a.t;
  e.vals = a.vals;
  e.cols = a.cols;
  e.counts = a.counts;
  e.g_dump = a.g_dump;
  e.rows = a.ovf_rows;
  e.n_ovf = a.n_ovf;
  e.cap = a.ovf_cap;
  e.ovf_h = a.ovf_h;
  const int ncb = (a.F + BN - 1) / BN;

  // 1. GEMM (or given g) + TwELL pack epilogue
  e.mode = MODE_PACK;
  if (a.g_in) {
    const int64_t mb = (a.N + SBM - 1) / SBM;
    if (a.is_bf16)
      TWELL_LAUNCH("pack_from_g", (pack_from_g<uint16_t, MODE_PACK>), dim3(mb * ncb), 256, 0, s, a.g_in, ncb, e);
    else
      TWELL_LAUNCH("pack_from_g", (pack_from_g<float, MODE_PACK>), dim3(mb * ncb), 256, 0, s, a.g_in, ncb, e);
  } else if (a.is_bf16) {
    const int64_t mb = (a.N + BM - 1) / BM;
    TWELL_LAUNCH("gate_mfma_bf16", gate_mfma_bf16<MODE_PACK>, dim3(mb * ncb), 256, 0, s, (const uint16_t*)a.x, (const uint16_t*)a.w, a.D, ncb, e);
  } else {
    const int64_t mb = (a.N + SBM - 1) / SBM;
    TWELL_LAUNCH("gate_simt_f32", gate_simt_f32<MODE_PACK>, dim3(mb * ncb), 256, 0, s, (const float*)a.x, (const float*)a.w, a.D, ncb, e);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 2. overflow rows from the true counts
  TWELL_LAUNCH("ovf_flags", ovf_flags, dim3((a.N + 255) / 256), 256, 0, s, a.counts, a.N, a.n_tiles, a.slots, a.ovf_flag);
  err = launch_compact(a.ovf_flag, a.N, a.ovf_rows, a.ovf_cap, a.n_ovf, a.status, 1u /*TWELL_DEV_OVF_CAPACITY*/, s);
  if (err != hipSuccess || a.ovf_cap == 0) return err;

  // 3. dense activation rows of the overflow rows, same arithmetic as step 1
  e.mode = MODE_DENSE;
  if (a.g_in) {
    const int64_t mb = (a.ovf_cap + SBM - 1) / SBM;
    if (a.is_bf16)
      TWELL_LAUNCH("pack_from_g_rows", (pack_from_g<uint16_t, MODE_DENSE>), dim3(mb * ncb), 256, 0, s, a.g_in, ncb, e);
    else
      TWELL_LAUNCH("pack_from_g_rows", (pack_from_g<float, MODE_DENSE>), dim3(mb * ncb), 256, 0, s, a.g_in, ncb, e);
  } else if (a.is_bf16) {
    const int64_t mb = (a.ovf_cap + BM - 1) / BM;
    TWELL_LAUNCH("gate_mfma_bf16_rows", gate_mfma_bf16<MODE_DENSE>, dim3(mb * ncb), 256, 0, s, (const uint16_t*)a.x, (const uint16_t*)a.w, a.D, ncb, e);
  } else {
    const int64_t mb = (a.ovf_cap + SBM - 1) / SBM;
    TWELL_LAUNCH("gate_simt_f32_rows", gate_simt_f32<MODE_DENSE>, dim3(mb * ncb), 256, 0, s, (const float*)a.x, (const float*)a.w, a.D, ncb, e);
  }
  return hipGetLastError();
}

}  // namespace twell
