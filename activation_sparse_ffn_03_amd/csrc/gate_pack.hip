// Stage 1: gate projection with the TwELL pack formed in the GEMM epilogue.
//
// Follows "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second
// paragraph: d_ff is cut into horizontal tiles of width T_n matched to the
// matmul tile, nonzeros are packed locally inside each tile, and the format is
// produced directly in the epilogue of the gate-projection kernel (no separate
// conversion pass, no extra round trip through global memory).
//
// Kernels
//   gate_mfma_dma    TwELL pack path: 256x384 output tile per 8-wave
//                    workgroup when the grid is one wave of tiles, 256x256
//                    on deeper grids (128x384 per 4-wave workgroup for FP8
//                    grids of several waves), v_mfma_f32_16x16x32_bf16,
//                    K-steps of 32 loaded straight into a 2- to 4-stage LDS
//                    ring by global_load_lds; XCD-aware tile order; the epilogue
//                    stages the fp32 tile in LDS one 128-column group at a
//                    time and packs it. With FP8 = true the operands are E4M3
//                    codes (64 k per 64-byte LDS row, one
//                    v_mfma_f32_32x32x64_f8f6f4 per 32x32 fragment pair and
//                    stage) and the epilogue applies the row and column scales.
//   gate_mfma_bf16   register-staged variant (128x128, K-steps of 64), used to
//                    recompute the overflow rows with identical arithmetic
//                    where gate_rows_skinny (dense_rows.hip) does not apply.
//   gate_simt_f32    64x128 fp32 tile, plain FMA (fp32 storage only).
//   gate_gemv_small  small batches (N <= 64, bf16): g as a GEMV over all CUs
//                    into a caller's buffer, then packed by pack_from_g.
//   pack_from_g      64x128 tile of a given pre-activation (test entry and the
//                    small-batch path); with slots >= tile_n it also writes the
//                    all-zero overflow outputs, and the overflow steps are
//                    skipped.
//   ovf_flags        overflow flag of every row from its true tile counts
//                    (the ascending list is built by launch_compact).
// The same kernels, with MODE_DENSE, recompute the dense activation rows of
// the overflow rows with identical arithmetic (gathered A rows); for bf16
// operands with d_model a multiple of 32 that is gate_rows_skinny
// (dense_rows.hip) instead, a wave per 16 columns over all of d_model with the
// same chain of MFMAs per output.
#include "../../include/twell.h"
#include "twell_device.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int kPackCols = 128;  // columns one pack_epilogue call covers (two 64-lane ballots)
constexpr int BN = kPackCols;   // N tile of the fp32 / pack_from_g kernels
constexpr int GS = kPackCols + 4;  // LDS row stride of the fp32 epilogue tile (floats)

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
  const float* x_scale;  // FP8 operands: per-token scale of x (else null)
  const float* w_scale;  // FP8 operands: per-unit scale of w_gate_t (else null)
  // No row can overflow (slots >= tile_n): workgroup 0 of the pack writes the
  // all-zero overflow outputs itself, in place of the flag and compaction
  // kernels (else null).
  uint8_t* clear_flag;
  int32_t* clear_n_ovf;
  uint32_t* clear_status;
};

__device__ __forceinline__ uint64_t mask_below(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1ull); }


__device__ __forceinline__ int dense_valid(const Epi& e) { return min(*e.n_ovf, e.cap); }

// Stage the threshold and the token of logical rows [m0, m0 + nrows) of a tile
// in LDS (token -1 past the last valid row), so the epilogue reads them
// without a dependent global load per row. Logical rows are tokens
// (MODE_PACK) or positions in the overflow list (MODE_DENSE).
template <int NT>
__device__ void stage_rows(int64_t m0, int nrows, const Epi& e, float* ts, int32_t* toks, float* xs = nullptr) {
  const int64_t limit = (e.mode == MODE_DENSE) ? (int64_t)dense_valid(e) : e.N;
  for (int r = threadIdx.x; r < nrows; r += NT) {
    const int64_t lr = m0 + r;
    int32_t tok = -1;
    float tv = 0.f, sx = 0.f;
    if (lr < limit) {
      tok = (e.mode == MODE_DENSE) ? e.rows[lr] : (int32_t)lr;
      tv = e.t[tok];
      if (xs != nullptr) sx = e.x_scale[tok];
    }
    ts[r] = tv;
    toks[r] = tok;
    if (xs != nullptr) xs[r] = sx;
  }
}

// Dense activation rows of overflow rows (MODE_DENSE): one wave per row of the
// fp32 tile Gs, lane l writing columns n0+l and n0+64+l of ovf_h row row0+r.
template <typename TS, int NW>
__device__ void dense_rows_out(const float* Gs, int rows, int64_t row0, int n0, const Epi& e, const float* ts,
                               const int32_t* toks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = NW;
  for (int r = wave; r < rows; r += nw) {
    if (toks[r] < 0) break;  // rows past the last valid one
    const float tv = ts[r];
    TS* oh = reinterpret_cast<TS*>(e.ovf_h) + (size_t)(row0 + r) * e.F;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = n0 + h * 64 + lane;
      const float g = Gs[r * GS + h * 64 + lane];
      if (c < e.F) oh[c] = g > tv ? Store<TS>::from_f32(g - tv) : TS(0);
    }
  }
}

// Debug copy of g (g_dump): one wave per row, coalesced.
template <int NW>
__device__ void dump_rows(const float* Gs, int rows, int n0, const Epi& e, const int32_t* toks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = NW;
  for (int r = wave; r < rows; r += nw) {
    const int32_t tok = toks[r];
    if (tok < 0) break;
    float* gd = e.g_dump + (size_t)tok * e.F;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = n0 + h * 64 + lane;
      if (c < e.F) gd[c] = Gs[r * GS + h * 64 + lane];
    }
  }
}

// Stores the active columns of one TwELL tile of one lane's row: `bits` are
// the lane's active columns (bit b = column colofs + b of the 128-column group
// in Gs, i.e. tile column tcol + b), its slots start at `base`, and iteration
// k of a wave-uniform loop stores every lane's k-th remaining column into slot
// base + k (slots >= S are not stored: such a row is an overflow row).
template <typename TS>
__device__ __forceinline__ void store_slots(uint64_t bits, int base, int colofs, int tcol, int jt, size_t tok,
                                            bool valid, const float* grow, float tv, const Epi& e) {
  const int S = e.slots;
  const int64_t N = e.N;
  TS* vals = reinterpret_cast<TS*>(e.vals);
  for (int k = 0;; ++k) {
    const bool more = valid && bits != 0ull && base + k < S;
    if (!ballot(more)) break;
    if (more) {
      const int b = __ffsll((unsigned long long)bits) - 1;
      bits &= bits - 1;
      const size_t pos = ((size_t)jt * S + base + k) * N + tok;
      vals[pos] = Store<TS>::from_f32(grow[colofs + b] - tv);
      e.cols[pos] = (uint16_t)(tcol + b);
    }
  }
}

// TwELL pack of `rows` rows of the fp32 tile Gs (row stride GS) whose first
// column is n0; ts / toks hold the threshold and token of each row (staged by
// stage_rows). Two lanes per row, so every wave of the block takes part: lane
// l of a wave takes row (l & 31) of the wave's 32 rows and the 64 columns of
// half l >> 5, reads them four at a time and builds their 64-bit active mask
// (g > t, columns < F). A 128-column TwELL tile spans both halves: the upper
// half's slots start after the lower half's entries (one exchange of the two
// popcounts across the halves of the wave); narrower tiles lie inside one
// half. Slot s of a tile holds its s-th active column in ascending order.
// Lanes of a half are consecutive tokens, so the slot-major stores of one
// iteration are contiguous runs.
template <typename TS, int NW>
__device__ void pack_rows(const float* Gs, int rows, int n0, const Epi& e, const float* ts, const int32_t* toks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = NW;
  const int h = lane >> 5;
  const int tn = e.tile_n;
  const int64_t N = e.N;
  const int ncol = min(kPackCols, e.F - n0);
  if (ncol <= 0) return;  // a 128-column group past the last column of d_ff
  const int hcols = ncol - 64 * h;  // valid columns of this lane's half (may be <= 0)
  for (int rb = wave * 32; rb < rows; rb += nw * 32) {
    const int r = rb + (lane & 31);
    const int32_t tk = r < rows ? toks[r] : -1;
    const bool valid = tk >= 0;
    if (!ballot(valid)) break;  // rows past the last valid one
    const float tv = valid ? ts[r] : 0.f;
    const float* grow = Gs + (valid ? r : 0) * GS;
    uint64_t m = 0ull;
    if (valid && hcols > 0) {
      const float* g = grow + 64 * h;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(g + 4 * q);
        const uint64_t b = (uint64_t)(v.x > tv) | ((uint64_t)(v.y > tv) << 1) | ((uint64_t)(v.z > tv) << 2) |
                           ((uint64_t)(v.w > tv) << 3);
        m |= b << (4 * q);
      }
      m &= mask_below(hcols);
    }
    const size_t tok = (size_t)(valid ? tk : 0);
    if (tn == kPackCols) {
      const int jt = n0 / kPackCols;
      const int pc = __popcll(m);
      const int other = __shfl_xor(pc, 32, 64);  // the other half's entries
      if (valid && h == 0) e.counts[(size_t)jt * N + tok] = (uint16_t)(pc + other);
      store_slots<TS>(m, h ? other : 0, 64 * h, 64 * h, jt, tok, valid, grow, tv, e);
    } else {
      for (int t0 = 0; t0 < 64; t0 += tn) {
        const int col0 = 64 * h + t0;  // first column of the tile in the group
        const bool exists = n0 + col0 < e.F;
        const int jt = (n0 + col0) / tn;
        const uint64_t sb = (m >> t0) & mask_below(tn);
        if (valid && exists) e.counts[(size_t)jt * N + tok] = (uint16_t)__popcll(sb);
        store_slots<TS>(sb, 0, col0, 0, jt, tok, valid && exists, grow, tv, e);
      }
    }
  }
}

// Epilogue of one (rows x 128-column) block of g held in LDS.
// NW: waves of the calling workgroup (a compile-time constant: reading the
// block size at run time costs a load whose wait also waits for every
// outstanding store of the wave).
template <typename TS, int NW>
__device__ void pack_epilogue(const float* Gs, int rows, int64_t row0, int n0, const Epi& e, const float* ts,
                              const int32_t* toks) {
  if (e.mode == MODE_DENSE) {
    dense_rows_out<TS, NW>(Gs, rows, row0, n0, e, ts, toks);
    return;
  }
  if (e.g_dump) dump_rows<NW>(Gs, rows, n0, e, toks);
  pack_rows<TS, NW>(Gs, rows, n0, e, ts, toks);
}

// ---------------------------------------------------------------- bf16 MFMA GEMM

// Block tile BM x BN of g = x . w^T, WGM x WGN waves, each owning a
// (BM/WGM) x (BN/WGN) sub-tile of 16x16 v_mfma_f32_16x16x32_bf16 fragments.
// K advances by BK through two LDS stages; the next stage is fetched global ->
// registers while the current one feeds the matrix cores.
template <int BM_, int BN_, int WGM_, int WGN_, int BK_ = 64, int OCC_ = 1>
struct MfmaCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int BK = BK_;    // K per LDS stage (32 or 64)
  static constexpr int OCC = OCC_;  // occupancy hint: waves per SIMD the register budget aims at
  static constexpr int KC = BK / 8;  // 16-byte chunks per row per stage
  static constexpr int AS = BK + 8;  // LDS row stride in bf16 (16 consecutive rows hit distinct bank groups)
  static constexpr int NT = WGM * WGN * 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_CH = BM * KC / NT;  // 16-byte chunks per thread per stage
  static constexpr int B_CH = BN * KC / NT;
  static constexpr int LDS = (2 * BM * AS + 2 * BN * AS) * 2;
  static constexpr int EPI_FIT = LDS / (GS * 4);
  static constexpr int EPI_ROWS = EPI_FIT >= 256 && BM >= 256 ? 256 : EPI_FIT >= 128 && BM >= 128 ? 128 : 64;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be whole fragments");
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(BM * KC % NT == 0 && BN * KC % NT == 0, "stage must split evenly over threads");
  static_assert(BN % 128 == 0, "N tile must be whole 128-column pack groups");
  static_assert(BM % EPI_ROWS == 0 && EPI_ROWS * GS * 4 <= LDS, "epilogue staging must fit");
  static_assert(LDS + BM * 8 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// Workgroup -> output tile. Workgroups are dealt to the 8 XCDs round-robin;
// the ids are renumbered so that each XCD gets one contiguous run of tiles,
// and the run is walked in groups of `kGroupM` row blocks (column-major inside
// a group), so the tiles an XCD has in flight share A and B rows in its L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;
__device__ __forceinline__ void tile_of_block(int b, int nblocks, int mbc, int ncb, int& mb, int& nb) {
  const int q = nblocks / kXcds, r = nblocks % kXcds, x = b % kXcds;
  const int L = x * q + min(x, r) + b / kXcds;
  const int per_group = kGroupM * ncb;
  const int first_m = (L / per_group) * kGroupM;
  const int gsz = min(mbc - first_m, kGroupM);
  const int in = L % per_group;
  mb = first_m + in % gsz;
  nb = in / gsz;
}

// In MODE_DENSE, A rows are gathered through the overflow list. Both operands
// are K-contiguous.
template <class C, int MODE>
__global__ __launch_bounds__(C::NT, C::OCC) void gate_mfma_bf16(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, int D, int mbc,
                                                          int ncb, Epi e) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ float ts[C::BM];
  __shared__ int32_t toks[C::BM];
  constexpr int AS = C::AS, KC = C::KC, BK = C::BK;
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * C::BM * AS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  int mb_id, nb_id;
  tile_of_block(blockIdx.x, gridDim.x, mbc, ncb, mb_id, nb_id);
  const int64_t m0 = (int64_t)mb_id * C::BM;
  const int n0 = nb_id * C::BN;

  int64_t mlimit;
  if (MODE == MODE_DENSE) {
    mlimit = dense_valid(e);
    if (m0 >= mlimit) return;
  } else {
    mlimit = e.N;
  }
  stage_rows<C::NT>(m0, C::BM, e, ts, toks);  // visible after the first barrier below

  // Rows past the last token (or overflow row) and columns past d_ff load row
  // 0 instead: their g is never stored (the epilogue skips those rows and
  // masks those columns), so the loads need no bounds branches.
  const uint16_t* a_src[C::A_CH];
#pragma unroll
  for (int r = 0; r < C::A_CH; ++r) {
    const int q = tid + C::NT * r;
    const int row = q / KC, kc = q % KC;
    const int64_t lr = m0 + row;
    int64_t tok = lr < mlimit ? lr : 0;
    if (MODE == MODE_DENSE) tok = lr < mlimit ? (int64_t)e.rows[lr] : 0;
    a_src[r] = x + tok * (int64_t)D + kc * 8;
  }
  const uint16_t* b_src[C::B_CH];
#pragma unroll
  for (int r = 0; r < C::B_CH; ++r) {
    const int q = tid + C::NT * r;
    const int row = q / KC, kc = q % KC;
    b_src[r] = w + (int64_t)((n0 + row) < e.F ? n0 + row : 0) * D + kc * 8;
  }

  struct Regs {
    u32x4_t a[C::A_CH], b[C::B_CH];
  };
  auto gload = [&](Regs& R, int k0) {
#pragma unroll
    for (int r = 0; r < C::A_CH; ++r) R.a[r] = *reinterpret_cast<const u32x4_t*>(a_src[r] + k0);
#pragma unroll
    for (int r = 0; r < C::B_CH; ++r) R.b[r] = *reinterpret_cast<const u32x4_t*>(b_src[r] + k0);
  };
  auto lstore = [&](const Regs& R, int buf) {
    uint16_t* A = As + buf * C::BM * AS;
    uint16_t* B = Bs + buf * C::BN * AS;
#pragma unroll
    for (int r = 0; r < C::A_CH; ++r) {
      const int q = tid + C::NT * r;
      *reinterpret_cast<u32x4_t*>(A + (q / KC) * AS + (q % KC) * 8) = R.a[r];
    }
#pragma unroll
    for (int r = 0; r < C::B_CH; ++r) {
      const int q = tid + C::NT * r;
      *reinterpret_cast<u32x4_t*>(B + (q / KC) * AS + (q % KC) * 8) = R.b[r];
    }
  };

  f32x4_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const uint16_t* A = As + buf * C::BM * AS;
    const uint16_t* B = Bs + buf * C::BN * AS;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int kc = ks * 4 + (lane >> 4);
      bf16x8_t af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        af[i] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(A + (wm * C::WM + i * 16 + (lane & 15)) * AS + kc * 8));
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        bfr[j] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(B + (wn * C::WN + j * 16 + (lane & 15)) * AS + kc * 8));
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  const int KT = D / BK;
  Regs R0;
  gload(R0, 0);
  lstore(R0, 0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(R0, (kt + 1) * BK);
    compute(kt & 1);
    if (kt + 1 < KT) lstore(R0, (kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: the fp32 tile goes through LDS one (EPI_ROWS x 128-column) block
  // at a time; each block is packed by pack_epilogue.
  float* Gs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int cg = 0; cg < C::BN / kPackCols; ++cg) {
#pragma unroll
    for (int p0 = 0; p0 < C::BM; p0 += C::EPI_ROWS) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          // 16x16 MFMA result: lane l holds rows 4*(l>>4)+r of column l&15
          const int rbase = wm * C::WM + i * 16 - p0;
          const int cbase = wn * C::WN + j * 16 - cg * kPackCols;
          if (rbase < 0 || rbase >= C::EPI_ROWS || cbase < 0 || cbase >= kPackCols) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Gs[(rbase + 4 * (lane >> 4) + r) * GS + cbase + (lane & 15)] = acc[i][j][r];
        }
      // LDS-only barriers: the epilogue's global stores need no ordering
      // between waves, and a full __syncthreads would wait for them to finish
      lds_barrier();
      pack_epilogue<uint16_t, C::NT / 64>(Gs, C::EPI_ROWS, m0 + p0, n0 + cg * kPackCols, e, ts + p0, toks + p0);
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA GEMM, LDS DMA pipeline

// Variant of gate_mfma_bf16 whose K-steps (32 wide) go straight from global
// memory into a ring of ST LDS stages with global_load_lds_dwordx4, so up to
// ST-1 steps are in flight without holding staging registers. Each DMA
// instruction writes 1 KB = 16 LDS rows of 64 bytes (lane l -> row l/4,
// 16-byte position l%4). The 16-byte chunk kc of LDS row r sits at position
// kc ^ dma_swz(r), which keeps the MFMA operand reads free of bank conflicts;
// each lane therefore fetches the global chunk that belongs at its position.
// The DMA and its waits are inline assembly: the compiler does not see these
// LDS writes, so the ring is synchronised by hand (vmcnt per wave, then a
// workgroup barrier) before a stage is read.
template <int BM_, int BN_, int WGM_, int WGN_, int ST_ = 4, int OCC_ = 2>
struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, ST = ST_, OCC = OCC_;
  static constexpr int NT = WGM * WGN * 64, NW = NT / 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int ROWB = 64;                    // LDS bytes per row per stage (32 bf16)
  static constexpr int STAGE = (BM + BN) * ROWB;     // bytes per stage: A rows then B rows
  static constexpr int RING = ST * STAGE;
  static constexpr int GROUPS = (BM + BN) / 16;      // 1 KB DMA groups per stage
  static constexpr int GPW = GROUPS / NW;            // DMA instructions per wave per stage
  // The epilogue stages min(BM, 256) rows of fp32 g at a time in the same LDS
  // (32 rows per wave, so every wave of an 8-wave 256-row tile packs in one
  // pass per 128-column group; that staging, 132 KB, is larger than the
  // operand ring, so the ring can take a third stage at no LDS cost).
  static constexpr int EPI_ROWS = BM >= 256 ? 256 : (BM >= 128 ? 128 : 64);
  static constexpr int LDS = RING > EPI_ROWS * GS * 4 ? RING : EPI_ROWS * GS * 4;
  static_assert(WM % 16 == 0 && WN % 16 == 0 && BM % 16 == 0 && BN % 16 == 0, "whole fragments");
  static_assert(GROUPS % NW == 0, "DMA groups must split evenly over waves");
  static_assert(BN % 128 == 0, "N tile must be whole 128-column pack groups");
  static_assert(ST >= 2 && ST <= 4, "ring depth");
  static_assert(BM % EPI_ROWS == 0, "epilogue passes must tile BM");
  static_assert(LDS + BM * 8 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// Row -> 2-bit XOR key of the 16-byte positions of a 64-byte LDS row. A
// fragment read (lane l: row l & 15 of a 16-row group, chunk l >> 4) with
// this key runs without LDS bank conflicts on gfx950 (measured: as fast as a
// linear 1 KB read, and the bank-conflict counter stays at zero; the key was
// chosen by timing all 256 linear 2-bit keys of the row index).
__device__ __forceinline__ int dma_swz(int r) { return ((r >> 3) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }


// FP8: x and w hold E4M3 codes (one byte per element). A 64-byte stage row is
// then 64 k, exactly the depth of gfx950's v_mfma_f32_32x32x64_f8f6f4, so each
// 32x32 fragment pair takes one MFMA per stage: lane l supplies row l & 31 of
// the fragment, half l >> 5 of the stage row (32 bytes, two 16-byte chunks),
// the same way for both operands; its 16 results are rows
// 8*(q>>2) + 4*(l>>5) + (q&3), column l & 31 (measured with an in-bounds
// probe, which also showed that the instruction sums each run of 8 bytes of a
// lane in fixed point, as the 16x16x32 FP8 instruction does). The epilogue
// scales g by the row's and the column's scales. Otherwise x and w are bf16.
template <class C, int MODE, bool FP8 = false>
__global__ __launch_bounds__(C::NT, C::OCC) void gate_mfma_dma(const void* __restrict__ xv,
                                                               const void* __restrict__ wv, int D, int mbc,
                                                               int ncb, Epi e) {
  constexpr int ESZ = FP8 ? 1 : 2;  // bytes per element
  const char* __restrict__ x = reinterpret_cast<const char*>(xv);
  const char* __restrict__ w = reinterpret_cast<const char*>(wv);
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  __shared__ float ts[C::BM];
  __shared__ int32_t toks[C::BM];
  __shared__ float xs[FP8 ? C::BM : 1];  // FP8: per-row scale of x
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  int mb_id, nb_id;
  tile_of_block(blockIdx.x, gridDim.x, mbc, ncb, mb_id, nb_id);
  const int64_t m0 = (int64_t)mb_id * C::BM;
  const int n0 = nb_id * C::BN;
  int64_t mlimit;
  if (MODE == MODE_DENSE) {
    mlimit = dense_valid(e);
    if (m0 >= mlimit) return;
  } else {
    mlimit = e.N;
  }
  stage_rows<C::NT>(m0, C::BM, e, ts, toks, FP8 ? xs : nullptr);

  // Sources of this wave's DMA groups (rows past the last token / column past
  // d_ff read row 0: never stored).
  const char* src[C::GPW];
  uint32_t grp_off[C::GPW];
  const int rin = lane >> 2, p = lane & 3;
  const int64_t rowb = (int64_t)D * ESZ;  // bytes per operand row
#pragma unroll
  for (int t = 0; t < C::GPW; ++t) {
    const int g = wave + C::NW * t;
    const char* base;
    int lrow;
    if (g < C::BM / 16) {
      lrow = g * 16 + rin;
      const int64_t lr = m0 + lrow;
      int64_t tok = lr < mlimit ? lr : 0;
      if (MODE == MODE_DENSE) tok = lr < mlimit ? (int64_t)e.rows[lr] : 0;
      base = x + tok * rowb;
    } else {
      const int r = (g - C::BM / 16) * 16 + rin;
      lrow = C::BM + r;
      base = w + (int64_t)((n0 + r) < e.F ? n0 + r : 0) * rowb;
    }
    src[t] = base + ((p ^ dma_swz(lrow & 15)) << 4);
    grp_off[t] = (uint32_t)((lrow - rin) * C::ROWB);
  }
  const uint32_t lds0 =
      (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(smem));
  auto issue = [&](int kt) {
    const uint32_t sb = lds0 + (uint32_t)((kt % C::ST) * C::STAGE);
#pragma unroll
    for (int t = 0; t < C::GPW; ++t) dma_16B(src[t] + (size_t)kt * 64, sb + grp_off[t]);
  };

  // bf16: 16x16 fragments; FP8: 32x32 fragments (the other array is unused)
  constexpr int FM = FP8 ? 1 : C::FM, FN = FP8 ? 1 : C::FN;
  constexpr int FM8 = FP8 ? C::WM / 32 : 1, FN8 = FP8 ? C::WN / 32 : 1;
  static_assert(!FP8 || (C::WM % 32 == 0 && C::WN % 32 == 0), "FP8 wave tiles are whole 32x32 fragments");
  f32x4_t acc[FM][FN];
  f32x16_t acc8[FM8][FN8];
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < FM8; ++i)
#pragma unroll
      for (int j = 0; j < FN8; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc8[i][j][q] = 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int KT = (int)(rowb / 64);  // 64-byte stages
#pragma unroll
  for (int st = 0; st < C::ST - 1; ++st)
    if (st < KT) issue(st);
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt is complete for this wave once at most the later stages issued
    // so far are pending; the barrier extends that to every wave
    const int later = min(C::ST - 2, KT - 1 - kt);
    if (later >= 2) wait_vmcnt<2 * C::GPW>();
    else if (later == 1) wait_vmcnt<C::GPW>();
    else wait_vmcnt<0>();
    lds_barrier();  // also: every wave is done reading the buffer refilled below
    if (kt + C::ST - 1 < KT) issue(kt + C::ST - 1);
    const char* A = smem + (kt % C::ST) * C::STAGE;
    const char* B = A + C::BM * C::ROWB;
    if constexpr (FP8) {
      // 32 bytes per lane: chunks 2h and 2h + 1 of the fragment row
      const int h = lane >> 5;
      auto frag = [&](const char* base, int R) {
        const char* row = base + R * C::ROWB;
        const int sw = dma_swz(R & 15);
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(row + (((2 * h) ^ sw) << 4));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(row + (((2 * h + 1) ^ sw) << 4));
        return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      i32x8_t af[FM8], bfr[FN8];
#pragma unroll
      for (int i = 0; i < FM8; ++i) af[i] = frag(A, wm * C::WM + i * 32 + (lane & 31));
#pragma unroll
      for (int j = 0; j < FN8; ++j) bfr[j] = frag(B, wn * C::WN + j * 32 + (lane & 31));
#pragma unroll
      for (int i = 0; i < FM8; ++i)
#pragma unroll
        for (int j = 0; j < FN8; ++j)
          // E4M3 for both operands (format 0), no block scales: the plain
          // v_mfma_f32_32x32x64_f8f6f4
          acc8[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc8[i][j], 0, 0, 0, 0, 0, 0);
    } else {
      const int kc = lane >> 4;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int R = wm * C::WM + i * 16 + (lane & 15);
        af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(A + R * C::ROWB + ((kc ^ dma_swz(R & 15)) << 4)));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int R = wn * C::WN + j * 16 + (lane & 15);
        bfr[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(B + R * C::ROWB + ((kc ^ dma_swz(R & 15)) << 4)));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  wait_vmcnt<0>();
  lds_barrier();  // the ring is reused for the epilogue below

  float* Gs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int cg = 0; cg < C::BN / kPackCols; ++cg) {
#pragma unroll
    for (int p0 = 0; p0 < C::BM; p0 += C::EPI_ROWS) {
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < FM8; ++i)
#pragma unroll
          for (int j = 0; j < FN8; ++j) {
            const int rbase = wm * C::WM + i * 32 - p0;
            const int cbase = wn * C::WN + j * 32 - cg * kPackCols;
            if (rbase < 0 || rbase >= C::EPI_ROWS || cbase < 0 || cbase >= kPackCols) continue;
            const int col = n0 + cg * kPackCols + cbase + (lane & 31);
            const float sw = col < e.F ? e.w_scale[col] : 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int row = rbase + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
              Gs[row * GS + cbase + (lane & 31)] = acc8[i][j][q] * xs[p0 + row] * sw;
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int rbase = wm * C::WM + i * 16 - p0;
            const int cbase = wn * C::WN + j * 16 - cg * kPackCols;
            if (rbase < 0 || rbase >= C::EPI_ROWS || cbase < 0 || cbase >= kPackCols) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              Gs[(rbase + 4 * (lane >> 4) + r) * GS + cbase + (lane & 15)] = acc[i][j][r];
          }
      }
      // LDS-only barriers: the epilogue's global stores need no ordering
      // between waves, and a full __syncthreads would wait for them to finish
      lds_barrier();
      pack_epilogue<uint16_t, C::NT / 64>(Gs, C::EPI_ROWS, m0 + p0, n0 + cg * kPackCols, e, ts + p0, toks + p0);
      lds_barrier();
    }
  }
}

// Tile configurations of the bf16 gate GEMM. All accumulate each output
// element over K in the same order (32-wide MFMA steps, ascending K), so they
// produce bit-identical g. The TwELL pack uses the LDS-DMA kernel, eight
// waves (two per SIMD), one workgroup per CU, the pack epilogue in 256-row
// passes with every wave busy. When every tile fits in one wave of
// workgroups the tile is 256x384 (waves of 128x96) with a two-stage ring
// (GatePackOne; measured on the 4096 x 5632 x 2048 gate: 92 us with two
// stages, 95 with three, 101 for the earlier 128x384 tile of four waves at two
// workgroups per CU). On deeper grids it is 256x256 (waves of 128x64) with a
// four-stage ring (GatePack): the smaller accumulator set leaves registers
// for more fragments, and the grid's last wave of tiles is finer (measured,
// us: 16384 x 11008 x 4096 gate 1278-1300 against 1305-1325 for 256x384 with
// three stages, 1311-1351 with three stages and 1376-1382 with two;
// 8192 x 14336 x 4096 823-827 against 813-826; 8192 x 8192 x 2048 256-257
// against 266-281). The overflow rows use the register-staged kernel (a few
// rows, gathered) where gate_rows_skinny (dense_rows.hip) does not apply:
// 64x128 tiles for d_model <= 2048 (half the padding rows of a 128-row tile),
// 128x128 above (with a long K the better operand reuse of the larger wave
// tiles wins; measured 46 -> 35 us at d_model 2048 and 80 -> 109 us at 4096
// for 64-row tiles).
using GatePack = DmaCfg<256, 256, 2, 4, 4, 1>;
using GatePackOne = DmaCfg<256, 384, 2, 4, 2, 1>;
// FP8 operands on grids of several waves keep the 128x384 tile of four waves
// at two workgroups per CU (measured on the 16384 x 11008 x 4096 gate: 0.70 ms
// against 0.71 ms for the 256x384 tile with three stages; on the 4096 x 5632 x
// 2048 gate, one wave of tiles, the two-stage 256x384 tile takes 55 us against
// 57 us with three stages and 59 us for the 128x384 tile).
using GatePackFp8 = DmaCfg<128, 384, 1, 4, 2, 2>;
static_assert(GatePackFp8::BN == GatePackOne::BN, "the FP8 configurations share the column grid");
constexpr int kCus = 256;  // compute units of an MI355X: workgroups of one wave of tiles
using GateRowsS = MfmaCfg<64, 128, 1, 4>;
using GateRowsL = MfmaCfg<128, 128, 2, 2>;


// ---------------------------------------------------------------- fp32 SIMT GEMM

template <int MODE>
__global__ __launch_bounds__(256) void gate_simt_f32(const float* __restrict__ x, const float* __restrict__ w,
                                                     int D, int n_col_blocks, Epi e) {
  __shared__ float Ak[SBK][SBM + 4];
  __shared__ float Bk[SBK][BN + 4];
  __shared__ float Gs[SBM * GS];
  __shared__ float ts[SBM];
  __shared__ int32_t toks[SBM];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int nb_id = blockIdx.x % n_col_blocks;
  const int64_t m0 = (int64_t)(blockIdx.x / n_col_blocks) * SBM;
  const int n0 = nb_id * BN;
  int64_t mlimit = e.N;
  if (MODE == MODE_DENSE) {
    mlimit = dense_valid(e);
    if (m0 >= mlimit) return;
  }
  stage_rows<256>(m0, SBM, e, ts, toks);  // visible after the first barrier of the K loop
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
  pack_epilogue<float, 4>(Gs, SBM, m0, n0, e, ts, toks);
}

// ---------------------------------------------------------------- pack from a given g

template <typename TS, int MODE>
__global__ __launch_bounds__(256) void pack_from_g(const float* __restrict__ g, int n_col_blocks, Epi e) {
  __shared__ float Gs[SBM * GS];
  __shared__ float ts[SBM];
  __shared__ int32_t toks[SBM];
  const int tid = threadIdx.x;
  const int n0 = (blockIdx.x % n_col_blocks) * BN;
  const int64_t m0 = (int64_t)(blockIdx.x / n_col_blocks) * SBM;
  int64_t mlimit = e.N;
  if (MODE == MODE_DENSE) {
    mlimit = dense_valid(e);
    if (m0 >= mlimit) return;
  }
  stage_rows<256>(m0, SBM, e, ts, toks);
  if (MODE == MODE_PACK && e.clear_flag != nullptr && blockIdx.x == 0) {
    for (int64_t i = tid; i < e.N; i += 256) e.clear_flag[i] = 0;
    if (tid == 0) {
      *e.clear_n_ovf = 0;
      *e.clear_status = 0u;
    }
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
  pack_epilogue<TS, 4>(Gs, SBM, m0, n0, e, ts, toks);
}

// ---------------------------------------------------------------- small batches

// Gate pre-activation of at most kSmallN tokens, written to g [N][F] fp32 for
// pack_from_g. A workgroup owns 16 * UW hidden units and its 8 waves split the
// operand rows into 8 ranges of 64-byte steps (32 k of bf16, or 64 k of E4M3
// codes feeding two v_mfma_f32_16x16x32_fp8_fp8 split as in gate_mfma_dma).
// Each wave issues the W_gate loads of B steps (UW x 16 rows x 64 bytes each)
// before their MFMAs, so the weight streams from HBM with enough bytes in
// flight although the grid has only F / (16 UW) workgroups; x is small and
// read from L2, once per 16 * UW units (UW grows with the token count to keep
// that re-read small). A wave runs the MFMAs over its range in ascending k,
// and the 8 partial sums are added in wave order through LDS: deterministic,
// but g may differ in its last bits from the large-batch GEMM's single chain
// over d_model. FP8: g = (sum * x_scale[i]) * w_scale[c] in fp32, as in the
// GEMM's epilogue. Tokens past N read zeros; columns past F read row F - 1 and
// are never stored.
constexpr int kSmallN = TWELL_SMALL_BATCH_MAX;
constexpr int kGemvWaves = 8;

template <int NF, int UW, int B, bool FP8>
__global__ __launch_bounds__(64 * kGemvWaves) void gate_gemv_small(const char* __restrict__ x,
                                                                    const char* __restrict__ w, int64_t N,
                                                                    int64_t rowb, int F, const float* x_scale,
                                                                    const float* w_scale, float* __restrict__ g) {
  __shared__ f32x4_t red[NF][UW][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 16 * UW + (lane & 15);
  const int kb = (lane >> 4) * 16;  // byte offset of this lane's 16 bytes in a 64-byte step
  const int S = (int)(rowb / 64);
  const int s_lo = S * wave / kGemvWaves, s_hi = S * (wave + 1) / kGemvWaves;
  const char* wrow[UW];
#pragma unroll
  for (int u = 0; u < UW; ++u) {
    const int col = c0 + 16 * u;
    wrow[u] = w + (int64_t)(col < F ? col : F - 1) * rowb + kb;
  }
  const char* xrow[NF];
  bool xok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int tok = 16 * f + (lane & 15);
    xok[f] = tok < N;
    xrow[f] = x + (int64_t)(xok[f] ? tok : 0) * rowb + kb;
  }
  f32x4_t acc[NF][UW];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int u = 0; u < UW; ++u) acc[f][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero{0u, 0u, 0u, 0u};
  for (int s0 = s_lo; s0 < s_hi; s0 += B) {
    u32x4_t b[B][UW], a[B][NF];
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int u = 0; u < UW; ++u)
        b[j][u] = s0 + j < s_hi ? *reinterpret_cast<const u32x4_t*>(wrow[u] + (int64_t)(s0 + j) * 64) : zero;
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        a[j][f] = (s0 + j < s_hi && xok[f]) ? *reinterpret_cast<const u32x4_t*>(xrow[f] + (int64_t)(s0 + j) * 64)
                                             : zero;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (s0 + j >= s_hi) break;  // wave-uniform
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int u = 0; u < UW; ++u) {
          if constexpr (FP8) {
            const u32x4_t av = a[j][f], bv = b[j][u];
            const long alo = (long)(((uint64_t)av.y << 32) | av.x), ahi = (long)(((uint64_t)av.w << 32) | av.z);
            const long blo = (long)(((uint64_t)bv.y << 32) | bv.x), bhi = (long)(((uint64_t)bv.w << 32) | bv.z);
            acc[f][u] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(alo, blo, acc[f][u], 0, 0, 0);
            acc[f][u] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ahi, bhi, acc[f][u], 0, 0, 0);
          } else {
            acc[f][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[j][f]),
                                                                __builtin_bit_cast(bf16x8_t, b[j][u]), acc[f][u], 0,
                                                                0, 0);
          }
        }
    }
  }
  // partial sums added in wave order 0, 1, ..., 7
  for (int p = 0; p < kGemvWaves; ++p) {
    if (wave == p) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int u = 0; u < UW; ++u) red[f][u][lane] = p == 0 ? acc[f][u] : red[f][u][lane] + acc[f][u];
    }
    __syncthreads();
  }
  for (int q = wave; q < NF * UW; q += kGemvWaves) {
    const int f = q / UW, u = q % UW;
    const int col = c0 + 16 * u;
    const f32x4_t sum = red[f][u][lane];
    if (col < F) {
      const float sw = FP8 ? w_scale[col] : 1.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = 16 * f + 4 * (lane >> 4) + r;
        if (tok < N) g[tok * F + col] = FP8 ? sum[r] * x_scale[tok] * sw : sum[r];
      }
    }
  }
}

template <int NF, int UW, int B, bool FP8>
void launch_gemv(const GateArgs& a, float* g, hipStream_t s) {
  const dim3 grid((unsigned)((a.F + 16 * UW - 1) / (16 * UW)));
  const int64_t rowb = (int64_t)a.D * (FP8 ? 1 : 2);
  TWELL_LAUNCH("gate_gemv_small", (gate_gemv_small<NF, UW, B, FP8>), grid, 64 * kGemvWaves, 0, s,
               (const char*)a.x, (const char*)a.w, a.N, rowb, a.F, a.x_scale, a.w_scale, g);
}

template <bool FP8>
void launch_gemv_n(const GateArgs& a, float* g, hipStream_t s) {
  switch ((a.N + 15) / 16) {  // token fragments; units per wave and steps per load batch
    case 1: launch_gemv<1, 1, 8, FP8>(a, g, s); break;
    case 2: launch_gemv<2, 2, 8, FP8>(a, g, s); break;
    case 3: launch_gemv<3, 4, 4, FP8>(a, g, s); break;
    default: launch_gemv<4, 4, 4, FP8>(a, g, s); break;
  }
}

// ---------------------------------------------------------------- overflow rows

// One lane per token, 64 tokens per workgroup: each tile's counts of the 64
// tokens are one coalesced 128-byte load, eight tiles in flight at a time.
__global__ __launch_bounds__(64) void ovf_flags(const uint16_t* __restrict__ counts, int64_t N, int n_tiles,
                                                int slots, uint8_t* __restrict__ flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  int mx = 0;
#pragma unroll 8
  for (int j = 0; j < n_tiles; ++j) mx = max(mx, (int)counts[(size_t)j * N + i]);
  flag[i] = mx > slots ? 1 : 0;
}

}  // namespace

bool gate_ovf_rows_heavy(const GateArgs& a) {
  const bool small = a.g_in == nullptr && a.is_bf16 && a.N <= kSmallN && a.g_ws != nullptr;
  return a.is_bf16 && !a.fp8 && a.g_in == nullptr && !small && a.D > 2048 && !gate_rows_skinny_applies(a.D);
}

hipError_t launch_gate_pack(const GateArgs& a, hipStream_t s) {
  hipStream_t so = s;
  return launch_gate_pack_split(a, s, false, &so, true);
}

hipError_t launch_gate_pack_split(const GateArgs& a, hipStream_t s, bool fork, hipStream_t* ovf_stream,
                                  bool list_on_main) {
  *ovf_stream = s;
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
  e.x_scale = a.x_scale;
  e.w_scale = a.w_scale;
  const int ncb = (a.F + BN - 1) / BN;

  // Small batches (bf16 or FP8 operands, a workspace given): g from the split
  // GEMV (into g_dump when asked for, else the workspace), then the pack and
  // the overflow rows both read that g.
  const float* g_in = a.g_in;
  if (g_in == nullptr && a.is_bf16 && a.N <= kSmallN && a.g_ws != nullptr) {
    float* gb = a.g_dump != nullptr ? a.g_dump : a.g_ws;
    if (a.fp8)
      launch_gemv_n<true>(a, gb, s);
    else
      launch_gemv_n<false>(a, gb, s);
    g_in = gb;
    e.g_dump = nullptr;  // g is already in the caller's g_dump, or not asked for
  }
  // With slots >= tile_n no tile can overflow: the pack from g clears the
  // overflow outputs and the flag, compaction and overflow-row steps are
  // skipped (their results would be all zero).
  const bool no_ovf = g_in != nullptr && a.slots >= a.tile_n;
  if (no_ovf) {
    e.clear_flag = a.ovf_flag;
    e.clear_n_ovf = a.n_ovf;
    e.clear_status = a.status;
  }

  // 1. GEMM (or given g) + TwELL pack epilogue
  e.mode = MODE_PACK;
  if (a.fp8 && g_in == nullptr) {
    const int mbc = (int)((a.N + GatePackOne::BM - 1) / GatePackOne::BM),
              nbc = (a.F + GatePackOne::BN - 1) / GatePackOne::BN;
    if ((int64_t)mbc * nbc <= kCus) {
      TWELL_LAUNCH("gate_mfma_fp8", (gate_mfma_dma<GatePackOne, MODE_PACK, true>), dim3(mbc * nbc), GatePackOne::NT,
                   0, s, a.x, a.w, a.D, mbc, nbc, e);
    } else {
      const int mb8 = (int)((a.N + GatePackFp8::BM - 1) / GatePackFp8::BM);
      TWELL_LAUNCH("gate_mfma_fp8", (gate_mfma_dma<GatePackFp8, MODE_PACK, true>), dim3(mb8 * nbc), GatePackFp8::NT,
                   0, s, a.x, a.w, a.D, mb8, nbc, e);
    }
  } else if (g_in) {
    const int64_t mb = (a.N + SBM - 1) / SBM;
    if (a.is_bf16)
      TWELL_LAUNCH("pack_from_g", (pack_from_g<uint16_t, MODE_PACK>), dim3(mb * ncb), 256, 0, s, g_in, ncb, e);
    else
      TWELL_LAUNCH("pack_from_g", (pack_from_g<float, MODE_PACK>), dim3(mb * ncb), 256, 0, s, g_in, ncb, e);
  } else if (a.is_bf16) {
    const int mbc = (int)((a.N + GatePackOne::BM - 1) / GatePackOne::BM),
              nbc = (a.F + GatePackOne::BN - 1) / GatePackOne::BN;
    if ((int64_t)mbc * nbc <= kCus) {
      TWELL_LAUNCH("gate_mfma_bf16", (gate_mfma_dma<GatePackOne, MODE_PACK>), dim3(mbc * nbc), GatePackOne::NT, 0, s,
                   (const uint16_t*)a.x, (const uint16_t*)a.w, a.D, mbc, nbc, e);
    } else {
      const int mbd = (int)((a.N + GatePack::BM - 1) / GatePack::BM), nbd = (a.F + GatePack::BN - 1) / GatePack::BN;
      TWELL_LAUNCH("gate_mfma_bf16", (gate_mfma_dma<GatePack, MODE_PACK>), dim3(mbd * nbd), GatePack::NT, 0, s,
                   (const uint16_t*)a.x, (const uint16_t*)a.w, a.D, mbd, nbd, e);
    }
  } else {
    const int64_t mb = (a.N + SBM - 1) / SBM;
    TWELL_LAUNCH("gate_simt_f32", gate_simt_f32<MODE_PACK>, dim3(mb * ncb), 256, 0, s, (const float*)a.x, (const float*)a.w, a.D, ncb, e);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || no_ovf) return err;

  // 2. overflow rows from the true counts: the flags, the list and the dense
  // rows on `so` (the side stream when asked to fork). With list_on_main the
  // flags and the list stay on `s` (two short launches that on a side stream
  // would wait for CUs behind a blocked up projection, which holds all of a
  // CU's LDS).
  hipStream_t so = s;
  if (fork && !list_on_main) {
    if ((err = fork_side(s, &so)) != hipSuccess) return err;
    *ovf_stream = so;
  }
  TWELL_LAUNCH("ovf_flags", ovf_flags, dim3((a.N + 63) / 64), 64, 0, so, a.counts, a.N, a.n_tiles, a.slots,
               a.ovf_flag);
  err = launch_compact(a.ovf_flag, a.N, a.ovf_rows, a.ovf_cap, a.n_ovf, a.status, 1u /*TWELL_DEV_OVF_CAPACITY*/, so);
  if (err != hipSuccess || a.ovf_cap == 0) return err;
  if (fork && list_on_main) {
    if ((err = fork_side(s, &so)) != hipSuccess) return err;
    *ovf_stream = so;
  }

  // 3. dense activation rows of the overflow rows, same arithmetic as step 1
  e.mode = MODE_DENSE;
  if (a.fp8 && g_in == nullptr) {
    const int mbc = (a.ovf_cap + GatePackFp8::BM - 1) / GatePackFp8::BM,
              nbc = (a.F + GatePackFp8::BN - 1) / GatePackFp8::BN;
    TWELL_LAUNCH("gate_mfma_fp8_rows", (gate_mfma_dma<GatePackFp8, MODE_DENSE, true>), dim3(mbc * nbc),
                 GatePackFp8::NT, 0,
                 so, a.x, a.w, a.D, mbc, nbc, e);
  } else if (g_in) {
    const int64_t mb = (a.ovf_cap + SBM - 1) / SBM;
    if (a.is_bf16)
      TWELL_LAUNCH("pack_from_g_rows", (pack_from_g<uint16_t, MODE_DENSE>), dim3(mb * ncb), 256, 0, so, g_in, ncb, e);
    else
      TWELL_LAUNCH("pack_from_g_rows", (pack_from_g<float, MODE_DENSE>), dim3(mb * ncb), 256, 0, so, g_in, ncb, e);
  } else if (a.is_bf16 && gate_rows_skinny_applies(a.D)) {
    return launch_gate_rows_skinny((const uint16_t*)a.x, (const uint16_t*)a.w, a.D, a.F, a.ovf_rows, a.n_ovf,
                                   a.ovf_cap, a.t, (uint16_t*)a.ovf_h, so);
  } else if (a.is_bf16) {
    auto rows = [&](auto cfg) {
      using R = decltype(cfg);
      const int mbc = (a.ovf_cap + R::BM - 1) / R::BM, nbc = (a.F + R::BN - 1) / R::BN;
      TWELL_LAUNCH("gate_mfma_bf16_rows", (gate_mfma_bf16<R, MODE_DENSE>), dim3(mbc * nbc), R::NT, 0, so,
                   (const uint16_t*)a.x, (const uint16_t*)a.w, a.D, mbc, nbc, e);
    };
    if (a.D <= 2048)
      rows(GateRowsS{});
    else
      rows(GateRowsL{});
  } else {
    const int64_t mb = (a.ovf_cap + SBM - 1) / SBM;
    TWELL_LAUNCH("gate_simt_f32_rows", gate_simt_f32<MODE_DENSE>, dim3(mb * ncb), 256, 0, so, (const float*)a.x, (const float*)a.w, a.D, ncb, e);
  }
  return hipGetLastError();
}

}  // namespace twell
