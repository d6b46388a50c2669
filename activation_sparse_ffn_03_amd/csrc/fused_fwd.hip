// Stage 2: up + down projection on the TwELL activation.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// the inference kernel reads the activations in TwELL and performs the up and
// down projections without writing the intermediate hidden state to global
// memory.
//
// On MI355X every packed entry (i, c) has to bring its own W_up and W_down row
// to the ALUs (at 1% density no block of tokens shares enough columns for
// register reuse), so what decides the speed is where those rows come from:
// the 4 MB L2 of the XCD, or the Infinity Cache / HBM behind it. The pass is
// therefore split in two launches that each keep a 1/8 slice of a weight in
// each XCD's L2 (workgroups are dealt to the 8 XCDs round-robin, so block b
// runs on XCD b % 8):
//
//   ffn_up_kernel    part p = b % 8 owns TwELL tiles [p*n_t/8, (p+1)*n_t/8).
//                    One wave per token: x_i in registers, the token's packed
//                    entries in those tiles collected into a register list,
//                    W_up rows gathered a few at a time, a = x_i . W_up^T[c]
//                    reduced with DPP, z = h * a stored in the token's
//                    (column, z) list (the sparse z, never a dense hidden
//                    state). When a 1/8 block of W_up exceeds the L2, d_model
//                    is taken in up_nq ranges, one after another in grid
//                    order, and ffn_up_finish adds their partial a.
//   ffn_down_kernel  part p = b % P owns the d_model slice of y
//                    [p*D/P, (p+1)*D/P). One wave per token: its (c, z) list,
//                    the slice of each W_down row, y slice in registers.
//
// Overflow rows (a tile count above S) are skipped by both. In bf16 layers
// (d_model a multiple of 128) all of them go through two skinny MFMA products
// (dense_rows.hip). Otherwise each dense activation row is split into column
// chunks of kDenseChunk, each chunk a work item of its own wave writing a
// partial y row (ffn_dense_rows). Either way dense_reduce adds the chunk
// partials in chunk order (deterministic, no atomics).
#include "row_ops.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int kParts = 8;  // one part per XCD

// Walk TwELL tiles [j0, j1) of token i (not an overflow row) and hand its
// packed entries to `flush` in lists of at most 64: lane k of the list holds
// entry k as (global column c, stored activation h, slot id j*S+s). The slot
// loads of all tiles are issued back to back into raw registers and decoded
// once per list, so a token's metadata costs a couple of memory round trips
// rather than one per tile. cnt_first, when not negative, is the caller's
// already loaded count of tile j0 + lane (clamped to S; 0 past j1), so the
// first batch needs no load of its own.
template <typename TS, typename Flush>
__device__ __forceinline__ void collect_pairs(const FwdArgs& a, int64_t i, int j0, int j1, int lane, Flush&& flush,
                                              int cnt_first = -1) {
  const int64_t N = a.N;
  const TS* __restrict__ vals = reinterpret_cast<const TS*>(a.vals);
  int n = 0;
  int base_l = 0, slot_l = 0;
  uint32_t col_raw = 0, val_raw = 0;
  auto emit = [&](int cnt) {
    const int c = base_l + (int)col_raw;
    float v;
    if constexpr (sizeof(TS) == 2)
      v = bf16_to_f32((uint16_t)val_raw);
    else
      v = __uint_as_float(val_raw);
    flush(c, v, slot_l, cnt);
  };
  for (int jb = j0; jb < j1; jb += 64) {
    const int jl = jb + lane;
    const int cnt_l = (jb == j0 && cnt_first >= 0) ? cnt_first
                      : jl < j1                    ? min((int)a.counts[(size_t)jl * N + i], a.slots)
                                                   : 0;
    uint64_t nz = ballot(cnt_l > 0);
    while (nz) {
      const int t = __ffsll((unsigned long long)nz) - 1;
      nz &= nz - 1;
      const int j = jb + t;
      const int cnt = readlane_i(cnt_l, t);
      for (int sb = 0; sb < cnt;) {
        if (n == 64) {
          emit(64);
          n = 0;
        }
        const int take = min(cnt - sb, 64 - n);
        if (lane >= n && lane < n + take) {
          const int slot = j * a.slots + sb + lane - n;
          const size_t pos = (size_t)slot * N + i;
          col_raw = a.cols[pos];
          if constexpr (sizeof(TS) == 2)
            val_raw = vals[pos];
          else
            val_raw = __float_as_uint(vals[pos]);
          base_l = j * a.tile_n;
          slot_l = slot;
        }
        n += take;
        sb += take;
      }
    }
  }
  if (n > 0) emit(n);
}

// ------------------------------------------------------------------ up: z = h * (x_i . W_up^T[c])

// Entries of token i in tiles [64, j0) (the first 64 tiles are summed by the
// caller from counts it loaded up front): where tile j0's entries start in the
// token's (column, z) list. Counts are small integers, so the float wave sums
// are exact.
__device__ __forceinline__ int entries_before_rest(const FwdArgs& a, int64_t i, int j0, int lane) {
  int before = 0;
  for (int jb = 64; jb < j0; jb += 64) {
    const int jl = jb + lane;
    const int c = jl < j0 ? min((int)a.counts[(size_t)jl * a.N + i], a.slots) : 0;
    before += (int)wave_sum_dpp((float)c);
  }
  return before;
}

// Workgroup b: part p = b % parts (the XCD's TwELL tiles), d_model range
// q = (b / parts) / tblocks (ranges in grid order, one W_up block per XCD in
// L2 at a time), four tokens of the block row. With one range the wave stores
// (c, z = h*a) and a_save itself; with several it stores its partial a, range
// 0 also (c, h) and the entry's slot, and ffn_up_finish adds the ranges.
template <typename TS, int M, bool SMALL>
__global__ __launch_bounds__(256) void ffn_up_kernel(FwdArgs a, int parts, int64_t tblocks, int64_t i0, int64_t i1) {
  constexpr int E = ChunkElems<TS>::E;
  // rows in flight per wave: more costs occupancy, measured slower on large
  // batches; small batches (few waves, weight rows from HBM) take more
  constexpr int U = SMALL ? (M <= 4 ? 8 : (M == 8 ? 4 : 2)) : (M <= 4 ? 2 : 1);
  const int lane = threadIdx.x & 63;
  const int part = blockIdx.x % parts;
  const int64_t r = blockIdx.x / parts;
  const int q = (int)(r / tblocks);
  const int64_t i = i0 + (r % tblocks) * 4 + (threadIdx.x >> 6);
  if (i >= i1) return;
  const int j0 = (int)((int64_t)part * a.n_tiles / parts), j1 = (int)((int64_t)(part + 1) * a.n_tiles / parts);
  const int D = a.D, Dq = D / a.up_nq, nch = Dq / E;
  const int64_t N = a.N;
  // Independent loads first, in one memory round trip: the counts of the
  // first 64 tiles and of this part's tiles, the x slice.
  const int ca = lane < a.n_tiles ? (int)a.counts[(size_t)lane * N + i] : 0;
  const int cf = j0 + lane < j1 ? (int)a.counts[(size_t)(j0 + lane) * N + i] : 0;
  u32x4_t xr[M];
  load_row<TS, M>(xr, reinterpret_cast<const TS*>(a.x) + (size_t)i * D + (size_t)q * Dq, nch, lane);
  // An overflow row (some tile count above S; the pack's flag, taken here
  // from the counts so that this kernel need not wait for the flag kernel) is
  // left to the dense-row path; its entry total is marked -1 for the down
  // projection and the finish pass.
  int cmax = ca;
  for (int jb = 64; jb < a.n_tiles; jb += 64)
    cmax = max(cmax, jb + lane < a.n_tiles ? (int)a.counts[(size_t)(jb + lane) * N + i] : 0);
  if (wave_max_int(cmax) > a.slots) {
    if (j1 == a.n_tiles && q == 0 && lane == 0) a.offs[i] = -1;
    return;
  }
  const int cb = lane < j0 ? ca : 0;
  const size_t L = (size_t)a.n_tiles * a.slots;
  const TS* __restrict__ w_up = reinterpret_cast<const TS*>(a.w_up) + (size_t)q * Dq;
  uint2* __restrict__ zl = a.zlist + (size_t)i * L;
  float* __restrict__ up = a.upart + ((size_t)q * a.N + i) * L;
  // list position of this part's first entry
  int lbase = (int)wave_sum_dpp((float)min(cb, a.slots)) + entries_before_rest(a, i, j0, lane);
  auto flush = [&](int c_l, float h_l, int slot_l, int n) {
    float a_l = 0.f;
    for (int k = 0; k < n; k += U) {
      u32x4_t wr[U][M];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = readlane_i(c_l, min(k + u, n - 1));
        ok[u] = (unsigned)c < (unsigned)a.F;  // a corrupted column contributes nothing
        load_row<TS, M>(wr[u], w_up + (size_t)(ok[u] ? c : 0) * D, nch, lane);
      }
      float dot[U];
#pragma unroll
      for (int u = 0; u < U; ++u) dot[u] = dot_rows<TS, M>(xr, wr[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) dot[u] = wave_sum_dpp(dot[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (lane == k + u) a_l = ok[u] ? dot[u] : 0.f;
    }
    // lane k holds entry k: one coalesced store per list
    if (lane < n) {
      if (a.up_nq == 1) {
        zl[lbase + lane] = make_uint2((uint32_t)c_l, __float_as_uint(h_l * a_l));
        if (a.a_save) a.a_save[(size_t)slot_l * a.N + i] = a_l;
      } else {
        up[lbase + lane] = a_l;
        if (q == 0) {
          zl[lbase + lane] = make_uint2((uint32_t)c_l, __float_as_uint(h_l));
          if (a.a_save) a.uslot[(size_t)i * L + lbase + lane] = slot_l;
        }
      }
    }
    lbase += n;
  };
  collect_pairs<TS>(a, i, j0, j1, lane, flush, min(cf, a.slots));
  if (j1 == a.n_tiles && q == 0 && lane == 0) a.offs[i] = lbase;  // the row's total
}

// a = sum of the up passes' partials in range order; z = h * a into the
// (column, h) list written by range 0, a into a_save at the entry's slot.
// Wave per token, 64 entries per step: a plain streaming pass.
__global__ __launch_bounds__(256) void ffn_up_finish(FwdArgs a, int64_t i0, int64_t i1) {
  const int lane = threadIdx.x & 63;
  const int64_t i = i0 + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= i1) return;
  const int total = a.offs[i];
  if (total < 0) return;  // an overflow row
  const size_t L = (size_t)a.n_tiles * a.slots;
  const size_t qstride = (size_t)a.N * L;
  uint2* __restrict__ zl = a.zlist + (size_t)i * L;
  const float* __restrict__ up = a.upart + (size_t)i * L;
  for (int k = lane; k < total; k += 64) {
    float sum = 0.f;
    for (int q = 0; q < a.up_nq; ++q) sum += up[q * qstride + k];
    const uint2 e = zl[k];
    zl[k] = make_uint2(e.x, __float_as_uint(__uint_as_float(e.y) * sum));
    if (a.a_save) a.a_save[(size_t)a.uslot[(size_t)i * L + k] * a.N + i] = sum;
  }
}

// ------------------------------------------------------------------ down: y_i[slice] = sum z * W_down[c][slice]

// Wave per (row i, d_model slice p); the slice is read 16 bytes per lane, so a
// load instruction covers RPI rows of W_down (see pick_l2_slices). Slices go
// G8 at a time (slice_block), so an XCD holds one slice of W_down at a time.
template <typename TS, int EPL, int RPI, bool SMALL>
__global__ __launch_bounds__(256) void ffn_down_kernel(FwdArgs a, int G8, int64_t tblocks, int64_t i0, int64_t i1) {
  constexpr int LPR = 64 / RPI;
  // load instructions in flight; small batches take more (the entry order of
  // the sums is the same either way)
  constexpr int U = SMALL ? (RPI <= 4 ? 16 : 64 / RPI) : sliced_inflight<RPI>();
  const int lane = threadIdx.x & 63;
  int p;
  int64_t rb;
  slice_block(blockIdx.x, G8, tblocks, p, rb);
  if (a.rb_order) {  // heaviest blocks first (the whole batch in one launch)
    rb = a.rb_order[rb];
    if ((uint64_t)rb >= (uint64_t)tblocks) return;
  }
  const int64_t i = i0 + rb * 4 + (threadIdx.x >> 6);
  if (i >= i1) return;
  const int D = a.D;
  const int d0 = p * (LPR * EPL) + (lane % LPR) * EPL;
  const TS* __restrict__ w_down = reinterpret_cast<const TS*>(a.w_down) + d0;
  const int L = a.n_tiles * a.slots;
  const uint2* __restrict__ zl = a.zlist + (size_t)i * L;
  // Independent loads first, in one memory round trip: the row's entry total
  // (-1 for an overflow row) and (speculatively, inside the row's list) its
  // first 64 entries.
  const int total = a.offs[i];
  const uint2 ent0 = lane < L ? zl[lane] : make_uint2(0u, 0u);
  if (total < 0) return;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int kb = 0; kb < total; kb += 64) {
    const int n = min(64, total - kb);
    const uint2 ent = lane >= n ? make_uint2(0u, 0u) : kb == 0 ? ent0 : zl[kb + lane];
    sliced_axpy<TS, EPL, RPI, U>(w_down, D, a.F, (int)ent.x, __uint_as_float(ent.y), n, lane, acc);
  }
  combine_groups<EPL, RPI>(acc);
  if (lane < LPR) {
    float* dst = a.y + (size_t)i * D + d0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = acc[e];
  }
}

// ------------------------------------------------------------------ overflow rows

// Work item (o, g): overflow row o, columns [g*kDenseChunk, ...) of its dense
// activation row; writes the partial y row part[o][g]. The active columns of
// each 64-column block are handled in two batched passes: a for U columns at a
// time (U W_up rows in flight), then y += z * W_down[c] likewise. The grid is
// capped (kRowsGrid workgroups) and each wave strides over the work items of
// the rows that really overflowed, so a step without overflow rows costs one
// small launch whatever the capacity.
template <typename TS, int M>
__device__ __forceinline__ void dense_row_item(const FwdArgs& a, int G, int o, int g) {
  constexpr int E = ChunkElems<TS>::E;
  constexpr int U = M <= 4 ? 4 : (M == 8 ? 2 : 1);
  const int lane = threadIdx.x & 63;
  const int D = a.D, nch = D / E;
  const TS* __restrict__ w_up = reinterpret_cast<const TS*>(a.w_up);
  const TS* __restrict__ w_down = reinterpret_cast<const TS*>(a.w_down);
  const int64_t i = a.ovf_rows[o];
  u32x4_t xr[M];
  float acc[M][8];
  zero_acc<M>(acc);
  load_row<TS, M>(xr, reinterpret_cast<const TS*>(a.x) + (size_t)i * D, nch, lane);
  const TS* __restrict__ hrow = reinterpret_cast<const TS*>(a.ovf_h) + (size_t)o * a.F;
  const int c0 = g * kDenseChunk, c1 = min(a.F, c0 + kDenseChunk);
  for (int cb = c0; cb < c1; cb += 64) {
    const int c = cb + lane;
    const float h_l = c < c1 ? Store<TS>::load(hrow, c) : 0.f;
    const uint64_t m = ballot(h_l > 0.f);
    const int n = __popcll(m);
    if (n == 0) continue;
    // compact the active columns: lane q of the list gets the q-th active one,
    // found by binary search on prefix popcounts of the ballot
    int lo = 0, hi = 63;
    for (int step = 0; step < 6; ++step) {
      const int mid = (lo + hi) >> 1;
      const uint64_t below = mid >= 63 ? ~0ull : ((2ull << mid) - 1ull);
      if (__popcll(m & below) >= lane + 1) hi = mid; else lo = mid + 1;
    }
    const int col_l = cb + lo;
    const float h_q = __shfl(h_l, lo, 64);
    float z_l = 0.f;
    for (int q = 0; q < n; q += U) {
      u32x4_t wr[U][M];
#pragma unroll
      for (int u = 0; u < U; ++u)
        load_row<TS, M>(wr[u], w_up + (size_t)readlane_i(col_l, min(q + u, n - 1)) * D, nch, lane);
      float dot[U];
#pragma unroll
      for (int u = 0; u < U; ++u) dot[u] = wave_sum_dpp(dot_rows<TS, M>(xr, wr[u]));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (lane == q + u) z_l = h_q * dot[u];
    }
    for (int q = 0; q < n; q += U) {
      u32x4_t wr[U][M];
#pragma unroll
      for (int u = 0; u < U; ++u)
        load_row<TS, M>(wr[u], w_down + (size_t)readlane_i(col_l, min(q + u, n - 1)) * D, nch, lane);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (q + u < n) axpy_row<TS, M>(acc, readlane_f(z_l, q + u), wr[u]);
    }
  }
  store_row<TS, M>(a.part + ((size_t)o * G + g) * D, acc, nch, lane);
}

constexpr int kRowsGrid = 1024;

template <typename TS, int M>
__global__ __launch_bounds__(256) void ffn_dense_rows(FwdArgs a, int G) {
  const int n_rows = min(a.ovf_cap, *a.n_ovf);
  const int64_t items = (int64_t)n_rows * G;
  for (int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); k < items; k += (int64_t)gridDim.x * 4)
    dense_row_item<TS, M>(a, G, (int)(k / G), (int)(k % G));
}

// y[ovf_rows[o]] = sum_g part[o][g]  (fixed chunk order); a capped grid
// strides over the rows that really overflowed
__global__ __launch_bounds__(256) void dense_reduce(const float* __restrict__ part, const int32_t* __restrict__ rows,
                                                    const int32_t* __restrict__ n_rows, int cap, int G, int D,
                                                    float* __restrict__ out) {
  const int db = (D + 255) / 256;
  const int64_t nb = (int64_t)min(cap, *n_rows) * db;
  for (int64_t b = blockIdx.x; b < nb; b += gridDim.x) {
    const int o = (int)(b / db);
    const int d = (int)(b % db) * 256 + threadIdx.x;
    if (d >= D) continue;
    const float* p = part + (size_t)o * G * D + d;
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += p[(size_t)g * D];
    out[(size_t)rows[o] * D + d] = s;
  }
}

// Budget of an XCD's slice of W_down (see pick_l2_slices). It is larger than
// the 4 MB L2: every slice pass re-reads all (column, z) lists and fewer,
// wider slices halve that, which outweighs the slice's L2 misses (served by
// the Infinity Cache) up to 256-column slices of 5.6-7.3 MB; 512-column
// slices (11-15 MB) are slower again. Measured on the 16384 x 4096 x 11008
// forward: 873 us with 128-column slices, 749 with 256, 1278 with 512; on the
// 8192 x 4096 x 14336 one: 711, 660, 937.
constexpr int64_t kDownSliceBudget = 8ll << 20;

// Token rows per pair of up / down launches (0 = all rows in one pair).
constexpr int64_t kTokenChunk = 0;
// Up to this many rows the up / down launches use their small-batch forms.
constexpr int64_t kSmallRows = 64;

template <typename TS>
hipError_t launch_sparse_rows(const FwdArgs& a, hipStream_t s, int64_t chunk) {
  constexpr int E = ChunkElems<TS>::E;
  const int nch = a.D / E;
  if (a.up_nq < 1 || a.D % (a.up_nq * E) != 0) return hipErrorInvalidValue;
  const int Mq = pick_m(nch / a.up_nq);  // chunks per lane of one d_model range
  const dim3 blk(256);
  hipError_t err;

  // up: (column, z) list of the non-overflow rows, in up_nq d_model ranges;
  // down: their y rows, d_model cut into P slices (pick_l2_slices)
  const int parts = a.n_tiles < kParts ? a.n_tiles : kParts;
  const SliceGeom geom = pick_l2_slices(a.D, (int)sizeof(TS), a.F, kDownSliceBudget);
  const int P = geom.P, G8 = slice_group(P);
  if (chunk <= 0) chunk = a.N;
  for (int64_t i0 = 0; i0 < a.N; i0 += chunk) {
    const int64_t i1 = i0 + chunk < a.N ? i0 + chunk : a.N;
    const int64_t tblocks = (i1 - i0 + 3) / 4;
    const dim3 gup((unsigned)(tblocks * parts * a.up_nq));
    const bool small = i1 - i0 <= kSmallRows;
    FwdArgs b = a;  // the down launch's arguments: natural block order unless set below
    b.rb_order = nullptr;
    if (sizeof(TS) == 2 && chunk == a.N && up_blocked_applies(a)) {
      // large batches: token blocks x tile groups through LDS (up_blocked.hip),
      // which also orders the down projection's blocks
      if ((err = launch_up_blocked(a, s)) != hipSuccess) return err;
      if (down_order_applies(a)) b.rb_order = a.rb_order;
    } else {
#define TWELL_UP(MM)                                                                                          \
  case MM:                                                                                                    \
    if (small)                                                                                                \
      TWELL_LAUNCH("ffn_up_kernel", (ffn_up_kernel<TS, MM, true>), gup, blk, 0, s, a, parts, tblocks, i0, i1); \
    else                                                                                                      \
      TWELL_LAUNCH("ffn_up_kernel", (ffn_up_kernel<TS, MM, false>), gup, blk, 0, s, a, parts, tblocks, i0, i1); \
    break;
    switch (Mq) {
      TWELL_UP(1) TWELL_UP(2) TWELL_UP(4) TWELL_UP(8) TWELL_UP(16)
      default: return hipErrorInvalidValue;
    }
#undef TWELL_UP
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.up_nq > 1) {
      TWELL_LAUNCH("ffn_up_finish", ffn_up_finish, dim3((unsigned)tblocks), blk, 0, s, a, i0, i1);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    }
    const dim3 gdn((unsigned)(tblocks * P));
#define TWELL_DOWN(E, R)                                                                                    \
  if (small)                                                                                                \
    TWELL_LAUNCH("ffn_down_kernel", (ffn_down_kernel<TS, E, R, true>), gdn, blk, 0, s, b, G8, tblocks, i0, i1); \
  else                                                                                                      \
    TWELL_LAUNCH("ffn_down_kernel", (ffn_down_kernel<TS, E, R, false>), gdn, blk, 0, s, b, G8, tblocks, i0, i1)
    if constexpr (sizeof(TS) == 2) {
      TWELL_SLICED_CASES(8, TWELL_DOWN)
    } else {
      TWELL_SLICED_CASES(4, TWELL_DOWN)
    }
#undef TWELL_DOWN
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

// Overflow rows: dense chunks + fixed-order reduction into y.
template <typename TS>
hipError_t launch_overflow_rows(const FwdArgs& a, hipStream_t s) {
  if (sizeof(TS) == 2 && dense_mfma_applies(a)) return launch_dense_mfma(a, s);
  const int M = pick_m(a.D / ChunkElems<TS>::E);
  const int G = (a.F + kDenseChunk - 1) / kDenseChunk;
  const int64_t want = ((int64_t)a.ovf_cap * G + 3) / 4;
  const dim3 gov((unsigned)(want < kRowsGrid ? want : kRowsGrid)), blk(256);
  switch (M) {
    case 1: TWELL_LAUNCH("ffn_dense_rows", (ffn_dense_rows<TS, 1>), gov, blk, 0, s, a, G); break;
    case 2: TWELL_LAUNCH("ffn_dense_rows", (ffn_dense_rows<TS, 2>), gov, blk, 0, s, a, G); break;
    case 4: TWELL_LAUNCH("ffn_dense_rows", (ffn_dense_rows<TS, 4>), gov, blk, 0, s, a, G); break;
    case 8: TWELL_LAUNCH("ffn_dense_rows", (ffn_dense_rows<TS, 8>), gov, blk, 0, s, a, G); break;
    case 16: TWELL_LAUNCH("ffn_dense_rows", (ffn_dense_rows<TS, 16>), gov, blk, 0, s, a, G); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_dense_reduce(a.part, a.ovf_rows, a.n_ovf, a.ovf_cap, G, a.D, a.y, s);
}

// The two row kinds share no buffer (the sparse rows' list workspace vs the
// overflow partials; disjoint rows of y), so the overflow rows run on the side
// stream beside the up / down launches.
template <typename TS>
hipError_t launch_t(const FwdArgs& a, hipStream_t s, int64_t chunk, bool use_side = true) {
  hipStream_t side = s;
  hipError_t err = hipSuccess, err2 = hipSuccess;
  if (a.ovf_cap > 0) {
    if (use_side && (err = fork_side(s, &side)) != hipSuccess) return err;
    err = launch_overflow_rows<TS>(a, side);
  }
  if (err == hipSuccess) err = launch_sparse_rows<TS>(a, s, chunk);
  err2 = join_side(s, side);
  return err != hipSuccess ? err : err2;
}

}  // namespace

hipError_t launch_dense_reduce(const float* part, const int32_t* rows, const int32_t* n_rows, int cap, int G,
                               int D, float* out, hipStream_t s) {
  if (cap == 0) return hipSuccess;
  const int64_t want = ((D + 255) / 256) * (int64_t)cap;
  TWELL_LAUNCH("dense_reduce", dense_reduce, dim3((unsigned)(want < kRowsGrid ? want : kRowsGrid)), 256, 0, s, part,
               rows, n_rows, cap, G, D, out);
  return hipGetLastError();
}

hipError_t launch_ffn_fwd(const FwdArgs& a, hipStream_t s) {
  return a.is_bf16 ? launch_t<uint16_t>(a, s, kTokenChunk) : launch_t<float>(a, s, kTokenChunk);
}

hipError_t launch_forward(const GateArgs& g, const FwdArgs& f, hipStream_t s, bool use_side) {
  if (!use_side) {  // everything in order on `s`
    const hipError_t err = launch_gate_pack(g, s);
    if (err != hipSuccess) return err;
    return f.is_bf16 ? launch_t<uint16_t>(f, s, kTokenChunk, false) : launch_t<float>(f, s, kTokenChunk, false);
  }
  if (gate_ovf_rows_heavy(g)) {  // the two calls' order: overflow list and gate rows on `s` first
    const hipError_t err = launch_gate_pack(g, s);
    return err != hipSuccess ? err : launch_ffn_fwd(f, s);
  }
  hipStream_t side = s;
  hipError_t err = launch_gate_pack_split(g, s, true, &side, f.is_bf16 && up_blocked_applies(f));
  if (side == s) return err != hipSuccess ? err : launch_ffn_fwd(f, s);  // nothing was forked
  if (err == hipSuccess && f.ovf_cap > 0)
    err = f.is_bf16 ? launch_overflow_rows<uint16_t>(f, side) : launch_overflow_rows<float>(f, side);
  if (err == hipSuccess)
    err = f.is_bf16 ? launch_sparse_rows<uint16_t>(f, s, kTokenChunk) : launch_sparse_rows<float>(f, s, kTokenChunk);
  const hipError_t ej = join_side(s, side);
  return err != hipSuccess ? err : ej;
}

}  // namespace twell
