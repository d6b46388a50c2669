// Stage 3b: sparse backward through the hybrid ELL + dense-backup format.
//
// "How TwELL by Sakana AI and NVIDIA Accelerates LLMs by 20%"
// (aimodelsnavi.com), "Core of TwELL" and "Benchmark Data": dedicated kernels
// for training, speedup including backpropagation; "Sakana AI and NVIDIA
// present TwELL" (edge.aivizor.me), second paragraph: the hybrid ELL / dense
// backup format used for training.
//
// For L = sum(dy*y) + lambda*sum(h), at every active (i, c):
//   dz = dy_i . W_down[c]     da = dz*h     dg = dz*a + lambda     z = h*a
//   dx_i += da*W_up^T[c] + dg*W_gate^T[c]
//   dW_down[c] += z*dy_i   dW_up^T[c] += da*x_i   dW_gate^T[c] += dg*x_i
//
// Pipeline (all deterministic, no floating-point atomics):
//   dense_groups  per dense row: active count per column chunk -> offsets
//   row_scan      CSR offsets of every row's entries (one workgroup, rows
//                 held in registers); with the blocked dz, row_scan_groups
//                 runs it in workgroup 0 and the dz's per-row group
//                 positions (ell_groups.h) in the others
//   bwd_dz_ell    wave per ELL row and column part: dz, da, dg, z; writes
//                 each entry's column and (z, da, dg) in CSR order (bf16
//                 batches take the blocked form of bwd_blocked.hip instead)
//   bwd_dz_dense  wave per dense-row chunk: the same, recomputing
//                 a = x_i . W_up^T[c] for dense rows (bf16 layers with d_model
//                 a multiple of 128 take the skinny MFMA products of
//                 bwd_dense.hip instead, which also give those rows' dx)
//   bwd_dx        wave per row: dx from the records
//   csc_*         stable counting sort of the entries by column (per block of
//                 32 rows a bit mask per column, so each column lists its rows
//                 ascending and every record is placed independently)
//   bwd_dw        wave per (column, D-part): the three weight-gradient rows
#include "block_scan.h"
#include "ell_groups.h"
#include "row_ops.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int RB = kTransposeRows;

// --------------------------------------------------------------- dense groups

template <typename TS>
__global__ __launch_bounds__(256) void dense_groups(BwdArgs a, int G, int32_t* dense_nnz) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= a.dense_cap || o >= *a.n_dense) return;
  const TS* h = reinterpret_cast<const TS*>(a.dense_h) + (size_t)o * a.F;
  int run = 0;
  if constexpr (sizeof(TS) == 2) {
    if ((a.F & 7) == 0 && (reinterpret_cast<uintptr_t>(a.dense_h) & 15) == 0) {
      // a 512-column chunk is one 16-byte load per lane (lane l: columns
      // 8l .. 8l+7), eight chunks in flight; a bf16 h is active iff its bits
      // are in [1, 0x7fff] (positive, not zero)
      const uint4* hv = reinterpret_cast<const uint4*>(h);
      const int nv = a.F / 8;
      for (int g0 = 0; g0 < G; g0 += 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int q = (g0 + u) * 64 + lane;
          v[u] = q < nv ? hv[q] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (g0 + u >= G) break;
          if (lane == 0) a.ws.grp_off[(size_t)o * G + g0 + u] = run;
          int cnt = 0;
          const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            cnt += ((w[e] & 0xffffu) - 1u < 0x7fffu) + ((w[e] >> 16) - 1u < 0x7fffu);
          run += (int)wave_sum_dpp((float)cnt);  // exact: at most 512
        }
      }
      if (lane == 0) dense_nnz[o] = run;
      return;
    }
  }
#pragma unroll 2
  for (int g = 0; g < G; ++g) {
    if (lane == 0) a.ws.grp_off[(size_t)o * G + g] = run;
    // the chunk's eight 64-column blocks are loaded together (clamped column,
    // no branch around the load), then counted
    float v[kDenseChunk / 64];
#pragma unroll
    for (int b = 0; b < kDenseChunk / 64; ++b) {
      const int c = g * kDenseChunk + b * 64 + lane;
      const float hv = Store<TS>::load(h, min(c, a.F - 1));
      v[b] = c < a.F ? hv : 0.f;
    }
#pragma unroll
    for (int b = 0; b < kDenseChunk / 64; ++b) run += __popcll(ballot(v[b] > 0.f));
  }
  if (lane == 0) dense_nnz[o] = run;
}

// --------------------------------------------------------------- CSR offsets

__device__ void block_exclusive_scan(int32_t* part, int tid) {
  // part[0..1023] -> inclusive scan in place (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
}

// Effective entry count of a row: row_nnz for ELL rows, the dense row's own
// count for dense rows inside the capacity, 0 for dense rows beyond it. One
// workgroup; thread t owns rows [t*C, t*C + C), held in registers, so all of
// a thread's loads are issued together.
template <int C>
__device__ __forceinline__ void row_scan_block(const BwdArgs& a, const int32_t* dense_nnz) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x;
  const int64_t N = a.N;
  const int64_t b = (int64_t)tid * C;
  const int nd = min(*a.n_dense, a.dense_cap);
  bool dn[C];
  int32_t nz[C];
  int32_t cnt = 0;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    const int64_t i = b + k;
    dn[k] = i < N && a.is_dense[i] != 0;
    nz[k] = i < N ? min(a.row_nnz[i], a.row_cap) : 0;
    cnt += dn[k];
  }
  int32_t tot;
  int32_t dpos = block_excl_1024(cnt, wsum, &tot);
  int32_t eff[C], dp[C];
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    dp[k] = dn[k] ? dpos++ : -1;
    eff[k] = dn[k] ? (dp[k] < nd ? dense_nnz[dp[k]] : 0) : nz[k];
    s += eff[k];
  }
  int32_t run = block_excl_1024(s, wsum, &tot);
#pragma unroll
  for (int k = 0; k < C; ++k) {
    const int64_t i = b + k;
    if (i < N) {
      a.ws.dense_pos[i] = dp[k];
      a.ws.row_ptr[i] = run;
    }
    run += eff[k];
  }
  if (tid == 1023) a.ws.row_ptr[N] = tot;
}

template <int C>
__global__ __launch_bounds__(1024) void row_scan(BwdArgs a, const int32_t* dense_nnz) {
  row_scan_block<C>(a, dense_nnz);
}

// The row offsets (workgroup 0) and the blocked dz's per-row group positions
// (the other workgroups, a wave per row, each XCD a contiguous run of rows)
// in one launch: the two are independent, and the single-workgroup scan is
// bound by the latency of its loads, so the group pass runs in its shadow.
template <int C>
__global__ __launch_bounds__(1024) void row_scan_groups(BwdArgs a, const int32_t* dense_nnz, int n_groups) {
  if (blockIdx.x == 0) {
    row_scan_block<C>(a, dense_nnz);
    return;
  }
  const int64_t i = xcd_run_block(blockIdx.x - 1, gridDim.x - 1) * 16 + (threadIdx.x >> 6);
  if (i < a.N) ell_groups_row(a, n_groups, i);
}

// The same for any N (beyond 32768 rows): thread t walks rows
// [t*chunk, (t+1)*chunk) three times.
__global__ __launch_bounds__(1024) void row_scan_any(BwdArgs a, const int32_t* dense_nnz) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t N = a.N;
  const int64_t chunk = (N + 1023) / 1024;
  const int64_t b = min(N, (int64_t)tid * chunk), en = min(N, b + chunk);
  const int nd = min(*a.n_dense, a.dense_cap);
  int32_t c = 0;
  for (int64_t i = b; i < en; ++i) c += a.is_dense[i] != 0;
  part[tid] = c;
  __syncthreads();
  block_exclusive_scan(part, tid);
  int32_t dpos = part[tid] - c;
  int32_t s = 0;
  for (int64_t i = b; i < en; ++i) {
    int32_t eff;
    if (a.is_dense[i]) {
      a.ws.dense_pos[i] = dpos;
      eff = dpos < nd ? dense_nnz[dpos] : 0;
      ++dpos;
    } else {
      a.ws.dense_pos[i] = -1;
      eff = min(a.row_nnz[i], a.row_cap);
    }
    s += eff;
  }
  __syncthreads();
  part[tid] = s;
  __syncthreads();
  block_exclusive_scan(part, tid);
  int32_t run = part[tid] - s;
  for (int64_t i = b; i < en; ++i) {
    a.ws.row_ptr[i] = run;
    const int32_t dp = a.ws.dense_pos[i];
    run += dp >= 0 ? (dp < nd ? dense_nnz[dp] : 0) : min(a.row_nnz[i], a.row_cap);
  }
  if (tid == 1023) a.ws.row_ptr[N] = part[1023];
}

// --------------------------------------------------------------- dz pass

// ELL rows. Part p (= XCD p when parts = 8) owns the columns
// [p*F/parts, (p+1)*F/parts), so each XCD gathers only its 1/8 of W_down's
// rows. One wave per (row, part): dy_i in registers, the row's ELL entries in
// range (contiguous: ELL columns ascend) taken 64 at a time, U W_down rows in
// flight, dz = dy_i . W_down[c] reduced with DPP; then every lane writes the
// record of its entry: column and (z, da, dg) = (h*a, dz*h, dz*a + lambda).
template <typename TS, int M>
__global__ __launch_bounds__(256) void bwd_dz_ell(BwdArgs a, int parts) {
  constexpr int E = ChunkElems<TS>::E;
  constexpr int U = M <= 4 ? 4 : (M == 8 ? 2 : 1);
  const int lane = threadIdx.x & 63;
  const int part = blockIdx.x % parts;
  const int64_t i = (int64_t)(blockIdx.x / parts) * 4 + (threadIdx.x >> 6);
  const int64_t N = a.N;
  if (i >= N || a.is_dense[i]) return;
  const int n = min(a.row_nnz[i], a.row_cap);
  const int clo = (int)((int64_t)part * a.F / parts), chi = (int)((int64_t)(part + 1) * a.F / parts);
  const int D = a.D, nch = D / E;
  const int32_t p0 = a.ws.row_ptr[i];
  const TS* __restrict__ wd = reinterpret_cast<const TS*>(a.w_down);
  const TS* __restrict__ ev = reinterpret_cast<const TS*>(a.ell_vals);
  u32x4_t dyr[M];
  bool have_dy = false;
  for (int kb = 0; kb < n; kb += 64) {
    const int k = kb + lane;
    const size_t off = (size_t)k * N + i;
    const int c_l = k < n ? a.ell_cols[off] : -1;
    const uint64_t m = ballot(c_l >= clo && c_l < chi);
    if (m == 0) continue;
    const int first = __ffsll((unsigned long long)m) - 1, cnt = __popcll(m);
    const bool mine = (m >> lane) & 1ull;
    float h_l = 0.f, a_l = 0.f;
    if (mine) {
      h_l = Store<TS>::load(ev, off);
      a_l = a.ell_a[off];
    }
    if (!have_dy) {
      load_row<TS, M>(dyr, reinterpret_cast<const TS*>(a.dy) + (size_t)i * D, nch, lane);
      have_dy = true;
    }
    float dz_l = 0.f;
    for (int q = 0; q < cnt; q += U) {
      u32x4_t wr[U][M];
#pragma unroll
      for (int u = 0; u < U; ++u)
        load_row<TS, M>(wr[u], wd + (size_t)readlane_i(c_l, first + min(q + u, cnt - 1)) * D, nch, lane);
      float dot[U];
#pragma unroll
      for (int u = 0; u < U; ++u) dot[u] = wave_sum_dpp(dot_rows<TS, M>(dyr, wr[u]));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (lane == first + q + u) dz_l = dot[u];
    }
    if (mine) {
      a.ws.pair_col[p0 + k] = c_l;
      a.ws.coef[p0 + k] = make_float4(h_l * a_l, dz_l * h_l, fmaf(dz_l, a_l, a.lam), 0.f);
    }
  }
}

// Dense-backup rows. Work item (o, g): dense row o, columns
// [g*kDenseChunk, ...). The active columns (h > 0) of each 64-column block are
// compacted into lanes; for each, dz = dy_i . W_down[c] and the up activation
// a = x_i . W_up^T[c] (not saved for these rows) are reduced, then the
// records go to positions row_ptr[i] + grp_off[o][g] + rank.
template <typename TS, int M>
__global__ __launch_bounds__(256) void bwd_dz_dense(BwdArgs a, int G) {
  constexpr int E = ChunkElems<TS>::E;
  constexpr int U = M <= 4 ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int o = (int)(item / G), g = (int)(item % G);
  if (o >= a.dense_cap || o >= *a.n_dense) return;
  const int D = a.D, nch = D / E;
  const int64_t i = a.dense_rows[o];
  const TS* __restrict__ wd = reinterpret_cast<const TS*>(a.w_down);
  const TS* __restrict__ wu = reinterpret_cast<const TS*>(a.w_up);
  const TS* __restrict__ hrow = reinterpret_cast<const TS*>(a.dense_h) + (size_t)o * a.F;
  u32x4_t dyr[M], xr[M];
  load_row<TS, M>(dyr, reinterpret_cast<const TS*>(a.dy) + (size_t)i * D, nch, lane);
  load_row<TS, M>(xr, reinterpret_cast<const TS*>(a.x) + (size_t)i * D, nch, lane);
  int32_t p = a.ws.row_ptr[i] + a.ws.grp_off[(size_t)o * G + g];
  const int c0 = g * kDenseChunk, c1 = min(a.F, c0 + kDenseChunk);
  for (int cb = c0; cb < c1; cb += 64) {
    const int c = cb + lane;
    const float h_c = c < c1 ? Store<TS>::load(hrow, c) : 0.f;
    const uint64_t m = ballot(h_c > 0.f);
    const int n = __popcll(m);
    if (n == 0) continue;
    // lane q of the list gets the q-th active column (binary search on prefix popcounts)
    int lo = 0, hi = 63;
    for (int step = 0; step < 6; ++step) {
      const int mid = (lo + hi) >> 1;
      const uint64_t below = mid >= 63 ? ~0ull : ((2ull << mid) - 1ull);
      if (__popcll(m & below) >= lane + 1) hi = mid; else lo = mid + 1;
    }
    const int col_l = cb + lo;
    const float h_l = __shfl(h_c, lo, 64);
    float dz_l = 0.f, a_l = 0.f;
    for (int q = 0; q < n; q += U) {
      u32x4_t wr[U][M], ur[U][M];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t row = (size_t)readlane_i(col_l, min(q + u, n - 1)) * D;
        load_row<TS, M>(wr[u], wd + row, nch, lane);
        load_row<TS, M>(ur[u], wu + row, nch, lane);
      }
      float dz[U], av[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        dz[u] = wave_sum_dpp(dot_rows<TS, M>(dyr, wr[u]));
        av[u] = wave_sum_dpp(dot_rows<TS, M>(xr, ur[u]));
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (lane == q + u) {
          dz_l = dz[u];
          a_l = av[u];
        }
    }
    if (lane < n) {
      a.ws.pair_col[p + lane] = col_l;
      a.ws.coef[p + lane] = make_float4(h_l * a_l, dz_l * h_l, fmaf(dz_l, a_l, a.lam), 0.f);
    }
    p += n;
  }
}

// --------------------------------------------------------------- dx pass

// Lane group g of a sliced wave reads entry k + u*RPI + g: a wave-uniform
// readlane when one group spans the wave, else a cross-lane shuffle.
template <int RPI>
__device__ __forceinline__ int entry_i(int v, int k) {
  if constexpr (RPI == 1) return __builtin_amdgcn_readlane(v, k);
  else return __shfl(v, k, 64);
}
template <int RPI>
__device__ __forceinline__ float entry_f(float v, int k) {
  if constexpr (RPI == 1) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
  else return __shfl(v, k, 64);
}

// Every row (ELL and dense-backup alike, except dense rows whose dx the MFMA
// path of bwd_dense.hip computes): its records are contiguous in CSR order. Part p owns a d_model slice of dx (pick_l2_slices; slices go G8 at a
// time, slice_block), so each XCD gathers only a slice of the weight that
// fits its L2, 16 bytes per lane. Two launches, one weight each:
//   GATE = false:  dx_i[slice]  = sum over records da * W_up^T[c][slice]
//   GATE = true:   dx_i[slice] += sum over records dg * W_gate^T[c][slice]
// Dense rows beyond the dense capacity have no records and get dx = 0.
template <typename TS, int EPL, int RPI, bool GATE>
__global__ __launch_bounds__(256) void bwd_dx(BwdArgs a, int G8, int64_t rblocks) {
  constexpr int LPR = 64 / RPI;
  constexpr int U = sliced_inflight<RPI>();
  const int lane = threadIdx.x & 63;
  int p;
  int64_t rb;
  slice_block(blockIdx.x, G8, rblocks, p, rb);
  const int64_t i = rb * 4 + (threadIdx.x >> 6);
  if (i >= a.N) return;
  if (a.ws.dxpart != nullptr) {  // dense rows inside the capacity: dx from the MFMA path
    const int dp = a.ws.dense_pos[i];
    if (dp >= 0 && dp < min(*a.n_dense, a.dense_cap)) return;
  }
  const int D = a.D;
  const int d0 = p * (LPR * EPL) + (lane % LPR) * EPL;
  const TS* __restrict__ wt = reinterpret_cast<const TS*>(GATE ? a.w_gate : a.w_up) + d0;
  const int32_t q0 = a.ws.row_ptr[i], q1 = a.ws.row_ptr[i + 1];
  float* dst = a.dx + (size_t)i * D + d0;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = (GATE && lane < LPR) ? dst[e] : 0.f;
  for (int qb = q0; qb < q1; qb += 64) {
    const int n = min(64, q1 - qb);
    int c_l = 0;
    float k_l = 0.f;
    if (lane < n) {
      c_l = a.ws.pair_col[qb + lane];
      const float4 cf = a.ws.coef[qb + lane];
      k_l = GATE ? cf.z : cf.y;
    }
    sliced_axpy<TS, EPL, RPI, U>(wt, D, a.F, c_l, k_l, n, lane, acc);
  }
  combine_groups<EPL, RPI>(acc);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = acc[e];
  }
}

// --------------------------------------------------------------- column transpose

// Stable counting sort of the records by column, in blocks of RB = 32 rows.
// For every block and column, bit r of mask[b][c] says whether row b*32 + r
// has an entry in column c; it is built with LDS atomicOr, which gives the
// same bits in any order, so everything below is deterministic. A record of
// row i in column c then goes to
//   col_ptr[c] + rel[b][c] + popcount(mask[b][c] & (bits below i's)),
// where rel[b][c] counts the column's entries in earlier blocks: rows ascend
// within every column, with every record placed independently.
constexpr int kMaxTransposeF = 32768;  // d_ff the LDS masks cover (the backward's limit)

// Wave w of the block takes rows r0 + w, r0 + w + 4, ...; lane l entries l,
// l + 64, ... of the row. `body` gets the record index, its column and the
// row's bit in the block.
template <typename Body>
__device__ __forceinline__ void csc_block_rows(const int32_t* __restrict__ row_ptr,
                                               const int32_t* __restrict__ pair_col, int64_t r0, int64_t r1,
                                               Body&& body) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t i = r0 + wave; i < r1; i += 4) {
    const int32_t e = row_ptr[i + 1];
    for (int32_t p = row_ptr[i] + lane; p < e; p += 64) body(p, pair_col[p], (int)(i - r0));
  }
}

// FMAX: the largest d_ff of the instantiation (its LDS is FMAX words, so
// smaller d_ff leave room for other workgroups on the CU).
template <int FMAX>
__global__ __launch_bounds__(256) void csc_mask(const int32_t* __restrict__ row_ptr,
                                                const int32_t* __restrict__ pair_col, int64_t N, int F,
                                                uint32_t* __restrict__ masks) {
  __shared__ uint32_t m[FMAX];
  for (int q = threadIdx.x; q < F; q += 256) m[q] = 0u;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * RB, r1 = min(N, r0 + RB);
  csc_block_rows(row_ptr, pair_col, r0, r1, [&](int32_t, int c, int r) { atomicOr(&m[c], 1u << r); });
  __syncthreads();
  uint32_t* out = masks + (size_t)blockIdx.x * F;
  for (int q = threadIdx.x; q < F; q += 256) out[q] = m[q];
}

// Per column: rel[b][c] = entries of column c in blocks before b, and the
// column's total into col_ptr[c]. A workgroup takes 64 columns; its 16 waves
// each sum a sixteenth of the blocks (popcounts kept in registers, 8 loads in
// flight), then add the sixteenths before theirs.
constexpr int kColpreWaves = 16;
__global__ __launch_bounds__(64 * kColpreWaves) void csc_colpre(const uint32_t* __restrict__ masks, int nrb, int F,
                                                                int32_t* __restrict__ rel,
                                                                int32_t* __restrict__ col_ptr) {
  __shared__ int32_t part[kColpreWaves][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int b0 = (int)((int64_t)nrb * q / kColpreWaves), b1 = (int)((int64_t)nrb * (q + 1) / kColpreWaves);
  int32_t s = 0;
  if (c < F) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = masks[(size_t)(b + u) * F + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += __popc(v[u]);
    }
    for (; b < b1; ++b) s += __popc(masks[(size_t)b * F + c]);
  }
  part[q][lane] = s;
  __syncthreads();
  int32_t run = 0;
  for (int k = 0; k < q; ++k) run += part[k][lane];
  if (c >= F) return;
  for (int b = b0; b < b1; ++b) {
    rel[(size_t)b * F + c] = run;
    run += __popc(masks[(size_t)b * F + c]);
  }
  if (q == kColpreWaves - 1) col_ptr[c] = run;
}

// col_ptr[0..F) -> exclusive offsets, col_ptr[F] = total (one workgroup,
// C consecutive columns per thread).
template <int C>
__global__ __launch_bounds__(1024) void csc_colscan(int32_t* col_ptr, int F) {
  __shared__ int32_t wsum[16];
  const int b = threadIdx.x * C;
  int32_t v[C];
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    v[k] = b + k < F ? col_ptr[b + k] : 0;
    s += v[k];
  }
  int32_t tot;
  int32_t run = block_excl_1024(s, wsum, &tot);
#pragma unroll
  for (int k = 0; k < C; ++k) {
    if (b + k < F) col_ptr[b + k] = run;
    run += v[k];
  }
  if (threadIdx.x == 0) col_ptr[F] = tot;
}

__global__ __launch_bounds__(256) void csc_fill(const int32_t* __restrict__ row_ptr,
                                                const int32_t* __restrict__ pair_col,
                                                const uint32_t* __restrict__ masks, const int32_t* __restrict__ rel,
                                                const int32_t* __restrict__ col_ptr, int64_t N, int F,
                                                int32_t* __restrict__ csc_pair, int32_t* __restrict__ csc_row) {
  const int64_t r0 = (int64_t)blockIdx.x * RB, r1 = min(N, r0 + RB);
  const size_t bo = (size_t)blockIdx.x * F;
  csc_block_rows(row_ptr, pair_col, r0, r1, [&](int32_t p, int c, int r) {
    const int32_t pos = col_ptr[c] + rel[bo + c] + __popc(masks[bo + c] & ((1u << r) - 1u));
    csc_pair[pos] = p;
    csc_row[pos] = (int32_t)(r0 + r);
  });
}

// --------------------------------------------------------------- weight gradients

// Wave per (column c, d_model slice p): the column's records in ascending row
// order (from the column transpose), token-row slices read 16 bytes per lane,
// one slice per XCD (slice_block). Two launches, one token matrix each:
//   X = false:  dW_down[c][slice]   = sum z  * dy_i[slice]
//   X = true:   dW_up^T[c][slice]   = sum da * x_i[slice],
//               dW_gate^T[c][slice] = sum dg * x_i[slice].
template <typename TS, int EPL, int RPI, bool X>
__global__ __launch_bounds__(256) void bwd_dw(BwdArgs a, int G8, int64_t cblocks) {
  constexpr int LPR = 64 / RPI;
  constexpr int U = sliced_inflight<RPI>();
  const int lane = threadIdx.x & 63, g = lane / LPR;
  int p;
  int64_t cb;
  slice_block(blockIdx.x, G8, cblocks, p, cb);
  const int64_t c = cb * 4 + (threadIdx.x >> 6);
  if (c >= a.F) return;
  const int D = a.D;
  const int d0 = p * (LPR * EPL) + (lane % LPR) * EPL;
  const TS* __restrict__ src = reinterpret_cast<const TS*>(X ? a.x : a.dy) + d0;
  float acc0[EPL], acc1[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc0[e] = acc1[e] = 0.f;
  const int32_t q0 = a.ws.col_ptr[c], q1 = a.ws.col_ptr[c + 1];
  for (int qb = q0; qb < q1; qb += 64) {
    const int n = min(64, q1 - qb);
    int i_l = 0;
    float4 cf = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < n) {
      i_l = a.ws.csc_row[qb + lane];
      cf = a.ws.coef[a.ws.csc_pair[qb + lane]];
    }
    const float k0_l = X ? cf.y : cf.x;
    for (int k = 0; k < n; k += U * RPI) {
      Slice<TS, EPL> sr[U];
      float k0[U], k1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k + u * RPI + g;
        const int ks = min(kk, n - 1);
        const bool ok = kk < n;
        const size_t row = (size_t)entry_i<RPI>(i_l, ks) * D;
        const float v0 = entry_f<RPI>(k0_l, ks);
        k0[u] = ok ? v0 : 0.f;
        if (X) {
          const float v1 = entry_f<RPI>(cf.z, ks);
          k1[u] = ok ? v1 : 0.f;
        }
        sr[u].load(src + row);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sr[u].fma(k0[u], acc0);
        if (X) sr[u].fma(k1[u], acc1);
      }
    }
  }
  combine_groups<EPL, RPI>(acc0);
  if (X) combine_groups<EPL, RPI>(acc1);
  if (lane < LPR) {
    const size_t ro = (size_t)c * D + d0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if (X) {
        a.dw_up[ro + e] = acc0[e];
        a.dw_gate[ro + e] = acc1[e];
      } else {
        a.dw_down[ro + e] = acc0[e];
      }
    }
  }
}

// Column transpose of the records (stable: rows ascend within a column).
hipError_t launch_csc(const BwdArgs& a, hipStream_t s, int nrb) {
  if (a.F > kMaxTransposeF) return hipErrorInvalidValue;
  uint32_t* masks = reinterpret_cast<uint32_t*>(a.ws.blk_cnt);
  int32_t* rel = a.ws.blk_cnt + (size_t)nrb * a.F;
  if (a.F <= 8192)
    TWELL_LAUNCH("csc_mask", csc_mask<8192>, dim3(nrb), 256, 0, s, a.ws.row_ptr, a.ws.pair_col, a.N, a.F, masks);
  else if (a.F <= 16384)
    TWELL_LAUNCH("csc_mask", csc_mask<16384>, dim3(nrb), 256, 0, s, a.ws.row_ptr, a.ws.pair_col, a.N, a.F, masks);
  else
    TWELL_LAUNCH("csc_mask", csc_mask<kMaxTransposeF>, dim3(nrb), 256, 0, s, a.ws.row_ptr, a.ws.pair_col, a.N, a.F,
                 masks);
  TWELL_LAUNCH("csc_colpre", csc_colpre, dim3((a.F + 63) / 64), 64 * kColpreWaves, 0, s, masks, nrb, a.F, rel,
               a.ws.col_ptr);
  if (a.F <= 8192)
    TWELL_LAUNCH("csc_colscan", csc_colscan<8>, 1, 1024, 0, s, a.ws.col_ptr, a.F);
  else
    TWELL_LAUNCH("csc_colscan", csc_colscan<32>, 1, 1024, 0, s, a.ws.col_ptr, a.F);
  TWELL_LAUNCH("csc_fill", csc_fill, dim3(nrb), 256, 0, s, a.ws.row_ptr, a.ws.pair_col, masks, rel, a.ws.col_ptr,
               a.N, a.F, a.ws.csc_pair, a.ws.csc_row);
  return hipGetLastError();
}

// dx: every row, d_model sliced to fit a slice of W_up (F rows) in L2.
template <typename TS>
hipError_t launch_dx(const BwdArgs& a, hipStream_t s) {
  const dim3 blk(256);
  const SliceGeom geom = pick_l2_slices(a.D, (int)sizeof(TS), a.F);
  const int P = geom.P, G8 = slice_group(P);
  const int64_t rblocks = (a.N + 3) / 4;
  const dim3 gdx((unsigned)(rblocks * P));
#define TWELL_DX(E, R) TWELL_LAUNCH("bwd_dx", (bwd_dx<TS, E, R, false>), gdx, blk, 0, s, a, G8, rblocks)
#define TWELL_DXG(E, R) TWELL_LAUNCH("bwd_dx_gate", (bwd_dx<TS, E, R, true>), gdx, blk, 0, s, a, G8, rblocks)
  if constexpr (sizeof(TS) == 2) {
    TWELL_SLICED_CASES(8, TWELL_DX)
    TWELL_SLICED_CASES(8, TWELL_DXG)
  } else {
    TWELL_SLICED_CASES(4, TWELL_DX)
    TWELL_SLICED_CASES(4, TWELL_DXG)
  }
#undef TWELL_DX
#undef TWELL_DXG
  return hipGetLastError();
}

// Weight gradients: column-owned, d_model in 1/8 slices (slicing x / dy
// further to fit L2 measured slower here: a column's tokens ascend, so its
// gathers already fall close together).
template <typename TS>
hipError_t launch_dw(const BwdArgs& a, hipStream_t s) {
  const dim3 blk(256);
  const SliceGeom geom = pick_slices(a.D, (int)sizeof(TS));
  const int P = geom.P, G8 = slice_group(P);
  const int64_t cblocks = (a.F + 3) / 4;
  const dim3 gdw((unsigned)(cblocks * P));
#define TWELL_DWD(E, R) TWELL_LAUNCH("bwd_dw_down", (bwd_dw<TS, E, R, false>), gdw, blk, 0, s, a, G8, cblocks)
#define TWELL_DW(E, R) TWELL_LAUNCH("bwd_dw", (bwd_dw<TS, E, R, true>), gdw, blk, 0, s, a, G8, cblocks)
  if constexpr (sizeof(TS) == 2) {
    TWELL_SLICED_CASES(8, TWELL_DWD)
    TWELL_SLICED_CASES(8, TWELL_DW)
  } else {
    TWELL_SLICED_CASES(4, TWELL_DWD)
    TWELL_SLICED_CASES(4, TWELL_DW)
  }
#undef TWELL_DWD
#undef TWELL_DW
  return hipGetLastError();
}

// Rows per thread of row_scan: the smallest power of two covering N / 1024
// (64 and more would spill: those N take row_scan_any).
int row_scan_rows(int64_t N) {
  int c = 1;
  while ((int64_t)c * 1024 < N && c < 64) c *= 2;
  return c;
}

template <typename TS>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
  constexpr int E = ChunkElems<TS>::E;
  const int nch = a.D / E;
  const int M = pick_m(nch);
  const int G = (a.F + kDenseChunk - 1) / kDenseChunk;
  const int nrb = (int)((a.N + RB - 1) / RB);
  int32_t* dense_nnz = a.ws.row_ptr + a.N + 1;  // [dense_cap] lives after row_ptr
  const dim3 blk(256);
  hipError_t err;

  // The dense-backup rows' dz and a (matrix cores) need only the dense-row
  // list, so they start on the side stream first, beside the row offsets and
  // the ELL rows' dz; their records follow once the offsets exist.
  hipStream_t side = s;
  const bool dense_mfma = sizeof(TS) == 2 && bwd_dense_mfma_applies(a);
  if (a.dense_cap > 0 && dense_mfma) {
    if ((err = fork_side(s, &side)) != hipSuccess) return err;
    if ((err = launch_bwd_dense_nt(a, side)) != hipSuccess) {
      (void)join_side(s, side);
      return err;
    }
  }
  if (a.dense_cap > 0) {
    TWELL_LAUNCH("dense_groups", dense_groups<TS>, dim3((a.dense_cap + 3) / 4), blk, 0, s, a, G, dense_nnz);
  }
  // with the blocked dz, its per-row group positions ride along with the row
  // offsets (one launch: 1 + one workgroup per 16 rows)
  const bool dz_blocked = sizeof(TS) == 2 && dz_blocked_applies(a);
  const int rs = row_scan_rows(a.N);
  const bool fused = dz_blocked && rs <= 32;
  if (fused) {
    const int ng = dz_groups(a.F);
    const dim3 gg((unsigned)(1 + (a.N + 15) / 16));
    switch (rs) {
      case 1: TWELL_LAUNCH("row_scan_groups", row_scan_groups<1>, gg, 1024, 0, s, a, dense_nnz, ng); break;
      case 2: TWELL_LAUNCH("row_scan_groups", row_scan_groups<2>, gg, 1024, 0, s, a, dense_nnz, ng); break;
      case 4: TWELL_LAUNCH("row_scan_groups", row_scan_groups<4>, gg, 1024, 0, s, a, dense_nnz, ng); break;
      case 8: TWELL_LAUNCH("row_scan_groups", row_scan_groups<8>, gg, 1024, 0, s, a, dense_nnz, ng); break;
      case 16: TWELL_LAUNCH("row_scan_groups", row_scan_groups<16>, gg, 1024, 0, s, a, dense_nnz, ng); break;
      default: TWELL_LAUNCH("row_scan_groups", row_scan_groups<32>, gg, 1024, 0, s, a, dense_nnz, ng); break;
    }
  } else {
    switch (rs) {
      case 1: TWELL_LAUNCH("row_scan", row_scan<1>, 1, 1024, 0, s, a, dense_nnz); break;
      case 2: TWELL_LAUNCH("row_scan", row_scan<2>, 1, 1024, 0, s, a, dense_nnz); break;
      case 4: TWELL_LAUNCH("row_scan", row_scan<4>, 1, 1024, 0, s, a, dense_nnz); break;
      case 8: TWELL_LAUNCH("row_scan", row_scan<8>, 1, 1024, 0, s, a, dense_nnz); break;
      case 16: TWELL_LAUNCH("row_scan", row_scan<16>, 1, 1024, 0, s, a, dense_nnz); break;
      case 32: TWELL_LAUNCH("row_scan", row_scan<32>, 1, 1024, 0, s, a, dense_nnz); break;
      default: TWELL_LAUNCH("row_scan", row_scan_any, 1, 1024, 0, s, a, dense_nnz); break;
    }
  }

  // dz records: ELL rows by column part (main stream), dense rows by column
  // chunk (side stream: disjoint record ranges), past the row offsets
  if (a.dense_cap > 0) {
    hipStream_t side2 = s;
    if ((err = fork_side(s, &side2)) != hipSuccess) {
      (void)join_side(s, side);
      return err;
    }
    if (side2 != side) {  // not the stream of the first fork: finish that branch first
      if ((err = join_side(s, side)) != hipSuccess) return err;
      side = side2;
    }
    const dim3 gdd((unsigned)(((int64_t)a.dense_cap * G + 3) / 4));
    if (dense_mfma) {
      err = launch_bwd_dense_records(a, side);
      if (err != hipSuccess) {
        (void)join_side(s, side);
        return err;
      }
    } else {
    switch (M) {
      case 1: TWELL_LAUNCH("bwd_dz_dense", (bwd_dz_dense<TS, 1>), gdd, blk, 0, side, a, G); break;
      case 2: TWELL_LAUNCH("bwd_dz_dense", (bwd_dz_dense<TS, 2>), gdd, blk, 0, side, a, G); break;
      case 4: TWELL_LAUNCH("bwd_dz_dense", (bwd_dz_dense<TS, 4>), gdd, blk, 0, side, a, G); break;
      case 8: TWELL_LAUNCH("bwd_dz_dense", (bwd_dz_dense<TS, 8>), gdd, blk, 0, side, a, G); break;
      case 16: TWELL_LAUNCH("bwd_dz_dense", (bwd_dz_dense<TS, 16>), gdd, blk, 0, side, a, G); break;
      default: (void)join_side(s, side); return hipErrorInvalidValue;
    }
    if ((err = hipGetLastError()) != hipSuccess) {
      (void)join_side(s, side);
      return err;
    }
    }
  }
  const int parts = 8;
  const dim3 gdz((unsigned)(((a.N + 3) / 4) * parts));
  if (dz_blocked) {
    err = launch_dz_blocked(a, s, fused);
  } else {
  switch (M) {
    case 1: TWELL_LAUNCH("bwd_dz_ell", (bwd_dz_ell<TS, 1>), gdz, blk, 0, s, a, parts); break;
    case 2: TWELL_LAUNCH("bwd_dz_ell", (bwd_dz_ell<TS, 2>), gdz, blk, 0, s, a, parts); break;
    case 4: TWELL_LAUNCH("bwd_dz_ell", (bwd_dz_ell<TS, 4>), gdz, blk, 0, s, a, parts); break;
    case 8: TWELL_LAUNCH("bwd_dz_ell", (bwd_dz_ell<TS, 8>), gdz, blk, 0, s, a, parts); break;
    case 16: TWELL_LAUNCH("bwd_dz_ell", (bwd_dz_ell<TS, 16>), gdz, blk, 0, s, a, parts); break;
    default: (void)join_side(s, side); return hipErrorInvalidValue;
  }
  err = hipGetLastError();
  }
  const hipError_t ej = join_side(s, side);
  if (err != hipSuccess) return err;
  if (ej != hipSuccess) return ej;

  // column transpose of the records on the side stream (only the weight
  // gradients read it), beside dx on the main stream
  if ((err = fork_side(s, &side)) != hipSuccess) return err;
  if ((err = launch_csc(a, side, nrb)) != hipSuccess) {
    (void)join_side(s, side);
    return err;
  }
  // then, past a mark the weight gradients wait for, dx of the dense rows
  // (bwd_dx leaves those rows alone); it runs on beside the weight gradients
  if ((err = mark_side(s, side)) != hipSuccess || (dense_mfma && (err = launch_bwd_dense_dx(a, side)) != hipSuccess)) {
    (void)join_side(s, side);
    return err;
  }

  err = launch_dx<TS>(a, s);
  const hipError_t ej2 = wait_mark(s, side);
  if (err != hipSuccess || ej2 != hipSuccess) {
    (void)join_side(s, side);
    return err != hipSuccess ? err : ej2;
  }

  err = launch_dw<TS>(a, s);
  const hipError_t ej3 = join_side(s, side);
  return err != hipSuccess ? err : ej3;
}

}  // namespace

hipError_t launch_ffn_bwd(const BwdArgs& a, hipStream_t s) {
  return a.is_bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace twell
