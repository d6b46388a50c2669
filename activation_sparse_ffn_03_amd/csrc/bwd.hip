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
//   row_scan      CSR offsets of every row's entries (one workgroup)
//   bwd_rows      wave per ELL row / per dense-row chunk: dz, da, dg, z and the
//                 dx row (dense rows recompute a = x_i . W_up^T[c]); writes
//                 each entry's column and (z, da, dg) in CSR order
//   dense_reduce  dx of dense rows = sum of the chunk partials
//   csc_*         stable counting sort of the entries by column (row blocks
//                 processed row by row, so each column lists rows ascending)
//   bwd_dw        wave per (column, D-part): the three weight-gradient rows
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
  for (int g = 0; g < G; ++g) {
    if (lane == 0) a.ws.grp_off[(size_t)o * G + g] = run;
    const int c1 = min(a.F, (g + 1) * kDenseChunk);
    for (int cb = g * kDenseChunk; cb < c1; cb += 64) {
      const int c = cb + lane;
      run += __popcll(ballot(c < c1 && Store<TS>::load(h, c) > 0.f));
    }
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
// count for dense rows inside the capacity, 0 for dense rows beyond it.
__global__ __launch_bounds__(1024) void row_scan(BwdArgs a, const int32_t* dense_nnz) {
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

// --------------------------------------------------------------- row pass

template <typename TS, int M>
__device__ __forceinline__ void bwd_pair(const BwdArgs& a, int nch, int lane, const u32x4_t (&dyr)[M],
                                         const u32x4_t (&xr)[M], bool recompute_a, float (&acc)[M][8], int c,
                                         float h, float av, int32_t p) {
  const TS* __restrict__ wd = reinterpret_cast<const TS*>(a.w_down);
  const TS* __restrict__ wu = reinterpret_cast<const TS*>(a.w_up);
  const TS* __restrict__ wg = reinterpret_cast<const TS*>(a.w_gate);
  const int D = a.D;
  const bool ok = c >= 0 && c < a.F;  // defensive: a corrupted column contributes nothing
  if (!ok) {
    c = 0;
    h = 0.f;
  }
  u32x4_t wr[M];
  load_row<TS, M>(wr, wd + (size_t)c * D, nch, lane);
  const float dz = wave_sum(dot_rows<TS, M>(dyr, wr));
  load_row<TS, M>(wr, wu + (size_t)c * D, nch, lane);
  if (recompute_a) av = wave_sum(dot_rows<TS, M>(xr, wr));
  const float da = ok ? dz * h : 0.f;
  const float dg = ok ? fmaf(dz, av, a.lam) : 0.f;
  const float z = h * av;
  axpy_row<TS, M>(acc, da, wr);
  load_row<TS, M>(wr, wg + (size_t)c * D, nch, lane);
  axpy_row<TS, M>(acc, dg, wr);
  if (lane == 0) {
    a.ws.pair_col[p] = c;
    a.ws.coef[p] = make_float4(z, da, dg, 0.f);
  }
}

template <typename TS, int M>
__global__ __launch_bounds__(256) void bwd_rows(BwdArgs a, int G) {
  constexpr int E = ChunkElems<TS>::E;
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t N = a.N;
  const int D = a.D, nch = D / E;
  const TS* __restrict__ x = reinterpret_cast<const TS*>(a.x);
  const TS* __restrict__ dy = reinterpret_cast<const TS*>(a.dy);
  u32x4_t dyr[M], xr[M];
  float acc[M][8];
  zero_acc<M>(acc);
  if (item < N) {
    const int64_t i = item;
    if (a.is_dense[i]) return;
    const int n = min(a.row_nnz[i], a.row_cap);
    const int32_t p0 = a.ws.row_ptr[i];
    load_row<TS, M>(dyr, dy + (size_t)i * D, nch, lane);
    const TS* ev = reinterpret_cast<const TS*>(a.ell_vals);
    for (int kb = 0; kb < n; kb += 64) {
      const int k = kb + lane;
      int c_l = 0;
      float h_l = 0.f, a_l = 0.f;
      if (k < n) {
        const size_t off = (size_t)k * N + i;
        c_l = a.ell_cols[off];
        h_l = Store<TS>::load(ev, off);
        a_l = a.ell_a[off];
      }
      const int nb = min(64, n - kb);
      for (int t = 0; t < nb; ++t)
        bwd_pair<TS, M>(a, nch, lane, dyr, xr, false, acc, readlane_i(c_l, t), readlane_f(h_l, t),
                        readlane_f(a_l, t), p0 + kb + t);
    }
    store_row<TS, M>(a.dx + (size_t)i * D, acc, nch, lane);
    return;
  }
  const int64_t k = item - N;
  const int o = (int)(k / G), g = (int)(k % G);
  if (o >= a.dense_cap || o >= *a.n_dense) return;
  const int64_t i = a.dense_rows[o];
  int32_t p = a.ws.row_ptr[i] + a.ws.grp_off[(size_t)o * G + g];
  load_row<TS, M>(dyr, dy + (size_t)i * D, nch, lane);
  load_row<TS, M>(xr, x + (size_t)i * D, nch, lane);
  const TS* hrow = reinterpret_cast<const TS*>(a.dense_h) + (size_t)o * a.F;
  const int c0 = g * kDenseChunk, c1 = min(a.F, c0 + kDenseChunk);
  for (int cb = c0; cb < c1; cb += 64) {
    const int c = cb + lane;
    const float h_l = c < c1 ? Store<TS>::load(hrow, c) : 0.f;
    uint64_t m = ballot(h_l > 0.f);
    while (m) {
      const int t = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      bwd_pair<TS, M>(a, nch, lane, dyr, xr, true, acc, cb + t, readlane_f(h_l, t), 0.f, p++);
    }
  }
  store_row<TS, M>(a.ws.part + ((size_t)o * G + g) * D, acc, nch, lane);
}

// --------------------------------------------------------------- column transpose

// Per block of RB rows: how many of its entries fall in each column. Counters
// are 16-bit halves of 32-bit LDS words (a column gets at most RB per block).
__global__ __launch_bounds__(256) void csc_hist(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ pair_col,
                                                int64_t N, int F, int32_t* __restrict__ blk_cnt) {
  extern __shared__ uint32_t cnt[];
  const int nw = (F + 1) / 2;
  for (int q = threadIdx.x; q < nw; q += blockDim.x) cnt[q] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * RB, r1 = min(N, r0 + RB);
  for (int32_t p = row_ptr[r0] + threadIdx.x; p < row_ptr[r1]; p += blockDim.x) {
    const int c = pair_col[p];
    atomicAdd(&cnt[c >> 1], 1u << ((c & 1) * 16));
  }
  __syncthreads();
  int32_t* out = blk_cnt + (size_t)blockIdx.x * F;
  for (int c = threadIdx.x; c < F; c += blockDim.x) out[c] = (cnt[c >> 1] >> ((c & 1) * 16)) & 0xffffu;
}

__global__ __launch_bounds__(256) void csc_coltotal(const int32_t* __restrict__ blk_cnt, int nrb, int F,
                                                    int32_t* __restrict__ col_ptr) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= F) return;
  int32_t s = 0;
  for (int b = 0; b < nrb; ++b) s += blk_cnt[(size_t)b * F + c];
  col_ptr[c] = s;
}

__global__ __launch_bounds__(1024) void csc_colscan(int32_t* col_ptr, int F) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int chunk = (F + 1023) / 1024;
  const int b = min(F, tid * chunk), en = min(F, b + chunk);
  int32_t s = 0;
  for (int c = b; c < en; ++c) s += col_ptr[c];
  part[tid] = s;
  __syncthreads();
  block_exclusive_scan(part, tid);
  int32_t run = part[tid] - s;
  for (int c = b; c < en; ++c) {
    const int32_t v = col_ptr[c];
    col_ptr[c] = run;
    run += v;
  }
  if (tid == 1023) col_ptr[F] = part[1023];
}

__global__ __launch_bounds__(256) void csc_offsets(int32_t* __restrict__ blk_cnt, const int32_t* __restrict__ col_ptr,
                                                   int nrb, int F) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= F) return;
  int32_t run = col_ptr[c];
  for (int b = 0; b < nrb; ++b) {
    const int32_t v = blk_cnt[(size_t)b * F + c];
    blk_cnt[(size_t)b * F + c] = run;
    run += v;
  }
}

// One wave per row block walks its rows in order; the entries of one row have
// distinct columns, so their ranks come from one atomic each without any
// ordering ambiguity, and each column receives its rows in ascending order.
__global__ __launch_bounds__(64) void csc_fill(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ pair_col,
                                               const int32_t* __restrict__ blk_off, int64_t N, int F,
                                               int32_t* __restrict__ csc_pair, int32_t* __restrict__ csc_row) {
  extern __shared__ uint32_t cnt[];
  const int nw = (F + 1) / 2;
  for (int q = threadIdx.x; q < nw; q += 64) cnt[q] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * RB, r1 = min(N, r0 + RB);
  const int32_t* off = blk_off + (size_t)blockIdx.x * F;
  for (int64_t r = r0; r < r1; ++r) {
    const int32_t e = row_ptr[r + 1];
    for (int32_t p = row_ptr[r] + threadIdx.x; p < e; p += 64) {
      const int c = pair_col[p];
      const int sh = (c & 1) * 16;
      const uint32_t old = atomicAdd(&cnt[c >> 1], 1u << sh);
      const int32_t pos = off[c] + (int32_t)((old >> sh) & 0xffffu);
      csc_pair[pos] = p;
      csc_row[pos] = (int32_t)r;
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------- weight gradients

template <typename TS, int MP>
__global__ __launch_bounds__(256) void bwd_dw(BwdArgs a, int parts) {
  constexpr int E = ChunkElems<TS>::E;
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)a.F * parts) return;
  const int c = (int)(item / parts), pr = (int)(item % parts);
  const int D = a.D, nch = D / E;
  const int ch0 = pr * MP * 64;
  const int nchp = min(MP * 64, nch - ch0);
  const TS* __restrict__ x = reinterpret_cast<const TS*>(a.x) + (size_t)ch0 * E;
  const TS* __restrict__ dy = reinterpret_cast<const TS*>(a.dy) + (size_t)ch0 * E;
  float accD[MP][8], accU[MP][8], accG[MP][8];
  zero_acc<MP>(accD);
  zero_acc<MP>(accU);
  zero_acc<MP>(accG);
  const int32_t q0 = a.ws.col_ptr[c], q1 = a.ws.col_ptr[c + 1];
  for (int32_t qb = q0; qb < q1; qb += 64) {
    const int32_t q = qb + lane;
    int i_l = 0;
    float4 cf = make_float4(0.f, 0.f, 0.f, 0.f);
    if (q < q1) {
      i_l = a.ws.csc_row[q];
      cf = a.ws.coef[a.ws.csc_pair[q]];
    }
    const int nb = min(64, q1 - qb);
    for (int t = 0; t < nb; ++t) {
      const int64_t i = readlane_i(i_l, t);
      const float z = readlane_f(cf.x, t), da = readlane_f(cf.y, t), dg = readlane_f(cf.z, t);
      u32x4_t r[MP];
      load_row<TS, MP>(r, dy + (size_t)i * D, nchp, lane);
      axpy_row<TS, MP>(accD, z, r);
      load_row<TS, MP>(r, x + (size_t)i * D, nchp, lane);
      axpy_row<TS, MP>(accU, da, r);
      axpy_row<TS, MP>(accG, dg, r);
    }
  }
  const size_t ro = (size_t)c * D + (size_t)ch0 * E;
  store_row<TS, MP>(a.dw_down + ro, accD, nchp, lane);
  store_row<TS, MP>(a.dw_up + ro, accU, nchp, lane);
  store_row<TS, MP>(a.dw_gate + ro, accG, nchp, lane);
}

template <typename TS>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
  constexpr int E = ChunkElems<TS>::E;
  const int nch = a.D / E;
  const int M = pick_m(nch);
  const int G = (a.F + kDenseChunk - 1) / kDenseChunk;
  const int nrb = (int)((a.N + RB - 1) / RB);
  int32_t* dense_nnz = a.ws.row_ptr + a.N + 1;  // [dense_cap] lives after row_ptr
  hipError_t err;

  if (a.dense_cap > 0) {
    TWELL_LAUNCH("dense_groups", dense_groups<TS>, dim3((a.dense_cap + 3) / 4), 256, 0, s, a, G, dense_nnz);
  }
  TWELL_LAUNCH("row_scan", row_scan, 1, 1024, 0, s, a, dense_nnz);
  const int64_t items = a.N + (int64_t)a.dense_cap * G;
  const dim3 grid((unsigned)((items + 3) / 4));
  switch (M) {
    case 1: TWELL_LAUNCH("bwd_rows", (bwd_rows<TS, 1>), grid, 256, 0, s, a, G); break;
    case 2: TWELL_LAUNCH("bwd_rows", (bwd_rows<TS, 2>), grid, 256, 0, s, a, G); break;
    case 4: TWELL_LAUNCH("bwd_rows", (bwd_rows<TS, 4>), grid, 256, 0, s, a, G); break;
    case 8: TWELL_LAUNCH("bwd_rows", (bwd_rows<TS, 8>), grid, 256, 0, s, a, G); break;
    case 16: TWELL_LAUNCH("bwd_rows", (bwd_rows<TS, 16>), grid, 256, 0, s, a, G); break;
    default: return hipErrorInvalidValue;
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_dense_reduce(a.ws.part, a.dense_rows, a.n_dense, a.dense_cap, G, a.D, a.dx, s)) != hipSuccess)
    return err;

  const size_t lds = (size_t)((a.F + 1) / 2) * 4;
  TWELL_LAUNCH("csc_hist", csc_hist, dim3(nrb), 256, lds, s, a.ws.row_ptr, a.ws.pair_col, a.N, a.F, a.ws.blk_cnt);
  TWELL_LAUNCH("csc_coltotal", csc_coltotal, dim3((a.F + 255) / 256), 256, 0, s, a.ws.blk_cnt, nrb, a.F, a.ws.col_ptr);
  TWELL_LAUNCH("csc_colscan", csc_colscan, 1, 1024, 0, s, a.ws.col_ptr, a.F);
  TWELL_LAUNCH("csc_offsets", csc_offsets, dim3((a.F + 255) / 256), 256, 0, s, a.ws.blk_cnt, a.ws.col_ptr, nrb, a.F);
  TWELL_LAUNCH("csc_fill", csc_fill, dim3(nrb), 64, lds, s, a.ws.row_ptr, a.ws.pair_col, a.ws.blk_cnt, a.N, a.F, a.ws.csc_pair,
                                      a.ws.csc_row);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  const int MP = M < 4 ? M : 4;
  const int parts = (nch + MP * 64 - 1) / (MP * 64);
  const dim3 gdw((unsigned)(((int64_t)a.F * parts + 3) / 4));
  switch (MP) {
    case 1: TWELL_LAUNCH("bwd_dw", (bwd_dw<TS, 1>), gdw, 256, 0, s, a, parts); break;
    case 2: TWELL_LAUNCH("bwd_dw", (bwd_dw<TS, 2>), gdw, 256, 0, s, a, parts); break;
    case 4: TWELL_LAUNCH("bwd_dw", (bwd_dw<TS, 4>), gdw, 256, 0, s, a, parts); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_bwd(const BwdArgs& a, hipStream_t s) {
  return a.is_bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace twell
