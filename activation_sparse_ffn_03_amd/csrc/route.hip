// Stage 3a: hybrid row router for training.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// for training a hybrid format routes rows dynamically either into a compact
// ELL matrix (sparse rows) or into a dense backup for overflows; fourth
// paragraph: the maximum nonzeros per row can far exceed the mean.
//
// Readings: row_nnz = sum of the row's true tile counts; a row is dense iff
// row_nnz > K or it overflowed a TwELL tile; ELL positions follow ascending
// global column (tile by tile, slot by slot); dense rows are listed in
// ascending order.
//
// Kernels
//   route_rows     wave per row, 16 rows per workgroup (their TwELL slot
//                  loads share cache lines), each XCD a contiguous run of
//                  row blocks (a 128-byte line of a [.][N] array spans 64
//                  or 32 rows; split over XCDs, every L2 fetched it):
//                  row_nnz, is_dense, and the ELL entries of ELL rows (vals,
//                  global cols, saved a).
//   launch_compact ascending dense-row list + capacity status.
//   route_dense_h  dense activation rows, rebuilt from TwELL slots or copied
//                  from the overflow rows: for bf16 rows up to 32768 columns
//                  a workgroup per row building it in LDS, else a thread per
//                  (dense row, column).
#include "twell_device.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

// Maximum of v over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// Exclusive prefix sum of v over the 64 lanes of a wave.
__device__ __forceinline__ int wave_excl_scan(int v) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if ((threadIdx.x & 63) >= off) x += y;
  }
  return x - v;
}

constexpr int kRouteBatch = 4;

// One wave per row. Pass 1: row_nnz and the dense decision from the tile
// counts (64 tiles per load). Pass 2 (ELL rows): lane l takes tile jb+l of a
// 64-tile batch; iteration s copies slot s of every lane's tile to ELL
// position (start of the tile + s), so all loads of one iteration are in
// flight together.
template <typename TS>
__global__ __launch_bounds__(1024) void route_rows(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = xcd_run_block(blockIdx.x, gridDim.x) * 16 + (threadIdx.x >> 6);
  if (i >= a.N) return;
  const int64_t N = a.N;
  int nnz = 0;
  for (int jb = 0; jb < a.n_tiles; jb += 64) {
    const int jl = jb + lane;
    nnz += (int)wave_sum_dpp(jl < a.n_tiles ? (float)a.counts[(size_t)jl * N + i] : 0.f);  // exact: < 2^24
  }
  const bool dense = nnz > a.row_cap || a.ovf_flag[i] != 0;
  if (lane == 0) {
    a.row_nnz[i] = nnz;
    a.is_dense[i] = dense ? 1 : 0;
  }
  if (dense) return;
  const TS* vals = reinterpret_cast<const TS*>(a.vals);
  TS* ev = reinterpret_cast<TS*>(a.ell_vals);
  int base = 0;
  for (int jb = 0; jb < a.n_tiles; jb += 64) {
    const int jl = jb + lane;
    const int cnt = jl < a.n_tiles ? (int)a.counts[(size_t)jl * N + i] : 0;  // <= S: the row did not overflow
    const int start = base + wave_excl_scan(cnt);
    const int maxc = wave_max_i(cnt);
    // kRouteBatch slots at a time: every load of the batch is issued before
    // its stores, so a lane has 3 * kRouteBatch loads in flight
    for (int sl0 = 0; sl0 < maxc; sl0 += kRouteBatch) {
      TS v[kRouteBatch];
      uint16_t c[kRouteBatch];
      float av[kRouteBatch];
#pragma unroll
      for (int u = 0; u < kRouteBatch; ++u) {
        const int sl = sl0 + u;
        if (sl < cnt) {
          const size_t src = ((size_t)jl * a.slots + sl) * N + i;
          v[u] = vals[src];
          c[u] = a.cols[src];
          av[u] = a.a_save[src];
        }
      }
#pragma unroll
      for (int u = 0; u < kRouteBatch; ++u) {
        const int sl = sl0 + u;
        if (sl < cnt) {
          const size_t dst = (size_t)(start + sl) * N + i;
          ev[dst] = v[u];
          a.ell_cols[dst] = jl * a.tile_n + c[u];
          a.ell_a[dst] = av[u];
        }
      }
    }
    base = __builtin_amdgcn_readlane(start + cnt, 63);  // start already includes base
  }
}

// Dense row o, column c: from the overflow row copy when the row overflowed
// (located by binary search in the ascending overflow list), else from the
// TwELL slots of its tile.
template <typename TS>
__global__ __launch_bounds__(256) void route_dense_h(RouteArgs a) {
  const int cb = (a.F + 255) / 256;
  const int o = blockIdx.x / cb;
  if (o >= a.dense_cap || o >= *a.n_dense) return;
  const int c = (blockIdx.x % cb) * 256 + threadIdx.x;
  if (c >= a.F) return;
  const int64_t N = a.N;
  const int64_t i = a.dense_rows[o];
  TS* out = reinterpret_cast<TS*>(a.dense_h) + (size_t)o * a.F;
  const TS* vals = reinterpret_cast<const TS*>(a.vals);
  TS h = TS(0);
  if (a.ovf_flag[i]) {
    const int n = min(*a.n_ovf, a.ovf_cap);
    int lo = 0, hi = n;  // first position with ovf_rows[pos] >= i
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.ovf_rows[mid] < i) lo = mid + 1; else hi = mid;
    }
    if (lo < n && a.ovf_rows[lo] == i) h = reinterpret_cast<const TS*>(a.ovf_h)[(size_t)lo * a.F + c];
  } else {
    const int j = c / a.tile_n, off = c - j * a.tile_n;
    const int cnt = min((int)a.counts[(size_t)j * N + i], a.slots);
    for (int s = 0; s < cnt; ++s) {
      const size_t src = ((size_t)j * a.slots + s) * N + i;
      if (a.cols[src] == off) h = vals[src];
    }
  }
  out[c] = h;
}

// The same, a workgroup per dense row for bf16 rows up to 32768 columns: the
// row is built in LDS (zeroed, then every TwELL slot of the row's tiles
// scattered to its column, at most one slot per column) and written out
// coalesced, so each slot is read once instead of once per column of its
// tile; an overflowed row is copied from its overflow row.
constexpr int kDenseHLdsCols = 32768;
__global__ __launch_bounds__(1024) void route_dense_h_lds(RouteArgs a) {
  extern __shared__ uint16_t hrow[];  // [F]
  const int o = blockIdx.x;
  if (o >= a.dense_cap || o >= *a.n_dense) return;  // uniform: no barrier skipped within a workgroup
  const int64_t N = a.N;
  const int F = a.F, tid = threadIdx.x;
  const int64_t i = a.dense_rows[o];
  uint16_t* out = reinterpret_cast<uint16_t*>(a.dense_h) + (size_t)o * F;
  if (a.ovf_flag[i]) {
    const int n = min(*a.n_ovf, a.ovf_cap);
    int lo = 0, hi = n;  // first position with ovf_rows[pos] >= i
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.ovf_rows[mid] < i) lo = mid + 1; else hi = mid;
    }
    const bool found = lo < n && a.ovf_rows[lo] == i;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(a.ovf_h) + (size_t)(found ? lo : 0) * F;
    for (int c = tid; c < F; c += 1024) out[c] = found ? src[c] : uint16_t(0);
    return;
  }
  for (int c = tid; c < F; c += 1024) hrow[c] = 0;
  __syncthreads();
  const uint16_t* vals = reinterpret_cast<const uint16_t*>(a.vals);
  const int items = a.n_tiles * a.slots;  // (tile, slot) pairs of the row
  for (int q = tid; q < items; q += 1024) {
    const int j = q / a.slots, sl = q - j * a.slots;
    if (sl < min((int)a.counts[(size_t)j * N + i], a.slots)) {
      const size_t src = ((size_t)j * a.slots + sl) * N + i;
      const int c = j * a.tile_n + a.cols[src];
      if (c < F) hrow[c] = vals[src];
    }
  }
  __syncthreads();
  for (int c = tid; c < F; c += 1024) out[c] = hrow[c];
}

template <typename TS>
hipError_t launch_t(const RouteArgs& a, hipStream_t s) {
  TWELL_LAUNCH("route_rows", route_rows<TS>, dim3((unsigned)((a.N + 15) / 16)), 1024, 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_compact(a.is_dense, a.N, a.dense_rows, a.dense_cap, a.n_dense, a.status, 2u /*TWELL_DEV_DENSE_CAPACITY*/, s);
  if (err != hipSuccess || a.dense_cap == 0) return err;
  if (sizeof(TS) == 2 && a.F <= kDenseHLdsCols)
    TWELL_LAUNCH("route_dense_h", route_dense_h_lds, dim3((unsigned)a.dense_cap), 1024, (size_t)a.F * 2, s, a);
  else
    TWELL_LAUNCH("route_dense_h", route_dense_h<TS>, dim3((unsigned)(((a.F + 255) / 256) * (int64_t)a.dense_cap)), 256,
                 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  return a.is_bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace twell
