// Stage 2: fused up + down projection on the TwELL activation.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// the inference kernel reads the activations in TwELL and performs the up and
// down projections at once, without writing the intermediate hidden state to
// global memory.
//
// Design (wave-stationary token): one wave owns one token. x_i (bf16 or fp32)
// and the fp32 accumulator of y_i live in registers for the whole pass. The
// wave walks the TwELL tiles in ascending order (so all waves on a chip sweep
// the weight rows in the same order, which keeps the rows of the current tiles
// hot in L2) and, for every packed entry (c, h):
//   a = x_i . W_up^T[c]   (coalesced row gather + bf16 dot2 + wave reduction)
//   z = h * a             (fp32, never stored)
//   y_i += z * W_down[c]  (coalesced row gather + fp32 FMA)
// Overflow rows (a tile count above S) are skipped here: their dense
// activation row is split into column chunks of kDenseChunk, each chunk is a
// work item of its own wave writing a partial y row, and dense_reduce adds the
// partials in chunk order (deterministic, no atomics).
#include "row_ops.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

template <typename TS, int M>
__device__ __forceinline__ void do_pair(const TS* __restrict__ w_up, const TS* __restrict__ w_down, int D, int F,
                                        int nch, int lane, const u32x4_t (&xr)[M], float (&acc)[M][8], int c,
                                        float h, float* a_out) {
  if ((unsigned)c >= (unsigned)F) return;  // defensive: never gather outside the weights
  u32x4_t wr[M];
  load_row<TS, M>(wr, w_up + (size_t)c * D, nch, lane);
  const float a = wave_sum(dot_rows<TS, M>(xr, wr));
  if (a_out != nullptr && lane == 0) *a_out = a;
  const float z = h * a;
  load_row<TS, M>(wr, w_down + (size_t)c * D, nch, lane);
  axpy_row<TS, M>(acc, z, wr);
}

template <typename TS, int M>
__global__ __launch_bounds__(256) void ffn_fwd_kernel(FwdArgs a, int G) {
  constexpr int E = ChunkElems<TS>::E;
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t N = a.N;
  const int D = a.D, nch = D / E;
  const TS* __restrict__ x = reinterpret_cast<const TS*>(a.x);
  const TS* __restrict__ w_up = reinterpret_cast<const TS*>(a.w_up);
  const TS* __restrict__ w_down = reinterpret_cast<const TS*>(a.w_down);
  u32x4_t xr[M];
  float acc[M][8];
  zero_acc<M>(acc);

  if (item < N) {
    const int64_t i = item;
    const uint16_t* __restrict__ counts = a.counts;
    for (int jb = 0; jb < a.n_tiles; jb += 64) {
      const int j = jb + lane;
      const int c = j < a.n_tiles ? counts[(size_t)j * N + i] : 0;
      if (ballot(c > a.slots)) return;  // overflow row: handled by the dense chunks
    }
    load_row<TS, M>(xr, x + (size_t)i * D, nch, lane);
    const TS* __restrict__ vals = reinterpret_cast<const TS*>(a.vals);
    for (int jb = 0; jb < a.n_tiles; jb += 64) {
      const int jl = jb + lane;
      const int cnt_l = jl < a.n_tiles ? counts[(size_t)jl * N + i] : 0;
      uint64_t nz = ballot(cnt_l > 0);
      while (nz) {
        const int t = __ffsll((unsigned long long)nz) - 1;
        nz &= nz - 1;
        const int j = jb + t;
        const int cnt = readlane_i(cnt_l, t);
        const size_t base = (size_t)j * a.slots * N + i;
        // slots are read 64 at a time (S may reach T_n = 128)
        for (int sb = 0; sb < cnt; sb += 64) {
          int col_l = 0;
          float h_l = 0.f;
          if (sb + lane < cnt) {
            col_l = a.cols[base + (size_t)(sb + lane) * N];
            h_l = Store<TS>::load(vals, base + (size_t)(sb + lane) * N);
          }
          const int nb = min(64, cnt - sb);
          for (int s = 0; s < nb; ++s) {
            const int c = j * a.tile_n + readlane_i(col_l, s);
            const float h = readlane_f(h_l, s);
            float* a_out = a.a_save ? a.a_save + base + (size_t)(sb + s) * N : nullptr;
            do_pair<TS, M>(w_up, w_down, D, a.F, nch, lane, xr, acc, c, h, a_out);
          }
        }
      }
    }
    store_row<TS, M>(a.y + (size_t)i * D, acc, nch, lane);
    return;
  }

  // dense chunk (overflow row o, columns [g*kDenseChunk, ...))
  const int64_t k = item - N;
  const int o = (int)(k / G), g = (int)(k % G);
  if (o >= a.ovf_cap || o >= *a.n_ovf) return;
  const int64_t i = a.ovf_rows[o];
  load_row<TS, M>(xr, x + (size_t)i * D, nch, lane);
  const TS* __restrict__ hrow = reinterpret_cast<const TS*>(a.ovf_h) + (size_t)o * a.F;
  const int c0 = g * kDenseChunk, c1 = min(a.F, c0 + kDenseChunk);
  for (int cb = c0; cb < c1; cb += 64) {
    const int c = cb + lane;
    const float h_l = c < c1 ? Store<TS>::load(hrow, c) : 0.f;
    uint64_t m = ballot(h_l > 0.f);
    while (m) {
      const int t = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      do_pair<TS, M>(w_up, w_down, D, a.F, nch, lane, xr, acc, cb + t, readlane_f(h_l, t), nullptr);
    }
  }
  store_row<TS, M>(a.part + ((size_t)o * G + g) * D, acc, nch, lane);
}

// y[ovf_rows[o]] = sum_g part[o][g]  (fixed chunk order)
__global__ __launch_bounds__(256) void dense_reduce(const float* __restrict__ part, const int32_t* __restrict__ rows,
                                                    const int32_t* __restrict__ n_rows, int cap, int G, int D,
                                                    float* __restrict__ out) {
  const int db = (D + 255) / 256;
  const int o = blockIdx.x / db;
  if (o >= cap || o >= *n_rows) return;
  const int d = (blockIdx.x % db) * 256 + threadIdx.x;
  if (d >= D) return;
  const float* p = part + (size_t)o * G * D + d;
  float s = 0.f;
  for (int g = 0; g < G; ++g) s += p[(size_t)g * D];
  out[(size_t)rows[o] * D + d] = s;
}

template <typename TS>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  constexpr int E = ChunkElems<TS>::E;
  const int M = pick_m(a.D / E);
  const int G = (a.F + kDenseChunk - 1) / kDenseChunk;
  const int64_t items = a.N + (int64_t)a.ovf_cap * G;
  const dim3 grid((unsigned)((items + 3) / 4));
  if (items > 0) {
    switch (M) {
      case 1: TWELL_LAUNCH("ffn_fwd_kernel", (ffn_fwd_kernel<TS, 1>), grid, 256, 0, s, a, G); break;
      case 2: TWELL_LAUNCH("ffn_fwd_kernel", (ffn_fwd_kernel<TS, 2>), grid, 256, 0, s, a, G); break;
      case 4: TWELL_LAUNCH("ffn_fwd_kernel", (ffn_fwd_kernel<TS, 4>), grid, 256, 0, s, a, G); break;
      case 8: TWELL_LAUNCH("ffn_fwd_kernel", (ffn_fwd_kernel<TS, 8>), grid, 256, 0, s, a, G); break;
      case 16: TWELL_LAUNCH("ffn_fwd_kernel", (ffn_fwd_kernel<TS, 16>), grid, 256, 0, s, a, G); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.ovf_cap == 0) return err;
  return launch_dense_reduce(a.part, a.ovf_rows, a.n_ovf, a.ovf_cap, G, a.D, a.y, s);
}

}  // namespace

hipError_t launch_dense_reduce(const float* part, const int32_t* rows, const int32_t* n_rows, int cap, int G,
                               int D, float* out, hipStream_t s) {
  if (cap == 0) return hipSuccess;
  TWELL_LAUNCH("dense_reduce", dense_reduce, dim3((unsigned)(((D + 255) / 256) * (int64_t)cap)), 256, 0, s, part, rows, n_rows, cap, G, D, out);
  return hipGetLastError();
}

hipError_t launch_ffn_fwd(const FwdArgs& a, hipStream_t s) {
  return a.is_bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace twell
