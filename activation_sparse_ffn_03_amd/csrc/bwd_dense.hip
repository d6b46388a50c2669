// Dense-backup rows of the backward on the matrix cores.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// rows that do not fit the training format's ELL part go to a dense backup;
// fourth paragraph: such rows can hold many times the mean number of active
// units. For the loss of the backward's header (bwd.hip) their share is, with
// the dense rows gathered (R of them) and M their active mask:
//
//   DZ = DY_R . W_down^T,  A = X_R . W_up^T          (R x d_ff, at every unit)
//   DA = M * DZ * H,  DG = M * (DZ * A + lambda)
//   dx_R = DA . W_up + DG . W_gate                    (R x d_model)
//
// three skinny products that stream each weight once per 64 rows (the same
// MFMA forms as the forward's overflow rows, skinny_mfma.h):
//   dense_bwd_nt     a wave per 16 columns: DZ and A over all of d_model
//                    (fp32, [dense_cap][F] each); it needs only the dense-row
//                    list, so it can start before the row offsets exist
//   dense_records    wave per (row, 512-column chunk): the records of the
//                    active units (column and (z, da, dg)) in CSR order, for
//                    the weight gradients, and DA, DG as bf16 high / low parts
//   dense_dx_mfma    DA . W_up + DG . W_gate in d_ff chunks; dense_reduce
//                    adds the chunks into dx (bwd_dx leaves these rows alone)
#include "skinny_mfma.h"
#include "twell_host.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

using namespace skinny;

__global__ __launch_bounds__(64 * kSkinnyWaves) void dense_bwd_nt(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const uint16_t* wd = reinterpret_cast<const uint16_t*>(a.w_down);
  const uint16_t* wu = reinterpret_cast<const uint16_t*>(a.w_up);
  int c0;
  const uint16_t* rd[kSkinnyUW];
  const uint16_t* ru[kSkinnyUW];
  if (!skinny_columns<kSkinnyUW>(wd, a.D, a.F, c0, rd)) return;
  (void)skinny_columns<kSkinnyUW>(wu, a.D, a.F, c0, ru);
  const int n = min(*a.n_dense, a.dense_cap);
  const size_t plane = (size_t)a.dense_cap * a.F;
  for (int m0 = blockIdx.z * kRowsPerPass; m0 < n; m0 += gridDim.z * kRowsPerPass) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      f32x4_t acc[NF][kSkinnyUW];
      skinny_nt<kSkinnyUW, kSkinnyB>(reinterpret_cast<const uint16_t*>(which == 0 ? a.dy : a.x), a.dense_rows, n, m0,
                                     which == 0 ? rd : ru, a.D, acc);
      float* out = a.ws.dza + which * plane;
      // 16x16 MFMA result: lane l holds rows 4*(l>>4)+r of column l&15
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = m0 + 16 * f + 4 * (lane >> 4) + r;
#pragma unroll
          for (int u = 0; u < kSkinnyUW; ++u) {
            const int col = c0 + 16 * u + (lane & 15);
            if (o < n && col < a.F) out[(size_t)o * a.F + col] = acc[f][u][r];
          }
        }
    }
  }
}

// Work item (dense row o, chunk g of kDenseChunk columns), 64 columns at a
// time; a capped grid of waves strides over the items of the rows that really
// went dense.
__device__ __forceinline__ void dense_record_item(const BwdArgs& a, int G, int Fz, int o, int g) {
  const int lane = threadIdx.x & 63;
  const int F = a.F;
  const int64_t i = a.dense_rows[o];
  const uint16_t* hrow = reinterpret_cast<const uint16_t*>(a.dense_h) + (size_t)o * F;
  const float* dzr = a.ws.dza + (size_t)o * F;
  const float* ar = a.ws.dza + (size_t)a.dense_cap * F + (size_t)o * F;
  const size_t zp = (size_t)a.dense_cap * Fz;
  uint16_t* dah = a.ws.dadg + (size_t)o * Fz;
  int32_t p = a.ws.row_ptr[i] + a.ws.grp_off[(size_t)o * G + g];
  const int c0 = g * kDenseChunk, c1 = min(F, c0 + kDenseChunk);
  for (int cb = c0; cb < c1; cb += 64) {
    const int c = cb + lane;
    const bool in = c < c1;
    const float h = in ? bf16_to_f32(hrow[c]) : 0.f;
    const bool act = h > 0.f;
    const uint64_t m = ballot(act);
    float da = 0.f, dg = 0.f;
    if (act) {
      const float dz = dzr[c], av = ar[c];
      da = dz * h;
      dg = fmaf(dz, av, a.lam);
      const int32_t q = p + (int32_t)lanemask_lt_popc(m, lane);
      a.ws.pair_col[q] = c;
      a.ws.coef[q] = make_float4(h * av, da, dg, 0.f);
    }
    if (in) {
      const uint16_t dah_hi = f32_to_bf16(da), dg_hi = f32_to_bf16(dg);
      dah[c] = dah_hi;
      dah[zp + c] = f32_to_bf16(da - bf16_to_f32(dah_hi));
      dah[2 * zp + c] = dg_hi;
      dah[3 * zp + c] = f32_to_bf16(dg - bf16_to_f32(dg_hi));
    }
    p += __popcll(m);
  }
}

constexpr int kRecordsGrid = 1024;

__global__ __launch_bounds__(256) void dense_records(BwdArgs a, int G, int Fz) {
  const int64_t items = (int64_t)min(*a.n_dense, a.dense_cap) * G;
  for (int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); k < items; k += (int64_t)gridDim.x * 4)
    dense_record_item(a, G, Fz, (int)(k / G), (int)(k % G));
}

__global__ __launch_bounds__(64 * kDownWaves) void dense_dx_mfma(BwdArgs a, int G, int Fz) {
  const size_t zp = (size_t)a.dense_cap * Fz;
  NnOperands<2> p;
  p.hi[0] = a.ws.dadg;
  p.lo[0] = a.ws.dadg + zp;
  p.w[0] = reinterpret_cast<const uint16_t*>(a.w_up);
  p.hi[1] = a.ws.dadg + 2 * zp;
  p.lo[1] = a.ws.dadg + 3 * zp;
  p.w[1] = reinterpret_cast<const uint16_t*>(a.w_gate);
  skinny_nn<2>(p, min(*a.n_dense, a.dense_cap), a.D, a.F, Fz, G, a.ws.dxpart);
}

}  // namespace

bool bwd_dense_mfma_applies(const BwdArgs& a) {
  return a.is_bf16 && a.D % kDownCols == 0 && a.D % 32 == 0 && a.dense_cap > 0 && a.ws.dza != nullptr;
}

hipError_t launch_bwd_dense_nt(const BwdArgs& a, hipStream_t s) {
  TWELL_LAUNCH("dense_bwd_nt", dense_bwd_nt, dim3(skinny_blocks(a.F, kSkinnyUW), 1, kPassSplit), 64 * kSkinnyWaves, 0,
               s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dense_records(const BwdArgs& a, hipStream_t s) {
  const int G = (a.F + kDenseChunk - 1) / kDenseChunk;
  const int64_t want = ((int64_t)a.dense_cap * G + 3) / 4;
  TWELL_LAUNCH("dense_records", dense_records, dim3((unsigned)(want < kRecordsGrid ? want : kRecordsGrid)), 256, 0,
               s, a, G, dense_z_stride(a.F));
  return hipGetLastError();
}

hipError_t launch_bwd_dense_dx(const BwdArgs& a, hipStream_t s) {
  const int G = (a.F + kDenseChunk - 1) / kDenseChunk;
  TWELL_LAUNCH("dense_dx_mfma", dense_dx_mfma, skinny_nn_grid(a.D, G), 64 * kDownWaves, 0, s, a, G,
               dense_z_stride(a.F));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_dense_reduce(a.ws.dxpart, a.dense_rows, a.n_dense, a.dense_cap, G, a.D, a.dx, s);
}

}  // namespace twell
