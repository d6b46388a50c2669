// dz of the ELL rows of the backward with weight-row reuse through LDS.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// training runs on the hybrid format, whose compact ELL part holds the rows
// that fit it. For the loss of the backward's header (bwd.hip), every active
// entry (i, c) of an ELL row needs dz = dy_i . W_down[c], a sampled product of
// the same shape as the forward's up projection (x -> dy, W_up -> W_down), so
// it runs on the same blocked kernel (blocked_sddmm.h): 512 tokens x 512
// columns per workgroup, dy and W_down staged through LDS.
//
// ell_groups, a small pass before, finds for every ELL row the ELL position
// of its first entry in each 512-column group (its columns ascend). The
// blocked kernel then writes each entry's record at row_ptr[i] + its ELL
// position, as bwd_dz_ell does: column and (z, da, dg) = (h*a, dz*h,
// dz*a + lambda).
#include "blocked_sddmm.h"
#include "ell_groups.h"
#include "twell_host.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int kGroupCols = blk::kGroupCols;
constexpr int kMaxGroups = 64;  // d_ff up to 32768

// Wave per row, 4 rows per workgroup, each XCD a contiguous run of rows (the
// [.][N] arrays' lines stay in one L2).
__global__ __launch_bounds__(256) void ell_groups(BwdArgs a, int n_groups) {
  const int64_t i = xcd_run_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (i < a.N) ell_groups_row(a, n_groups, i);
}

// The backward's pattern: the ELL entries of the ELL rows; records at
// row_ptr[i] + ELL position.
struct DzPolicy {
  BwdArgs a;
  static constexpr int kSub = 1;
  __device__ const uint16_t* rows_a() const { return reinterpret_cast<const uint16_t*>(a.dy); }
  __device__ const uint16_t* rows_b() const { return reinterpret_cast<const uint16_t*>(a.w_down); }
  __device__ int64_t n() const { return a.N; }
  __device__ int d() const { return a.D; }
  __device__ int f() const { return a.F; }
  __device__ int c0(int g) const { return g * kGroupCols; }
  __device__ bool own(int64_t i) const { return !a.is_dense[i]; }
  __device__ int count(int64_t i, int g, int) const {
    return a.ws.egrp[(size_t)(g + 1) * a.N + i] - a.ws.egrp[(size_t)g * a.N + i];
  }
  __device__ void entry(int64_t i, int g, int, int k, uint32_t& cg, uint32_t& key, uint32_t& hb) const {
    const int kk = a.ws.egrp[(size_t)g * a.N + i] + k;
    const size_t off = (size_t)kk * a.N + i;
    cg = (uint32_t)(a.ell_cols[off] - c0(g));
    key = (uint32_t)kk;
    hb = (uint32_t)reinterpret_cast<const uint16_t*>(a.ell_vals)[off] << 16;
  }
  __device__ int base(int64_t i, int g) const { return a.ws.row_ptr[i] + a.ws.egrp[(size_t)g * a.N + i]; }
  __device__ void store(int64_t i, int g, uint32_t cg, uint32_t key, float h, int pos, float dz) const {
    const float av = a.ell_a[(size_t)key * a.N + i];
    a.ws.pair_col[pos] = c0(g) + (int)cg;
    a.ws.coef[pos] = make_float4(h * av, dz * h, fmaf(dz, av, a.lam), 0.f);
  }
};

using DzBlk = blk::Default;

__global__ __launch_bounds__(DzBlk::NT, 1) void bwd_dz_blocked(BwdArgs a, int n_groups, int64_t n_tblocks) {
  blk::sddmm_block<DzBlk>(DzPolicy{a}, n_groups, n_tblocks);
}

}  // namespace

int dz_groups(int F) { return (F + kGroupCols - 1) / kGroupCols; }

bool dz_blocked_applies(const BwdArgs& a) {
  const int64_t pairs = ((a.N + DzBlk::T - 1) / DzBlk::T) * dz_groups(a.F);
  return a.is_bf16 && a.N > 64 && a.D % 32 == 0 && a.row_cap < 1024 && dz_groups(a.F) <= kMaxGroups &&
         a.ws.egrp != nullptr && pairs >= blk::kCus;
}

hipError_t launch_dz_blocked(const BwdArgs& a, hipStream_t s, bool groups_done) {
  if (!dz_blocked_applies(a)) return hipErrorInvalidValue;
  const int n_groups = dz_groups(a.F);
  if (!groups_done) {
    TWELL_LAUNCH("ell_groups", ell_groups, dim3((unsigned)((a.N + 3) / 4)), 256, 0, s, a, n_groups);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int64_t ntb = (a.N + DzBlk::T - 1) / DzBlk::T;
  TWELL_LAUNCH("bwd_dz_blocked", bwd_dz_blocked, dim3((unsigned)blk::grid_blocks(ntb, n_groups)), DzBlk::NT, 0, s, a,
               n_groups, ntb);
  return hipGetLastError();
}

}  // namespace twell
