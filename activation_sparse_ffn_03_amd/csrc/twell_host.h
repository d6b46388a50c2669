// Host-only shape validation and buffer / workspace size arithmetic.
// Plain C++17 with no HIP dependency, so it can also be built and tested on
// its own (and under sanitizers) without a GPU toolchain.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/twell.h"

namespace twell {

constexpr size_t kWsAlign = 256;
// TwELL tiles per column group of the blocked up projection (up_blocked.hip).
constexpr int kUpGroupTiles = 4;

struct Shape {
  int64_t N;
  int D, F, tile_n, slots, row_cap, ovf_cap, dense_cap;
  int n_tiles;
  int esz;     // bytes per stored element (2 bf16, 4 fp32)
  int G;       // column chunks of a dense row
  int nrb;     // row blocks of the column transpose
  int64_t nnz_max;
};

// Offsets (bytes from the workspace base) of every backward workspace array.
struct BwdLayout {
  size_t row_ptr, dense_pos, pair_col, coef, csc_pair, csc_row, col_ptr, blk_cnt, grp_off, egrp;
  size_t dza, dadg, dxpart;  // 0 bytes (offset == next) unless bwd_dense_mfma(s)
  size_t total;
};

// Validate dims/dtype; on failure returns the status and sets *why.
twell_status check_shape(const twell_dims* dims, int dtype, Shape* out, std::string* why);
void compute_sizes(const Shape& s, twell_sizes* out);
BwdLayout bwd_layout(const Shape& s);
// The backward's dense-backup rows take the skinny MFMA products (bf16,
// d_model a multiple of 128, a dense capacity).
inline bool bwd_dense_mfma(const Shape& s) { return s.esz == 2 && s.D % 128 == 0 && s.dense_cap > 0; }
// Passes over d_model of the up projection. W_up's columns are dealt to the 8
// XCDs (F/8 rows of W_up each); when such a block is larger than the XCD's
// 4 MB L2, d_model is cut into up_passes power-of-two ranges (each a whole
// number of 16-byte loads of a 64-lane wave) so that one range's block fits,
// and the partial dot products of the ranges go through the workspace.
int up_passes(const Shape& s);
// Forward workspace, in order: per-row entry totals ([N] int32), the
// row-major (column, z) list ([N][n_t*S] x 8 bytes), and only when
// up_passes > 1 the passes' partial dot products ([up_passes][N][n_t*S] fp32)
// and the slot of every list entry ([N][n_t*S] int32); then the dense-row
// partials; then, for bf16 storage, the overflow rows' z = h*a as bf16 high
// and low parts ([2][ovf_cap][dense_z_stride(F)] uint16); then the list
// position of each kUpGroupTiles-tile group's first entry
// ([ceil(n_t / kUpGroupTiles)][N] int32); then the down projection's order of
// 4-row blocks ([ceil(N/4)] int32), each block's class code ([ceil(N/4)]
// int32) and the per-workgroup class counts ([ceil(N/256)][16] int32).
struct FwdLayout {
  size_t offs, zlist, upart, uslot, part, zov, gbase, rb_order, rb_code, rb_hist, total;
};
// Row stride (elements) of the overflow rows' z: d_ff rounded up to 32, so
// every 32-column block of a row lies inside it and rows stay 64-byte aligned.
inline int dense_z_stride(int F) { return (F + 31) / 32 * 32; }
FwdLayout fwd_layout(const Shape& s);
size_t fwd_ws_bytes(const Shape& s);

// Pointer checks: null (when bytes > 0) or not 16-byte aligned.
bool bad_ptr(const void* p, size_t bytes);

}  // namespace twell
