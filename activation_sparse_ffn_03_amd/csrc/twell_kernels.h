// Internal launch interface between the C ABI (twell_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace twell {

// Width of the column chunks that dense (overflow / backup) rows are split
// into so that one long row is spread over many waves.
constexpr int kDenseChunk = 512;
// Rows per block of the deterministic column transpose (one bit of a 32-bit
// mask each).
constexpr int kTransposeRows = 32;

// Ascending list of the rows whose flag is set (single-workgroup
// deterministic scan). Writes rows[0:min(count,cap)], *n_out = count and
// *status = count > cap ? bit : 0.
hipError_t launch_compact(const uint8_t* flag, int64_t N, int32_t* rows, int cap, int32_t* n_out,
                          uint32_t* status, uint32_t bit, hipStream_t s);

struct GateArgs {
  int64_t N;
  int D, F, tile_n, slots, n_tiles;
  int is_bf16;
  const void* x;       // [N][D]
  const void* w;       // [F][D]
  const float* g_in;   // pack_preact: [N][F] fp32 pre-activation (else null)
  const float* t;      // [N]
  void* vals;
  uint16_t* cols;
  uint16_t* counts;
  uint8_t* ovf_flag;
  int32_t* ovf_rows;
  void* ovf_h;
  int32_t* n_ovf;
  uint32_t* status;
  int ovf_cap;
  float* g_dump;       // optional
  float* g_ws;         // optional [N][F] fp32 buffer: enables the small-batch gate (N <= 64)
  int fp8;                // x and w hold E4M3 codes with per-row scales
  const float* x_scale;   // fp8: [N]
  const float* w_scale;   // fp8: [F]
};

hipError_t launch_gate_pack(const GateArgs& a, hipStream_t s);
// The same launches, with the overflow steps enqueued on the side stream
// when `fork` is set: the overflow rows' dense activations, and also the
// flags and the overflow list unless list_on_main (the pack always stays on
// `s`). *ovf_stream is the stream that ends the overflow branch: `s` when
// nothing was forked (no overflow steps, or fork unset), else the side stream,
// which the caller must join back into `s`.
hipError_t launch_gate_pack_split(const GateArgs& a, hipStream_t s, bool fork, hipStream_t* ovf_stream,
                                  bool list_on_main);
// True when the overflow rows' gate rows take the 128x128 register-staged
// GEMM (bf16, d_model > 2048 and not a multiple of 32, large batch): a long
// launch that, run beside the up projection, costs it more occupancy than it
// saves.
bool gate_ovf_rows_heavy(const GateArgs& a);

// Per-row E4M3 quantisation: q [rows][cols] codes, scale [rows] (quant.hip).
hipError_t launch_quantize_e4m3(const void* in, int is_bf16, int64_t rows, int cols, uint8_t* q, float* scale,
                                hipStream_t s);

struct FwdArgs {
  int64_t N;
  int D, F, tile_n, slots, n_tiles;
  int is_bf16;
  const void* vals;
  const uint16_t* cols;
  const uint16_t* counts;
  const uint8_t* ovf_flag;
  const int32_t* ovf_rows;
  const void* ovf_h;
  const int32_t* n_ovf;
  int ovf_cap;
  const void* x;
  const void* w_up;
  const void* w_down;
  float* y;
  float* a_save;
  int32_t* offs;  // [N]: number of packed entries of each row (workspace)
  uint2* zlist;   // [N][n_t*S]: (column, z = h*a) of every packed entry, row-major (workspace)
  float* upart;   // [up_nq][N][n_t*S]: partial a over each d_model range (workspace, up_nq > 1)
  int32_t* uslot; // [N][n_t*S]: slot of each list entry, for a_save (workspace, up_nq > 1)
  int up_nq;      // passes of the up projection over d_model (up_passes)
  float* part;    // [ovf_cap][G][D] fp32 partial outputs of dense-row chunks (workspace)
  uint16_t* zov;  // bf16: [2][ovf_cap][dense_z_stride(F)] high / low bf16 parts of the overflow rows' z (workspace)
  int32_t* gbase; // [ceil(n_t / kUpGroupTiles)][N]: list position of each tile group's first entry (workspace)
  // order of the down projection's 4-row blocks, heaviest first (large bf16
  // batches; null: natural order) and what up_rows leaves for it (workspace)
  int32_t* rb_order;  // [ceil(N / 4)]
  int32_t* rb_code;   // [ceil(N / 4)]: weight class << 16 | rank among its workgroup's blocks of that class
  int32_t* rb_hist;   // [ceil(N / 256)][16]: blocks of each class per up_rows workgroup
};

hipError_t launch_ffn_fwd(const FwdArgs& a, hipStream_t s);
// Up projection of large bf16 batches with weight-row reuse through LDS
// (up_blocked.hip): list lengths and group positions, then z and a_save.
bool up_blocked_applies(const FwdArgs& a);
hipError_t launch_up_blocked(const FwdArgs& a, hipStream_t s);
// launch_up_blocked also orders the down projection's 4-row blocks (a.rb_order,
// heaviest first) when this holds.
bool down_order_applies(const FwdArgs& a);
// Overflow rows of bf16 layers as two skinny MFMA products (dense_rows.hip):
// z = h * (X_o . W_up^T), then z . W_down in d_ff chunks and dense_reduce.
bool dense_mfma_applies(const FwdArgs& a);
hipError_t launch_dense_mfma(const FwdArgs& a, hipStream_t s);
// The overflow rows' dense activations h = Q(ReLU(g - t)) (bf16 gate), one
// wave per 16 columns over all of d_model, g bit-identical to the gate GEMM's.
bool gate_rows_skinny_applies(int D);
hipError_t launch_gate_rows_skinny(const uint16_t* x, const uint16_t* w, int D, int F, const int32_t* rows,
                                   const int32_t* n_ovf, int cap, const float* t, uint16_t* ovf_h, hipStream_t s);
// Gate + pack (g) followed by the up/down projection (f) in one call: the
// overflow branch of both (list, dense rows, their up/down products) runs on
// the side stream beside the up/down projection of the other rows. With
// `side` false everything is enqueued on `s` in order (no side stream is
// created or used); the results are the same.
hipError_t launch_forward(const GateArgs& g, const FwdArgs& f, hipStream_t s, bool side = true);

// Side stream of the caller's stream (one per caller stream and device,
// side_stream.hip) for the independent branch of a call: fork_side makes it
// wait for the work enqueued on `main` and returns it (or `main` itself when
// there is none: a capture in progress, too many caller streams, or a
// creation failure); join_side makes `main` wait for the work enqueued on it.
hipError_t fork_side(hipStream_t main, hipStream_t* side);
hipError_t join_side(hipStream_t main, hipStream_t side);
// A join in two steps: mark_side marks the work enqueued on `side` so far;
// wait_mark makes `main` wait for that mark (not for what `side` took on
// after it). No-ops when side == main.
hipError_t mark_side(hipStream_t main, hipStream_t side);
hipError_t wait_mark(hipStream_t main, hipStream_t side);

// out[rows[o]] = sum_g part[o][g] for o < min(*n_rows, cap), part [cap][G][D].
hipError_t launch_dense_reduce(const float* part, const int32_t* rows, const int32_t* n_rows, int cap, int G,
                               int D, float* out, hipStream_t s);

struct RouteArgs {
  int64_t N;
  int F, tile_n, slots, n_tiles, row_cap, dense_cap;
  int is_bf16;
  const void* vals;
  const uint16_t* cols;
  const uint16_t* counts;
  const uint8_t* ovf_flag;
  const int32_t* ovf_rows;
  const void* ovf_h;
  const int32_t* n_ovf;
  int ovf_cap;
  const float* a_save;
  void* ell_vals;
  int32_t* ell_cols;
  float* ell_a;
  int32_t* row_nnz;
  uint8_t* is_dense;
  int32_t* dense_rows;
  void* dense_h;
  int32_t* n_dense;
  uint32_t* status;
};

hipError_t launch_route(const RouteArgs& a, hipStream_t s);

struct BwdWorkspace {
  int32_t* row_ptr;    // [N+1]
  int32_t* dense_pos;  // [N] position in dense_rows or -1
  int32_t* pair_col;   // [nnz_max]
  float4* coef;        // [nnz_max] (z, da, dg, 0)
  int32_t* csc_pair;   // [nnz_max]
  int32_t* csc_row;    // [nnz_max]
  int32_t* col_ptr;    // [F+1]
  int32_t* blk_cnt;    // [2][n_rb][F]: per row block and column the row mask, then the column's earlier count
  int32_t* grp_off;    // [dense_cap][G]
  int32_t* egrp;       // [ceil(F / 512) + 1][N] ELL position of each row's first entry per 512-column group
  // dense-backup rows on the matrix cores (bf16, d_model a multiple of 128; else null):
  float* dza;          // [2][dense_cap][F] dz, then a, of every unit of the dense rows
  uint16_t* dadg;      // [4][dense_cap][dense_z_stride(F)] da high, da low, dg high, dg low (bf16)
  float* dxpart;       // [dense_cap][G][D] partial dx of the d_ff chunks
};

struct BwdArgs {
  int64_t N;
  int D, F, row_cap, dense_cap;
  int is_bf16;
  const void* ell_vals;
  const int32_t* ell_cols;
  const float* ell_a;
  const int32_t* row_nnz;
  const uint8_t* is_dense;
  const int32_t* dense_rows;
  const void* dense_h;
  const int32_t* n_dense;
  const void* x;
  const void* dy;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  float lam;
  float* dx;
  float* dw_gate;
  float* dw_up;
  float* dw_down;
  BwdWorkspace ws;
};

hipError_t launch_ffn_bwd(const BwdArgs& a, hipStream_t s);
// dz records of the ELL rows with weight-row reuse through LDS
// (bwd_blocked.hip): the per-row group positions (unless groups_done: the
// caller's row-offset launch wrote them), then the blocked product.
int dz_groups(int F);
bool dz_blocked_applies(const BwdArgs& a);
hipError_t launch_dz_blocked(const BwdArgs& a, hipStream_t s, bool groups_done);
// Dense-backup rows as skinny MFMA products (bwd_dense.hip): dz and a, then
// their records and da / dg; then dx of those rows (bwd_dx skips them).
bool bwd_dense_mfma_applies(const BwdArgs& a);
hipError_t launch_bwd_dense_nt(const BwdArgs& a, hipStream_t s);       // dz, a (needs the dense-row list)
hipError_t launch_bwd_dense_records(const BwdArgs& a, hipStream_t s);  // records, da, dg (needs row_ptr)
hipError_t launch_bwd_dense_dx(const BwdArgs& a, hipStream_t s);

}  // namespace twell
