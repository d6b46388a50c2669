// C ABI of libtwell: host-side validation, then kernel launches on the
// caller's stream. See include/twell.h for the contract of every call.
#include <string>

#include "twell_host.h"
#include "twell_internal.h"
#include "twell_kernels.h"

namespace {

thread_local std::string g_last_error;

twell_status fail(twell_status st, const std::string& why) {
  g_last_error = why;
  return st;
}

twell_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return TWELL_OK;
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return TWELL_ERR_HIP;
}

#define TWELL_CHECK_PTR(p, bytes, name)                                                   \
  do {                                                                                    \
    if (twell::bad_ptr((p), (bytes)))                                                     \
      return fail(TWELL_ERR_INVALID_ARG, std::string(name) + " is NULL or not 16-byte aligned"); \
  } while (0)

twell_status check_pack(const twell_pack* p, const twell_sizes& z) {
  if (p == nullptr) return fail(TWELL_ERR_INVALID_ARG, "pack is NULL");
  TWELL_CHECK_PTR(p->vals, z.vals, "pack.vals");
  TWELL_CHECK_PTR(p->cols, z.cols, "pack.cols");
  TWELL_CHECK_PTR(p->counts, z.counts, "pack.counts");
  TWELL_CHECK_PTR(p->ovf_flag, z.ovf_flag, "pack.ovf_flag");
  TWELL_CHECK_PTR(p->ovf_rows, z.ovf_rows, "pack.ovf_rows");
  TWELL_CHECK_PTR(p->ovf_h, z.ovf_h, "pack.ovf_h");
  TWELL_CHECK_PTR(p->n_ovf, z.n_ovf, "pack.n_ovf");
  TWELL_CHECK_PTR(p->status, z.status, "pack.status");
  return TWELL_OK;
}

twell_status prepare(const twell_dims* dims, twell_dtype dtype, twell::Shape* s, twell_sizes* z) {
  std::string why;
  const twell_status st = twell::check_shape(dims, (int)dtype, s, &why);
  if (st != TWELL_OK) return fail(st, why);
  twell::compute_sizes(*s, z);
  g_last_error.clear();
  return TWELL_OK;
}

}  // namespace

namespace twell {

twell_status set_error(twell_status st, const char* why) { return fail(st, why); }

}  // namespace twell

extern "C" {

const char* twell_status_str(int status) {
  switch (status) {
    case TWELL_OK: return "TWELL_OK";
    case TWELL_ERR_INVALID_ARG: return "TWELL_ERR_INVALID_ARG";
    case TWELL_ERR_UNSUPPORTED: return "TWELL_ERR_UNSUPPORTED";
    case TWELL_ERR_WORKSPACE: return "TWELL_ERR_WORKSPACE";
    case TWELL_ERR_CAPACITY: return "TWELL_ERR_CAPACITY";
    case TWELL_ERR_HIP: return "TWELL_ERR_HIP";
    default: return "TWELL_ERR_UNKNOWN";
  }
}

const char* twell_last_error(void) { return g_last_error.c_str(); }

int32_t twell_n_tiles(const twell_dims* dims) {
  if (dims == nullptr || dims->d_ff <= 0 || dims->tile_n <= 0) return -1;
  return (dims->d_ff + dims->tile_n - 1) / dims->tile_n;
}

twell_status twell_query_sizes(const twell_dims* dims, twell_dtype dtype, twell_sizes* out) {
  if (out == nullptr) return fail(TWELL_ERR_INVALID_ARG, "out is NULL");
  twell::Shape s;
  return prepare(dims, dtype, &s, out);
}

// Workspace of the small-batch gate (twell_sizes.ws_gate bytes; none needed
// when that is 0 or the caller did not take the _ws entry point).
static twell_status check_gate_ws(const twell_sizes& z, void* ws, size_t ws_bytes, bool use_ws) {
  if (!use_ws || z.ws_gate == 0) return TWELL_OK;
  if (ws_bytes < z.ws_gate) return fail(TWELL_ERR_WORKSPACE, "gate workspace smaller than twell_sizes.ws_gate");
  TWELL_CHECK_PTR(ws, z.ws_gate, "ws");
  return TWELL_OK;
}

// The launch arguments every gate entry point shares: shape, thresholds, the
// pack's outputs, the optional g copy and the small-batch workspace.
static twell::GateArgs gate_args(const twell::Shape& s, const twell_sizes& z, const float* t, const twell_pack* out,
                                 float* g_dump, void* ws, bool use_ws) {
  twell::GateArgs a{};
  a.N = s.N;
  a.D = s.D;
  a.F = s.F;
  a.tile_n = s.tile_n;
  a.slots = s.slots;
  a.n_tiles = s.n_tiles;
  a.t = t;
  a.vals = out->vals;
  a.cols = out->cols;
  a.counts = out->counts;
  a.ovf_flag = out->ovf_flag;
  a.ovf_rows = out->ovf_rows;
  a.ovf_h = out->ovf_h;
  a.n_ovf = out->n_ovf;
  a.status = out->status;
  a.ovf_cap = s.ovf_cap;
  a.g_dump = g_dump;
  a.g_ws = (use_ws && z.ws_gate > 0) ? static_cast<float*>(ws) : nullptr;
  return a;
}

// Validation and launch arguments of a bf16 / fp32 gate call (x and w_gate_t,
// or a given pre-activation g).
static twell_status gate_prepare(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                                 const float* g_in, bool from_g, const float* t, const twell_pack* out,
                                 float* g_dump, void* ws, size_t ws_bytes, bool use_ws, twell::Shape* s,
                                 twell_sizes* z, twell::GateArgs* a) {
  twell_status st = prepare(dims, dtype, s, z);
  if (st != TWELL_OK) return st;
  if ((st = check_gate_ws(*z, ws, ws_bytes, use_ws)) != TWELL_OK) return st;
  const size_t xd = (size_t)s->N * s->D * s->esz, wd = (size_t)s->F * s->D * s->esz;
  if (!from_g) {
    TWELL_CHECK_PTR(x, xd, "x");
    TWELL_CHECK_PTR(w_gate_t, wd, "w_gate_t");
  } else {
    TWELL_CHECK_PTR(g_in, (size_t)s->N * s->F * 4, "g");
  }
  TWELL_CHECK_PTR(t, (size_t)s->N * 4, "t");
  if ((st = check_pack(out, *z)) != TWELL_OK) return st;
  if (g_dump != nullptr) TWELL_CHECK_PTR(g_dump, (size_t)s->N * s->F * 4, "g_dump");
  *a = gate_args(*s, *z, t, out, g_dump, ws, use_ws);
  a->is_bf16 = dtype == TWELL_BF16;
  a->x = x;
  a->w = w_gate_t;
  a->g_in = g_in;
  return TWELL_OK;
}

static twell_status gate_common(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                                const float* g_in, bool from_g, const float* t, const twell_pack* out,
                                float* g_dump, void* ws, size_t ws_bytes, bool use_ws, void* stream) {
  twell::Shape s;
  twell_sizes z;
  twell::GateArgs a{};
  const twell_status st =
      gate_prepare(dims, dtype, x, w_gate_t, g_in, from_g, t, out, g_dump, ws, ws_bytes, use_ws, &s, &z, &a);
  if (st != TWELL_OK || s.N == 0) return st;
  return hip_status(twell::launch_gate_pack(a, (hipStream_t)stream), "twell_gate_pack");
}

twell_status twell_gate_pack(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                             const float* t, const twell_pack* out, float* g_dump, void* stream) {
  return gate_common(dims, dtype, x, w_gate_t, nullptr, false, t, out, g_dump, nullptr, 0, false, stream);
}

twell_status twell_gate_pack_ws(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                                const float* t, const twell_pack* out, float* g_dump, void* ws, size_t ws_bytes,
                                void* stream) {
  return gate_common(dims, dtype, x, w_gate_t, nullptr, false, t, out, g_dump, ws, ws_bytes, true, stream);
}

twell_status twell_quantize_e4m3(int64_t rows, int32_t cols, twell_dtype dtype, const void* in, uint8_t* q,
                                 float* scale, void* stream) {
  if (rows < 0 || cols <= 0) return fail(TWELL_ERR_INVALID_ARG, "rows must be >= 0 and cols > 0");
  if (dtype != TWELL_BF16 && dtype != TWELL_F32) return fail(TWELL_ERR_INVALID_ARG, "dtype must be bf16 or fp32");
  if (rows > 0x7FFFFFFFll) return fail(TWELL_ERR_UNSUPPORTED, "rows above 2^31 - 1");
  const size_t esz = dtype == TWELL_BF16 ? 2 : 4;
  TWELL_CHECK_PTR(in, (size_t)rows * cols * esz, "in");
  TWELL_CHECK_PTR(q, (size_t)rows * cols, "q");
  TWELL_CHECK_PTR(scale, (size_t)rows * 4, "scale");
  g_last_error.clear();
  return hip_status(twell::launch_quantize_e4m3(in, dtype == TWELL_BF16, rows, cols, q, scale, (hipStream_t)stream),
                    "twell_quantize_e4m3");
}

// Validation and launch arguments of an FP8 gate call.
static twell_status fp8_prepare(const twell_dims* dims, const uint8_t* x_q, const float* x_scale, const uint8_t* w_q,
                                const float* w_scale, const float* t, const twell_pack* out, float* g_dump, void* ws,
                                size_t ws_bytes, bool use_ws, twell::Shape* s, twell_sizes* z, twell::GateArgs* a) {
  twell_status st = prepare(dims, TWELL_BF16, s, z);
  if (st != TWELL_OK) return st;
  if ((st = check_gate_ws(*z, ws, ws_bytes, use_ws)) != TWELL_OK) return st;
  if (s->D % 64 != 0) return fail(TWELL_ERR_UNSUPPORTED, "the FP8 gate needs d_model to be a multiple of 64");
  TWELL_CHECK_PTR(x_q, (size_t)s->N * s->D, "x_q");
  TWELL_CHECK_PTR(x_scale, (size_t)s->N * 4, "x_scale");
  TWELL_CHECK_PTR(w_q, (size_t)s->F * s->D, "w_q");
  TWELL_CHECK_PTR(w_scale, (size_t)s->F * 4, "w_scale");
  TWELL_CHECK_PTR(t, (size_t)s->N * 4, "t");
  if ((st = check_pack(out, *z)) != TWELL_OK) return st;
  if (g_dump != nullptr) TWELL_CHECK_PTR(g_dump, (size_t)s->N * s->F * 4, "g_dump");
  *a = gate_args(*s, *z, t, out, g_dump, ws, use_ws);
  a->is_bf16 = 1;  // TwELL values and overflow rows are stored in bf16
  a->fp8 = 1;
  a->x = x_q;
  a->w = w_q;
  a->x_scale = x_scale;
  a->w_scale = w_scale;
  return TWELL_OK;
}

static twell_status fp8_common(const twell_dims* dims, const uint8_t* x_q, const float* x_scale, const uint8_t* w_q,
                               const float* w_scale, const float* t, const twell_pack* out, float* g_dump, void* ws,
                               size_t ws_bytes, bool use_ws, void* stream) {
  twell::Shape s;
  twell_sizes z;
  twell::GateArgs a{};
  const twell_status st =
      fp8_prepare(dims, x_q, x_scale, w_q, w_scale, t, out, g_dump, ws, ws_bytes, use_ws, &s, &z, &a);
  if (st != TWELL_OK || s.N == 0) return st;
  return hip_status(twell::launch_gate_pack(a, (hipStream_t)stream), "twell_gate_pack_fp8");
}

twell_status twell_gate_pack_fp8(const twell_dims* dims, const uint8_t* x_q, const float* x_scale,
                                 const uint8_t* w_q, const float* w_scale, const float* t, const twell_pack* out,
                                 float* g_dump, void* stream) {
  return fp8_common(dims, x_q, x_scale, w_q, w_scale, t, out, g_dump, nullptr, 0, false, stream);
}

twell_status twell_gate_pack_fp8_ws(const twell_dims* dims, const uint8_t* x_q, const float* x_scale,
                                    const uint8_t* w_q, const float* w_scale, const float* t, const twell_pack* out,
                                    float* g_dump, void* ws, size_t ws_bytes, void* stream) {
  return fp8_common(dims, x_q, x_scale, w_q, w_scale, t, out, g_dump, ws, ws_bytes, true, stream);
}

twell_status twell_pack_preact(const twell_dims* dims, twell_dtype dtype, const float* g, const float* t,
                               const twell_pack* out, void* stream) {
  return gate_common(dims, dtype, nullptr, nullptr, g, true, t, out, nullptr, nullptr, 0, false, stream);
}

// Validation and launch arguments of the up/down projection (shape already
// checked by the caller).
static twell_status fwd_prepare(const twell::Shape& s, const twell_sizes& z, twell_dtype dtype,
                                const twell_pack* pack, const void* x, const void* w_up_t, const void* w_down,
                                float* y, float* a_save, void* ws, size_t ws_bytes, twell::FwdArgs* out) {
  twell_status st;
  if ((st = check_pack(pack, z)) != TWELL_OK) return st;
  const size_t xd = (size_t)s.N * s.D * s.esz, wd = (size_t)s.F * s.D * s.esz;
  TWELL_CHECK_PTR(x, xd, "x");
  TWELL_CHECK_PTR(w_up_t, wd, "w_up_t");
  TWELL_CHECK_PTR(w_down, wd, "w_down");
  TWELL_CHECK_PTR(y, (size_t)s.N * s.D * 4, "y");
  if (a_save != nullptr) TWELL_CHECK_PTR(a_save, z.a_save, "a_save");
  if (ws_bytes < z.ws_fwd) return fail(TWELL_ERR_WORKSPACE, "forward workspace smaller than twell_sizes.ws_fwd");
  if (twell::bad_ptr(ws, z.ws_fwd))
    return fail(TWELL_ERR_WORKSPACE, "forward workspace is NULL or not 16-byte aligned");

  twell::FwdArgs a{};
  a.N = s.N;
  a.D = s.D;
  a.F = s.F;
  a.tile_n = s.tile_n;
  a.slots = s.slots;
  a.n_tiles = s.n_tiles;
  a.is_bf16 = dtype == TWELL_BF16;
  a.vals = pack->vals;
  a.cols = pack->cols;
  a.counts = pack->counts;
  a.ovf_flag = pack->ovf_flag;
  a.ovf_rows = pack->ovf_rows;
  a.ovf_h = pack->ovf_h;
  a.n_ovf = pack->n_ovf;
  a.ovf_cap = s.slots >= s.tile_n ? 0 : s.ovf_cap;  // slots >= tile_n: no row can overflow
  a.x = x;
  a.w_up = w_up_t;
  a.w_down = w_down;
  a.y = y;
  a.a_save = a_save;
  if (s.N > 0) {
    const twell::FwdLayout L = twell::fwd_layout(s);
    char* base = reinterpret_cast<char*>(ws);
    a.offs = reinterpret_cast<int32_t*>(base + L.offs);
    a.zlist = reinterpret_cast<uint2*>(base + L.zlist);
    a.upart = reinterpret_cast<float*>(base + L.upart);
    a.uslot = reinterpret_cast<int32_t*>(base + L.uslot);
    a.up_nq = twell::up_passes(s);
    a.part = reinterpret_cast<float*>(base + L.part);
    a.zov = reinterpret_cast<uint16_t*>(base + L.zov);
    a.gbase = reinterpret_cast<int32_t*>(base + L.gbase);
    a.rb_order = reinterpret_cast<int32_t*>(base + L.rb_order);
    a.rb_code = reinterpret_cast<int32_t*>(base + L.rb_code);
    a.rb_hist = reinterpret_cast<int32_t*>(base + L.rb_hist);
  }
  *out = a;
  return TWELL_OK;
}

twell_status twell_ffn_fwd(const twell_dims* dims, twell_dtype dtype, const twell_pack* pack, const void* x,
                           const void* w_up_t, const void* w_down, float* y, float* a_save, void* ws,
                           size_t ws_bytes, void* stream) {
  twell::Shape s;
  twell_sizes z;
  twell_status st = prepare(dims, dtype, &s, &z);
  if (st != TWELL_OK) return st;
  twell::FwdArgs a{};
  if ((st = fwd_prepare(s, z, dtype, pack, x, w_up_t, w_down, y, a_save, ws, ws_bytes, &a)) != TWELL_OK) return st;
  if (s.N == 0) return TWELL_OK;
  return hip_status(twell::launch_ffn_fwd(a, (hipStream_t)stream), "twell_ffn_fwd");
}

twell_status twell_ffn_forward_fp8(const twell_dims* dims, const uint8_t* x_q, const float* x_scale,
                                   const uint8_t* w_q, const float* w_scale, const float* t, const twell_pack* pack,
                                   const void* x, const void* w_up_t, const void* w_down, float* y, float* a_save,
                                   void* ws, size_t ws_bytes, void* gate_ws, size_t gate_ws_bytes, void* stream) {
  twell::Shape s;
  twell_sizes z;
  twell::GateArgs g{};
  twell_status st = fp8_prepare(dims, x_q, x_scale, w_q, w_scale, t, pack, nullptr, gate_ws, gate_ws_bytes,
                                gate_ws != nullptr, &s, &z, &g);
  if (st != TWELL_OK) return st;
  twell::FwdArgs f{};
  if ((st = fwd_prepare(s, z, TWELL_BF16, pack, x, w_up_t, w_down, y, a_save, ws, ws_bytes, &f)) != TWELL_OK)
    return st;
  if (s.N == 0) return TWELL_OK;
  return hip_status(twell::launch_forward(g, f, (hipStream_t)stream), "twell_ffn_forward_fp8");
}

twell_status twell_ffn_forward(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                               const float* t, const twell_pack* pack, const void* w_up_t, const void* w_down,
                               float* y, float* a_save, void* ws, size_t ws_bytes, void* gate_ws,
                               size_t gate_ws_bytes, void* stream) {
  return twell::ffn_forward_call(dims, dtype, x, w_gate_t, t, pack, w_up_t, w_down, y, a_save, ws, ws_bytes, gate_ws,
                                 gate_ws_bytes, true, false, stream);
}

static twell_status check_hybrid(const twell_hybrid* h, const twell_sizes& z) {
  if (h == nullptr) return fail(TWELL_ERR_INVALID_ARG, "hybrid is NULL");
  TWELL_CHECK_PTR(h->ell_vals, z.ell_vals, "hybrid.ell_vals");
  TWELL_CHECK_PTR(h->ell_cols, z.ell_cols, "hybrid.ell_cols");
  TWELL_CHECK_PTR(h->ell_a, z.ell_a, "hybrid.ell_a");
  TWELL_CHECK_PTR(h->row_nnz, z.row_nnz, "hybrid.row_nnz");
  TWELL_CHECK_PTR(h->is_dense, z.is_dense, "hybrid.is_dense");
  TWELL_CHECK_PTR(h->dense_rows, z.dense_rows, "hybrid.dense_rows");
  TWELL_CHECK_PTR(h->dense_h, z.dense_h, "hybrid.dense_h");
  TWELL_CHECK_PTR(h->n_dense, z.n_dense, "hybrid.n_dense");
  TWELL_CHECK_PTR(h->status, z.status, "hybrid.status");
  return TWELL_OK;
}

twell_status twell_route_hybrid(const twell_dims* dims, twell_dtype dtype, const twell_pack* pack,
                                const float* a_save, const twell_hybrid* out, void* stream) {
  twell::Shape s;
  twell_sizes z;
  twell_status st = prepare(dims, dtype, &s, &z);
  if (st != TWELL_OK) return st;
  if ((st = check_pack(pack, z)) != TWELL_OK) return st;
  TWELL_CHECK_PTR(a_save, z.a_save, "a_save");
  if ((st = check_hybrid(out, z)) != TWELL_OK) return st;
  if (s.N == 0) return TWELL_OK;
  twell::RouteArgs a{};
  a.N = s.N;
  a.F = s.F;
  a.tile_n = s.tile_n;
  a.slots = s.slots;
  a.n_tiles = s.n_tiles;
  a.row_cap = s.row_cap;
  a.dense_cap = s.dense_cap;
  a.is_bf16 = dtype == TWELL_BF16;
  a.vals = pack->vals;
  a.cols = pack->cols;
  a.counts = pack->counts;
  a.ovf_flag = pack->ovf_flag;
  a.ovf_rows = pack->ovf_rows;
  a.ovf_h = pack->ovf_h;
  a.n_ovf = pack->n_ovf;
  a.ovf_cap = s.ovf_cap;
  a.a_save = a_save;
  a.ell_vals = out->ell_vals;
  a.ell_cols = out->ell_cols;
  a.ell_a = out->ell_a;
  a.row_nnz = out->row_nnz;
  a.is_dense = out->is_dense;
  a.dense_rows = out->dense_rows;
  a.dense_h = out->dense_h;
  a.n_dense = out->n_dense;
  a.status = out->status;
  return hip_status(twell::launch_route(a, (hipStream_t)stream), "twell_route_hybrid");
}

twell_status twell_ffn_bwd(const twell_dims* dims, twell_dtype dtype, const twell_hybrid* hyb, const void* x,
                           const void* dy, const void* w_gate_t, const void* w_up_t, const void* w_down,
                           float l1_lambda, float* dx, float* dw_gate_t, float* dw_up_t, float* dw_down, void* ws,
                           size_t ws_bytes, void* stream) {
  twell::Shape s;
  twell_sizes z;
  twell_status st = prepare(dims, dtype, &s, &z);
  if (st != TWELL_OK) return st;
  if ((st = check_hybrid(hyb, z)) != TWELL_OK) return st;
  const size_t xd = (size_t)s.N * s.D * s.esz, wd = (size_t)s.F * s.D * s.esz;
  TWELL_CHECK_PTR(x, xd, "x");
  TWELL_CHECK_PTR(dy, xd, "dy");
  TWELL_CHECK_PTR(w_gate_t, wd, "w_gate_t");
  TWELL_CHECK_PTR(w_up_t, wd, "w_up_t");
  TWELL_CHECK_PTR(w_down, wd, "w_down");
  TWELL_CHECK_PTR(dx, (size_t)s.N * s.D * 4, "dx");
  TWELL_CHECK_PTR(dw_gate_t, (size_t)s.F * s.D * 4, "dw_gate_t");
  TWELL_CHECK_PTR(dw_up_t, (size_t)s.F * s.D * 4, "dw_up_t");
  TWELL_CHECK_PTR(dw_down, (size_t)s.F * s.D * 4, "dw_down");
  if (s.F > 32768)  // the column transpose keeps a 32-bit row mask for every column in LDS
    return fail(TWELL_ERR_UNSUPPORTED, "twell_ffn_bwd supports d_ff <= 32768");
  if (!(l1_lambda == l1_lambda) || l1_lambda - l1_lambda != 0.f)
    return fail(TWELL_ERR_INVALID_ARG, "l1_lambda must be finite");
  if (ws_bytes < z.ws_bwd) return fail(TWELL_ERR_WORKSPACE, "backward workspace smaller than twell_sizes.ws_bwd");
  if (twell::bad_ptr(ws, z.ws_bwd)) return fail(TWELL_ERR_WORKSPACE, "backward workspace is NULL or misaligned");
  if (s.N == 0) return TWELL_OK;

  const twell::BwdLayout L = twell::bwd_layout(s);
  char* base = reinterpret_cast<char*>(ws);
  twell::BwdArgs a{};
  a.N = s.N;
  a.D = s.D;
  a.F = s.F;
  a.row_cap = s.row_cap;
  a.dense_cap = s.dense_cap;
  a.is_bf16 = dtype == TWELL_BF16;
  a.ell_vals = hyb->ell_vals;
  a.ell_cols = hyb->ell_cols;
  a.ell_a = hyb->ell_a;
  a.row_nnz = hyb->row_nnz;
  a.is_dense = hyb->is_dense;
  a.dense_rows = hyb->dense_rows;
  a.dense_h = hyb->dense_h;
  a.n_dense = hyb->n_dense;
  a.x = x;
  a.dy = dy;
  a.w_gate = w_gate_t;
  a.w_up = w_up_t;
  a.w_down = w_down;
  a.lam = l1_lambda;
  a.dx = dx;
  a.dw_gate = dw_gate_t;
  a.dw_up = dw_up_t;
  a.dw_down = dw_down;
  a.ws.row_ptr = reinterpret_cast<int32_t*>(base + L.row_ptr);
  a.ws.dense_pos = reinterpret_cast<int32_t*>(base + L.dense_pos);
  a.ws.pair_col = reinterpret_cast<int32_t*>(base + L.pair_col);
  a.ws.coef = reinterpret_cast<float4*>(base + L.coef);
  a.ws.csc_pair = reinterpret_cast<int32_t*>(base + L.csc_pair);
  a.ws.csc_row = reinterpret_cast<int32_t*>(base + L.csc_row);
  a.ws.col_ptr = reinterpret_cast<int32_t*>(base + L.col_ptr);
  a.ws.blk_cnt = reinterpret_cast<int32_t*>(base + L.blk_cnt);
  a.ws.grp_off = reinterpret_cast<int32_t*>(base + L.grp_off);
  a.ws.egrp = reinterpret_cast<int32_t*>(base + L.egrp);
  if (twell::bwd_dense_mfma(s)) {
    a.ws.dza = reinterpret_cast<float*>(base + L.dza);
    a.ws.dadg = reinterpret_cast<uint16_t*>(base + L.dadg);
    a.ws.dxpart = reinterpret_cast<float*>(base + L.dxpart);
  }
  return hip_status(twell::launch_ffn_bwd(a, (hipStream_t)stream), "twell_ffn_bwd");
}

}  // extern "C"

namespace twell {

twell_status ffn_forward_call(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                              const float* t, const twell_pack* pack, const void* w_up_t, const void* w_down,
                              float* y, float* a_save, void* ws, size_t ws_bytes, void* gate_ws, size_t gate_ws_bytes,
                              bool use_side, bool validate_only, void* stream) {
  twell::Shape s;
  twell_sizes z;
  twell::GateArgs g{};
  twell_status st = gate_prepare(dims, dtype, x, w_gate_t, nullptr, false, t, pack, nullptr, gate_ws,
                                 gate_ws_bytes, gate_ws != nullptr, &s, &z, &g);
  if (st != TWELL_OK) return st;
  twell::FwdArgs f{};
  if ((st = fwd_prepare(s, z, dtype, pack, x, w_up_t, w_down, y, a_save, ws, ws_bytes, &f)) != TWELL_OK) return st;
  if (s.N == 0 || validate_only) return TWELL_OK;
  return hip_status(twell::launch_forward(g, f, (hipStream_t)stream, use_side), "twell_ffn_forward");
}

}  // namespace twell
