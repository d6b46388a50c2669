// Host-side check of libtwell's C ABI, built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_host_sanitize.py builds and runs
// it; no GPU and no device code are involved).
//
// The C ABI sources (validation, size queries, workspace layouts, launch
// argument marshalling, tracing, side stream) are compiled as plain C++ and
// linked against the stand-ins below for the launch functions of the kernel
// files. Each stand-in checks that every array the kernels would touch, at the
// extent the kernels index it, lies inside one of the buffers the caller
// allocated from twell_query_sizes, and reads the first and last byte of it
// (so the sanitizer sees an access outside an allocation). The driver calls
// every entry point with buffers of exactly the queried sizes, for every
// benchmark shape and a set of edge shapes, and checks the error paths.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "twell.h"
#include "twell_host.h"
#include "twell_kernels.h"

namespace {

int g_failures = 0;
std::string g_where;

#define CHECK(cond, ...)                                                  \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "FAIL [%s] %s:%d: ", g_where.c_str(), __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                                  \
      std::fprintf(stderr, "\n");                                         \
      ++g_failures;                                                       \
    }                                                                     \
  } while (0)

struct Buf {
  unsigned char* p;
  size_t n;
  const char* name;
};
std::vector<Buf> g_bufs;

// Exactly `n` bytes (16-byte aligned), registered for the extent checks.
void* alloc(size_t n, const char* name) {
  if (n == 0) return nullptr;
  void* p = std::aligned_alloc(256, (n + 255) / 256 * 256);
  if (p == nullptr) {
    std::fprintf(stderr, "out of host memory for %s (%zu bytes)\n", name, n);
    std::exit(2);
  }
  g_bufs.push_back({static_cast<unsigned char*>(p), n, name});
  return p;
}

void free_all() {
  for (auto& b : g_bufs) std::free(b.p);
  g_bufs.clear();
}

volatile unsigned char g_sink;

// [p, p + bytes) must lie inside one caller buffer.
void extent(const void* p, size_t bytes, const char* what) {
  if (bytes == 0) return;
  CHECK(p != nullptr, "%s: null pointer for %zu bytes", what, bytes);
  if (p == nullptr) return;
  const unsigned char* q = static_cast<const unsigned char*>(p);
  for (const Buf& b : g_bufs) {
    if (q >= b.p && q < b.p + b.n) {
      CHECK(q + bytes <= b.p + b.n, "%s: %zu bytes at offset %zu overrun buffer %s of %zu bytes", what, bytes,
            (size_t)(q - b.p), b.name, b.n);
      if (q + bytes <= b.p + b.n) g_sink = q[0] ^ q[bytes - 1];
      return;
    }
  }
  CHECK(false, "%s: pointer outside every caller buffer", what);
}

int g_launches = 0;

}  // namespace

// ---------------------------------------------------------------- stand-ins for the kernel files

namespace twell {

static void gate_extents(const GateArgs& a) {
  const size_t N = (size_t)a.N, D = (size_t)a.D, F = (size_t)a.F, nt = (size_t)a.n_tiles, S = (size_t)a.slots;
  const size_t esz = a.fp8 ? 1 : (a.is_bf16 ? 2 : 4), vsz = a.is_bf16 ? 2 : 4;
  if (a.g_in) {
    extent(a.g_in, N * F * 4, "g");
  } else {
    extent(a.x, N * D * esz, "x");
    extent(a.w, F * D * esz, "w_gate_t");
  }
  extent(a.t, N * 4, "t");
  extent(a.vals, nt * S * N * vsz, "vals");
  extent(a.cols, nt * S * N * 2, "cols");
  extent(a.counts, nt * N * 2, "counts");
  extent(a.ovf_flag, N, "ovf_flag");
  extent(a.ovf_rows, (size_t)a.ovf_cap * 4, "ovf_rows");
  extent(a.ovf_h, (size_t)a.ovf_cap * F * vsz, "ovf_h");
  extent(a.n_ovf, 4, "n_ovf");
  extent(a.status, 4, "status");
  if (a.g_dump) extent(a.g_dump, N * F * 4, "g_dump");
  if (a.g_ws) extent(a.g_ws, N * F * 4, "gate ws");
  if (a.fp8) {
    extent(a.x_scale, N * 4, "x_scale");
    extent(a.w_scale, F * 4, "w_scale");
  }
}

static void fwd_extents(const FwdArgs& a) {
  const size_t N = (size_t)a.N, D = (size_t)a.D, F = (size_t)a.F, nt = (size_t)a.n_tiles, S = (size_t)a.slots;
  const size_t esz = a.is_bf16 ? 2 : 4, L = nt * S;
  const size_t G = (F + kDenseChunk - 1) / kDenseChunk;
  extent(a.vals, nt * S * N * esz, "vals");
  extent(a.cols, nt * S * N * 2, "cols");
  extent(a.counts, nt * N * 2, "counts");
  extent(a.x, N * D * esz, "x");
  extent(a.w_up, F * D * esz, "w_up_t");
  extent(a.w_down, F * D * esz, "w_down");
  extent(a.y, N * D * 4, "y");
  if (a.a_save) extent(a.a_save, nt * S * N * 4, "a_save");
  extent(a.offs, N * 4, "ws.offs");
  extent(a.gbase, (nt + kUpGroupTiles - 1) / kUpGroupTiles * N * 4, "ws.gbase");
  extent(a.zlist, N * L * 8, "ws.zlist");
  extent(a.rb_order, (N + 3) / 4 * 4, "ws.rb_order");
  extent(a.rb_code, (N + 3) / 4 * 4, "ws.rb_code");
  extent(a.rb_hist, (N + 255) / 256 * 16 * 4, "ws.rb_hist");
  CHECK(a.up_nq >= 1 && D % (size_t)a.up_nq == 0, "up_nq %d does not divide d_model", a.up_nq);
  if (a.up_nq > 1) {
    extent(a.upart, (size_t)a.up_nq * N * L * 4, "ws.upart");
    extent(a.uslot, N * L * 4, "ws.uslot");
  }
  if (a.ovf_cap > 0) {
    extent(a.ovf_flag, N, "ovf_flag");
    extent(a.ovf_rows, (size_t)a.ovf_cap * 4, "ovf_rows");
    extent(a.ovf_h, (size_t)a.ovf_cap * F * esz, "ovf_h");
    extent(a.n_ovf, 4, "n_ovf");
    extent(a.part, (size_t)a.ovf_cap * G * D * 4, "ws.part");
    if (a.is_bf16) extent(a.zov, (size_t)2 * a.ovf_cap * dense_z_stride(a.F) * 2, "ws.zov");
  }
}

hipError_t launch_gate_pack(const GateArgs& a, hipStream_t) {
  gate_extents(a);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gate_pack_split(const GateArgs& a, hipStream_t s, bool, hipStream_t* o, bool) {
  *o = s;
  return launch_gate_pack(a, s);
}
bool gate_ovf_rows_heavy(const GateArgs&) { return false; }
hipError_t launch_quantize_e4m3(const void* in, int is_bf16, int64_t rows, int cols, uint8_t* q, float* scale,
                                hipStream_t) {
  extent(in, (size_t)rows * cols * (is_bf16 ? 2 : 4), "quantize in");
  extent(q, (size_t)rows * cols, "quantize q");
  extent(scale, (size_t)rows * 4, "quantize scale");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_ffn_fwd(const FwdArgs& a, hipStream_t) {
  fwd_extents(a);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_forward(const GateArgs& g, const FwdArgs& f, hipStream_t, bool) {
  gate_extents(g);
  fwd_extents(f);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_route(const RouteArgs& a, hipStream_t) {
  const size_t N = (size_t)a.N, F = (size_t)a.F, nt = (size_t)a.n_tiles, S = (size_t)a.slots;
  const size_t K = (size_t)a.row_cap, esz = a.is_bf16 ? 2 : 4;
  extent(a.vals, nt * S * N * esz, "vals");
  extent(a.cols, nt * S * N * 2, "cols");
  extent(a.counts, nt * N * 2, "counts");
  extent(a.ovf_flag, N, "ovf_flag");
  extent(a.ovf_rows, (size_t)a.ovf_cap * 4, "ovf_rows");
  extent(a.ovf_h, (size_t)a.ovf_cap * F * esz, "ovf_h");
  extent(a.a_save, nt * S * N * 4, "a_save");
  extent(a.ell_vals, K * N * esz, "ell_vals");
  extent(a.ell_cols, K * N * 4, "ell_cols");
  extent(a.ell_a, K * N * 4, "ell_a");
  extent(a.row_nnz, N * 4, "row_nnz");
  extent(a.is_dense, N, "is_dense");
  extent(a.dense_rows, (size_t)a.dense_cap * 4, "dense_rows");
  extent(a.dense_h, (size_t)a.dense_cap * F * esz, "dense_h");
  extent(a.n_dense, 4, "n_dense");
  extent(a.status, 4, "status");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_ffn_bwd(const BwdArgs& a, hipStream_t) {
  const size_t N = (size_t)a.N, D = (size_t)a.D, F = (size_t)a.F, K = (size_t)a.row_cap;
  const size_t esz = a.is_bf16 ? 2 : 4, dc = (size_t)a.dense_cap;
  const size_t nnz = N * K + dc * F, G = (F + kDenseChunk - 1) / kDenseChunk;
  const size_t nrb = (N + kTransposeRows - 1) / kTransposeRows;
  extent(a.ell_vals, K * N * esz, "ell_vals");
  extent(a.ell_cols, K * N * 4, "ell_cols");
  extent(a.ell_a, K * N * 4, "ell_a");
  extent(a.row_nnz, N * 4, "row_nnz");
  extent(a.is_dense, N, "is_dense");
  extent(a.dense_rows, dc * 4, "dense_rows");
  extent(a.dense_h, dc * F * esz, "dense_h");
  extent(a.n_dense, 4, "n_dense");
  extent(a.x, N * D * esz, "x");
  extent(a.dy, N * D * esz, "dy");
  extent(a.w_gate, F * D * esz, "w_gate_t");
  extent(a.w_up, F * D * esz, "w_up_t");
  extent(a.w_down, F * D * esz, "w_down");
  extent(a.dx, N * D * 4, "dx");
  extent(a.dw_gate, F * D * 4, "dw_gate_t");
  extent(a.dw_up, F * D * 4, "dw_up_t");
  extent(a.dw_down, F * D * 4, "dw_down");
  extent(a.ws.row_ptr, (N + 1 + dc) * 4, "ws.row_ptr (+ dense counts)");
  extent(a.ws.dense_pos, N * 4, "ws.dense_pos");
  extent(a.ws.pair_col, nnz * 4, "ws.pair_col");
  extent(a.ws.coef, nnz * 16, "ws.coef");
  extent(a.ws.csc_pair, nnz * 4, "ws.csc_pair");
  extent(a.ws.csc_row, nnz * 4, "ws.csc_row");
  extent(a.ws.col_ptr, (F + 1) * 4, "ws.col_ptr");
  extent(a.ws.blk_cnt, 2 * nrb * F * 4, "ws.blk_cnt");
  extent(a.ws.grp_off, dc * G * 4, "ws.grp_off");
  extent(a.ws.egrp, ((F + 511) / 512 + 1) * N * 4, "ws.egrp");
  if (a.ws.dza != nullptr) {
    extent(a.ws.dza, 2 * dc * F * 4, "ws.dza");
    extent(a.ws.dadg, 4 * dc * dense_z_stride((int)F) * 2, "ws.dadg");
    extent(a.ws.dxpart, dc * G * D * 4, "ws.dxpart");
  }
  ++g_launches;
  return hipSuccess;
}

}  // namespace twell

// ---------------------------------------------------------------- driver

namespace {

struct Case {
  const char* name;
  int64_t N;
  int D, F, T, S, K, ovf_cap, dense_cap;
  twell_dtype dt;
};

void run_case(const Case& c) {
  g_where = c.name;
  twell_dims d{c.N, c.D, c.F, c.T, c.S, c.K, c.ovf_cap, c.dense_cap};
  twell_sizes z;
  std::memset(&z, 0, sizeof z);
  int st = twell_query_sizes(&d, c.dt, &z);
  CHECK(st == TWELL_OK, "query_sizes: %s (%s)", twell_status_str(st), twell_last_error());
  if (st != TWELL_OK) return;
  const size_t N = (size_t)c.N, D = (size_t)c.D, F = (size_t)c.F, esz = c.dt == TWELL_BF16 ? 2 : 4;
  const int nt = twell_n_tiles(&d);
  CHECK(nt == (c.F + c.T - 1) / c.T, "n_tiles %d", nt);

  twell_pack pk{};
  pk.vals = alloc(z.vals, "vals");
  pk.cols = (uint16_t*)alloc(z.cols, "cols");
  pk.counts = (uint16_t*)alloc(z.counts, "counts");
  pk.ovf_flag = (uint8_t*)alloc(z.ovf_flag, "ovf_flag");
  pk.ovf_rows = (int32_t*)alloc(z.ovf_rows, "ovf_rows");
  pk.ovf_h = alloc(z.ovf_h, "ovf_h");
  pk.n_ovf = (int32_t*)alloc(z.n_ovf, "n_ovf");
  pk.status = (uint32_t*)alloc(z.status, "status");
  void* x = alloc(N * D * esz, "x");
  void* wg = alloc(F * D * esz, "w_gate_t");
  void* wu = alloc(F * D * esz, "w_up_t");
  void* wd = alloc(F * D * esz, "w_down");
  float* t = (float*)alloc(N * 4, "t");
  float* y = (float*)alloc(N * D * 4, "y");
  float* a_save = (float*)alloc(z.a_save, "a_save");
  float* g_dump = (float*)alloc(N * F * 4, "g_dump");
  void* ws = alloc(z.ws_fwd, "ws_fwd");
  void* gws = alloc(z.ws_gate, "ws_gate");

  const int before = g_launches;
  st = twell_gate_pack(&d, c.dt, x, wg, t, &pk, nullptr, nullptr);
  CHECK(st == TWELL_OK, "gate_pack: %s (%s)", twell_status_str(st), twell_last_error());
  st = twell_gate_pack(&d, c.dt, x, wg, t, &pk, g_dump, nullptr);
  CHECK(st == TWELL_OK, "gate_pack with g_dump: %s", twell_status_str(st));
  st = twell_gate_pack_ws(&d, c.dt, x, wg, t, &pk, nullptr, gws, z.ws_gate, nullptr);
  CHECK(st == TWELL_OK, "gate_pack_ws: %s (%s)", twell_status_str(st), twell_last_error());
  st = twell_pack_preact(&d, c.dt, g_dump, t, &pk, nullptr);
  CHECK(st == TWELL_OK, "pack_preact: %s", twell_status_str(st));
  st = twell_ffn_fwd(&d, c.dt, &pk, x, wu, wd, y, nullptr, ws, z.ws_fwd, nullptr);
  CHECK(st == TWELL_OK, "ffn_fwd: %s (%s)", twell_status_str(st), twell_last_error());
  st = twell_ffn_fwd(&d, c.dt, &pk, x, wu, wd, y, a_save, ws, z.ws_fwd, nullptr);
  CHECK(st == TWELL_OK, "ffn_fwd with a_save: %s", twell_status_str(st));
  st = twell_ffn_forward(&d, c.dt, x, wg, t, &pk, wu, wd, y, a_save, ws, z.ws_fwd, gws, z.ws_gate, nullptr);
  CHECK(st == TWELL_OK, "ffn_forward: %s (%s)", twell_status_str(st), twell_last_error());
  if (c.N > 0) CHECK(g_launches > before, "no launch reached the stand-ins");

  // error paths: nothing may reach a launch
  const int mark = g_launches;
  if (z.ws_fwd > 0) {
    st = twell_ffn_fwd(&d, c.dt, &pk, x, wu, wd, y, nullptr, ws, z.ws_fwd - 1, nullptr);
    CHECK(st == TWELL_ERR_WORKSPACE, "short workspace accepted: %s", twell_status_str(st));
  }
  if (z.ws_gate > 0) {
    st = twell_gate_pack_ws(&d, c.dt, x, wg, t, &pk, nullptr, gws, z.ws_gate - 1, nullptr);
    CHECK(st == TWELL_ERR_WORKSPACE, "short gate workspace accepted: %s", twell_status_str(st));
  }
  if (c.N > 0) {
    st = twell_gate_pack(&d, c.dt, static_cast<char*>(x) + 8, wg, t, &pk, nullptr, nullptr);
    CHECK(st == TWELL_ERR_INVALID_ARG, "misaligned x accepted: %s", twell_status_str(st));
    st = twell_ffn_fwd(&d, c.dt, nullptr, x, wu, wd, y, nullptr, ws, z.ws_fwd, nullptr);
    CHECK(st == TWELL_ERR_INVALID_ARG, "null pack accepted: %s", twell_status_str(st));
  }
  CHECK(g_launches == mark, "an invalid call reached a launch");

  if (c.dt == TWELL_BF16 && c.D % 64 == 0) {
    uint8_t* xq = (uint8_t*)alloc(N * D, "x_q");
    uint8_t* wq = (uint8_t*)alloc(F * D, "w_q");
    float* xs = (float*)alloc(N * 4, "x_scale");
    float* wsc = (float*)alloc(F * 4, "w_scale");
    st = twell_quantize_e4m3((int64_t)N, c.D, TWELL_BF16, x, xq, xs, nullptr);
    CHECK(st == TWELL_OK, "quantize x: %s", twell_status_str(st));
    st = twell_quantize_e4m3((int64_t)F, c.D, TWELL_BF16, wg, wq, wsc, nullptr);
    CHECK(st == TWELL_OK, "quantize w: %s", twell_status_str(st));
    st = twell_gate_pack_fp8(&d, xq, xs, wq, wsc, t, &pk, g_dump, nullptr);
    CHECK(st == TWELL_OK, "gate_pack_fp8: %s (%s)", twell_status_str(st), twell_last_error());
    st = twell_gate_pack_fp8_ws(&d, xq, xs, wq, wsc, t, &pk, nullptr, gws, z.ws_gate, nullptr);
    CHECK(st == TWELL_OK, "gate_pack_fp8_ws: %s (%s)", twell_status_str(st), twell_last_error());
    st = twell_ffn_forward_fp8(&d, xq, xs, wq, wsc, t, &pk, x, wu, wd, y, nullptr, ws, z.ws_fwd, gws, z.ws_gate,
                               nullptr);
    CHECK(st == TWELL_OK, "ffn_forward_fp8: %s (%s)", twell_status_str(st), twell_last_error());
  }

  if (c.K > 0) {
    twell_hybrid hb{};
    hb.ell_vals = alloc(z.ell_vals, "ell_vals");
    hb.ell_cols = (int32_t*)alloc(z.ell_cols, "ell_cols");
    hb.ell_a = (float*)alloc(z.ell_a, "ell_a");
    hb.row_nnz = (int32_t*)alloc(z.row_nnz, "row_nnz");
    hb.is_dense = (uint8_t*)alloc(z.is_dense, "is_dense");
    hb.dense_rows = (int32_t*)alloc(z.dense_rows, "dense_rows");
    hb.dense_h = alloc(z.dense_h, "dense_h");
    hb.n_dense = (int32_t*)alloc(z.n_dense, "n_dense");
    hb.status = (uint32_t*)alloc(z.status, "hybrid status");
    void* dy = alloc(N * D * esz, "dy");
    float* dx = (float*)alloc(N * D * 4, "dx");
    float* dwg = (float*)alloc(F * D * 4, "dw_gate_t");
    float* dwu = (float*)alloc(F * D * 4, "dw_up_t");
    float* dwd = (float*)alloc(F * D * 4, "dw_down");
    void* wsb = alloc(z.ws_bwd, "ws_bwd");
    st = twell_route_hybrid(&d, c.dt, &pk, a_save, &hb, nullptr);
    CHECK(st == TWELL_OK, "route_hybrid: %s (%s)", twell_status_str(st), twell_last_error());
    st = twell_ffn_bwd(&d, c.dt, &hb, x, dy, wg, wu, wd, 1e-4f, dx, dwg, dwu, dwd, wsb, z.ws_bwd, nullptr);
    CHECK(st == TWELL_OK, "ffn_bwd: %s (%s)", twell_status_str(st), twell_last_error());
    if (z.ws_bwd > 0) {
      st = twell_ffn_bwd(&d, c.dt, &hb, x, dy, wg, wu, wd, 1e-4f, dx, dwg, dwu, dwd, wsb, z.ws_bwd - 1, nullptr);
      CHECK(st == TWELL_ERR_WORKSPACE, "short backward workspace accepted: %s", twell_status_str(st));
    }
  }
  free_all();
}

}  // namespace

int main() {
  const Case cases[] = {
      // the benchmark workloads, with the benchmark's capacities
      {"tiny fp32 64x128x512", 64, 128, 512, 64, 16, 0, 64, 0, TWELL_F32},
      {"1B-class 4096x2048x5632", 4096, 2048, 5632, 128, 16, 0, 512, 0, TWELL_BF16},
      {"7B-class 16384x4096x11008", 16384, 4096, 11008, 128, 16, 0, 2048, 0, TWELL_BF16},
      {"skewed 8192x4096x14336", 8192, 4096, 14336, 128, 16, 0, 1024, 0, TWELL_BF16},
      {"training 8192x2048x8192", 8192, 2048, 8192, 128, 16, 512, 1024, 1024, TWELL_BF16},
      {"1B-class 1 token S=T_n", 1, 2048, 5632, 128, 128, 0, 64, 0, TWELL_BF16},
      {"7B-class 64 tokens S=T_n", 64, 4096, 11008, 128, 128, 0, 64, 0, TWELL_BF16},
      // edge shapes
      {"empty batch", 0, 256, 1000, 64, 8, 16, 8, 8, TWELL_BF16},
      {"ragged d_ff, S=0", 37, 192, 1000, 64, 0, 12, 40, 40, TWELL_BF16},
      {"S = T_n = 16, fp32", 130, 64, 48, 16, 16, 48, 3, 3, TWELL_F32},
      {"d_model 8192, one row", 1, 8192, 300, 32, 4, 0, 1, 0, TWELL_BF16},
      {"no capacity", 100, 128, 640, 128, 16, 64, 0, 0, TWELL_BF16},
  };
  for (const Case& c : cases) run_case(c);

  g_where = "invalid shapes";
  twell_dims bad{16, 100, 512, 64, 8, 0, 0, 0};  // d_model not a multiple of 64
  twell_sizes z;
  CHECK(twell_query_sizes(&bad, TWELL_BF16, &z) == TWELL_ERR_UNSUPPORTED, "d_model 100 accepted");
  CHECK(std::strlen(twell_last_error()) > 0, "no error message");
  bad = {16, 128, 512, 48, 8, 0, 0, 0};  // tile_n 48
  CHECK(twell_query_sizes(&bad, TWELL_BF16, &z) == TWELL_ERR_UNSUPPORTED, "tile_n 48 accepted");
  bad = {16, 128, 512, 64, 65, 0, 0, 0};  // slots > tile_n
  CHECK(twell_query_sizes(&bad, TWELL_BF16, &z) == TWELL_ERR_INVALID_ARG, "slots > tile_n accepted");
  bad = {-1, 128, 512, 64, 8, 0, 0, 0};
  CHECK(twell_query_sizes(&bad, TWELL_BF16, &z) == TWELL_ERR_INVALID_ARG, "negative N accepted");
  CHECK(twell_query_sizes(nullptr, TWELL_BF16, &z) == TWELL_ERR_INVALID_ARG, "null dims accepted");
  CHECK(twell_n_tiles(nullptr) == -1, "n_tiles(NULL)");
  CHECK(std::strcmp(twell_status_str(99), "TWELL_ERR_UNKNOWN") == 0, "unknown status string");

  // tracing without a device: the calls must fail cleanly or record nothing
  g_where = "trace";
  (void)twell_trace_start(16);
  CHECK(twell_trace_stop() == TWELL_OK, "trace_stop");
  const char* nm = nullptr;
  float ms = 0.f;
  CHECK(twell_trace_get(twell_trace_count(), &nm, &ms) == TWELL_ERR_INVALID_ARG, "trace_get past the end");
  CHECK(twell_trace_start(0) == TWELL_ERR_INVALID_ARG, "trace capacity 0 accepted");

  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host check ok: %d launches checked\n", g_launches);
  return 0;
}
