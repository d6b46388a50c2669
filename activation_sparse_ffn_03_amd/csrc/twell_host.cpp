// Host-only validation and size arithmetic (see twell_host.h).
#include "twell_host.h"

#include <limits>

namespace twell {

namespace {
constexpr int kChunk = 512;  // must match kDenseChunk of the kernels
constexpr int kRows = 32;    // must match kTransposeRows of the kernels

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
}  // namespace

bool bad_ptr(const void* p, size_t bytes) {
  if (bytes == 0) return false;
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) != 0;
}

twell_status check_shape(const twell_dims* d, int dtype, Shape* s, std::string* why) {
  if (d == nullptr) {
    *why = "dims is NULL";
    return TWELL_ERR_INVALID_ARG;
  }
  if (dtype != TWELL_BF16 && dtype != TWELL_F32) {
    *why = "unknown dtype";
    return TWELL_ERR_INVALID_ARG;
  }
  if (d->n_tokens < 0 || d->d_model <= 0 || d->d_ff <= 0 || d->tile_n <= 0 || d->slots < 0 || d->row_cap < 0 ||
      d->ovf_cap < 0 || d->dense_cap < 0) {
    *why = "negative or zero size in dims";
    return TWELL_ERR_INVALID_ARG;
  }
  if (d->slots > d->tile_n) {
    *why = "slots must not exceed tile_n";
    return TWELL_ERR_INVALID_ARG;
  }
  if (d->d_model % 64 != 0) {
    *why = "d_model must be a multiple of 64";
    return TWELL_ERR_UNSUPPORTED;
  }
  const int dmax = dtype == TWELL_BF16 ? 8192 : 4096;
  if (d->d_model > dmax) {
    *why = "d_model above the supported maximum (8192 bf16 / 4096 fp32)";
    return TWELL_ERR_UNSUPPORTED;
  }
  if (d->tile_n != 16 && d->tile_n != 32 && d->tile_n != 64 && d->tile_n != 128) {
    *why = "tile_n must be 16, 32, 64 or 128";
    return TWELL_ERR_UNSUPPORTED;
  }
  if (d->d_ff > 65535) {
    *why = "d_ff above 65535";
    return TWELL_ERR_UNSUPPORTED;
  }
  if (d->row_cap > d->d_ff) {
    *why = "row_cap must not exceed d_ff";
    return TWELL_ERR_INVALID_ARG;
  }
  if (d->n_tokens >= (int64_t(1) << 31) - 1) {
    *why = "n_tokens must fit a 32-bit row index";
    return TWELL_ERR_UNSUPPORTED;
  }
  s->N = d->n_tokens;
  s->D = d->d_model;
  s->F = d->d_ff;
  s->tile_n = d->tile_n;
  s->slots = d->slots;
  s->row_cap = d->row_cap;
  s->ovf_cap = d->ovf_cap;
  s->dense_cap = d->dense_cap;
  s->n_tiles = (d->d_ff + d->tile_n - 1) / d->tile_n;
  s->esz = dtype == TWELL_BF16 ? 2 : 4;
  s->G = (d->d_ff + kChunk - 1) / kChunk;
  s->nrb = (int)((d->n_tokens + kRows - 1) / kRows);
  s->nnz_max = d->n_tokens * (int64_t)d->row_cap + (int64_t)d->dense_cap * d->d_ff;
  if (s->nnz_max >= (int64_t(1) << 31) - 1) {
    *why = "n_tokens*row_cap + dense_cap*d_ff must stay below 2^31 entries";
    return TWELL_ERR_CAPACITY;
  }
  if (d->ovf_cap > (1 << 24) || d->dense_cap > (1 << 24)) {
    *why = "ovf_cap / dense_cap above 2^24 rows";
    return TWELL_ERR_UNSUPPORTED;
  }
  return TWELL_OK;
}

int up_passes(const Shape& s) {
  const int parts = s.n_tiles < 8 ? s.n_tiles : 8;
  if (parts <= 0) return 1;
  const int64_t rows = ((int64_t)s.F + parts - 1) / parts;
  const int64_t wave_elems = 64 * (16 / s.esz);  // one 16-byte load per lane
  int nq = 1;
  while (rows * (s.D / nq) * s.esz > (4ll << 20) && s.D % (2 * nq * wave_elems) == 0) nq *= 2;
  return nq;
}

FwdLayout fwd_layout(const Shape& s) {
  FwdLayout L{};
  const size_t entries = (size_t)s.N * s.n_tiles * s.slots;
  const int nq = up_passes(s);
  L.offs = 0;
  L.zlist = align_up((size_t)s.N * 4);
  L.upart = L.zlist + align_up(entries * 8);
  L.uslot = L.upart + (nq > 1 ? align_up((size_t)nq * entries * 4) : 0);
  L.part = L.uslot + (nq > 1 ? align_up(entries * 4) : 0);
  L.zov = L.part + align_up((size_t)s.ovf_cap * s.G * s.D * 4);
  L.gbase = L.zov + (s.esz == 2 ? align_up((size_t)2 * s.ovf_cap * dense_z_stride(s.F) * 2) : 0);
  const size_t groups = (size_t)(s.n_tiles + kUpGroupTiles - 1) / kUpGroupTiles;
  const size_t nrb4 = ((size_t)s.N + 3) / 4, nwg = ((size_t)s.N + 255) / 256;
  L.rb_order = L.gbase + align_up(groups * (size_t)s.N * 4);
  L.rb_code = L.rb_order + align_up(nrb4 * 4);
  L.rb_hist = L.rb_code + align_up(nrb4 * 4);
  L.total = L.rb_hist + nwg * 16 * 4;
  return L;
}

size_t fwd_ws_bytes(const Shape& s) { return s.N == 0 ? 0 : fwd_layout(s).total; }

BwdLayout bwd_layout(const Shape& s) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t nnz = (size_t)s.nnz_max;
  L.row_ptr = take(((size_t)s.N + 1 + s.dense_cap) * 4);
  L.dense_pos = take((size_t)s.N * 4);
  L.pair_col = take(nnz * 4);
  L.coef = take(nnz * 16);
  L.csc_pair = take(nnz * 4);
  L.csc_row = take(nnz * 4);
  L.col_ptr = take(((size_t)s.F + 1) * 4);
  L.blk_cnt = take((size_t)2 * s.nrb * s.F * 4);
  L.grp_off = take((size_t)s.dense_cap * s.G * 4);
  L.egrp = take(((size_t)(s.F + 511) / 512 + 1) * s.N * 4);
  const bool dm = bwd_dense_mfma(s);
  const size_t dc = (size_t)s.dense_cap;
  L.dza = take(dm ? 2 * dc * s.F * 4 : 0);
  L.dadg = take(dm ? 4 * dc * dense_z_stride(s.F) * 2 : 0);
  L.dxpart = take(dm ? dc * s.G * s.D * 4 : 0);
  L.total = off;
  return L;
}

void compute_sizes(const Shape& s, twell_sizes* o) {
  const size_t N = (size_t)s.N, nt = (size_t)s.n_tiles, S = (size_t)s.slots, K = (size_t)s.row_cap;
  const size_t F = (size_t)s.F, e = (size_t)s.esz;
  o->vals = nt * S * N * e;
  o->cols = nt * S * N * 2;
  o->counts = nt * N * 2;
  o->ovf_flag = N;
  o->ovf_rows = (size_t)s.ovf_cap * 4;
  o->ovf_h = (size_t)s.ovf_cap * F * e;
  o->n_ovf = 4;
  o->status = 4;
  o->ell_vals = K * N * e;
  o->ell_cols = K * N * 4;
  o->ell_a = K * N * 4;
  o->row_nnz = N * 4;
  o->is_dense = N;
  o->dense_rows = (size_t)s.dense_cap * 4;
  o->dense_h = (size_t)s.dense_cap * F * e;
  o->n_dense = 4;
  o->a_save = nt * S * N * 4;
  o->ws_fwd = fwd_ws_bytes(s);
  o->ws_bwd = bwd_layout(s).total;
  o->ws_gate = (s.esz == 2 && N > 0 && N <= TWELL_SMALL_BATCH_MAX) ? N * F * 4 : 0;
}

}  // namespace twell
