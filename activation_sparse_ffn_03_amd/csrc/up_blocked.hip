// Up projection of large batches with weight-row reuse through LDS.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// the inference kernel takes the activations in TwELL and does the up
// projection (then the down projection) without writing the hidden state.
// Here: a = x_i . W_up^T[c] at every packed entry (i, c), z = h * a into the
// token's (column, z) list (the sparse intermediate the down projection reads).
//
// Gathering one W_up row per entry moves nnz * 2 * d_model bytes out of L2,
// about 15 GB on a 16384 x 4096 x 11008 layer at 1 % density. The blocked
// sampled product of blocked_sddmm.h (512 tokens x a group of kUpGroupTiles
// TwELL tiles per workgroup, x and W_up staged through LDS) does it with
// (N / 512 + F / C) * d_model * 2 bytes of L2 reads per row pair instead.
//
// up_rows, a small pass before, gives every token its list length (-1 for an
// overflow row, which the dense-row path handles) and the list position of
// each tile group's first entry, and with order_blocks the down projection's
// heaviest-first order of 4-row blocks (block_order.h).
#include "block_order.h"
#include "blocked_sddmm.h"
#include "row_ops.h"
#include "twell_host.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int kTG = kUpGroupTiles;

// Thread per token: list length (offs, -1 for an overflow row) and the list
// position of every kTG-tile group's first entry (gbase); with rb_code set,
// also the down projection's block classes (block_order.h; overflow rows
// weigh nothing, the dense-row path takes them).
__global__ __launch_bounds__(256) void up_rows(const uint16_t* __restrict__ counts, int64_t N, int n_tiles, int slots,
                                               int32_t* __restrict__ offs, int32_t* __restrict__ gbase,
                                               int32_t* __restrict__ rb_code, int32_t* __restrict__ rb_hist) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int len = 0;
  if (i < N) {
    int run = 0;
    bool ovf = false;
#pragma unroll 8
    for (int j = 0; j < n_tiles; ++j) {
      if (j % kTG == 0) gbase[(size_t)(j / kTG) * N + i] = run;
      const int c = counts[(size_t)j * N + i];
      ovf |= c > slots;
      run += min(c, slots);
    }
    offs[i] = ovf ? -1 : run;
    len = ovf ? 0 : run;
  }
  if (rb_code != nullptr) blkord::block_classes(len, N, rb_code, rb_hist);  // uniform branch
}

// The forward's pattern: the packed TwELL entries of the non-overflow rows,
// tile by tile and slot by slot (ascending columns); results into the token's
// (column, z) list and, for training, a at the entry's TwELL slot.
struct UpPolicy {
  FwdArgs a;
  static constexpr int kSub = kTG;
  __device__ const uint16_t* rows_a() const { return reinterpret_cast<const uint16_t*>(a.x); }
  __device__ const uint16_t* rows_b() const { return reinterpret_cast<const uint16_t*>(a.w_up); }
  __device__ int64_t n() const { return a.N; }
  __device__ int d() const { return a.D; }
  __device__ int f() const { return a.F; }
  __device__ int c0(int g) const { return g * kTG * a.tile_n; }
  __device__ bool own(int64_t i) const { return a.offs[i] >= 0; }
  __device__ int count(int64_t i, int g, int s) const {
    const int j = g * kTG + s;
    return j < a.n_tiles ? min((int)a.counts[(size_t)j * a.N + i], a.slots) : 0;
  }
  __device__ void entry(int64_t i, int g, int s, int k, uint32_t& cg, uint32_t& key, uint32_t& hb) const {
    const size_t pos = ((size_t)(g * kTG + s) * a.slots + k) * a.N + i;
    cg = (uint32_t)(s * a.tile_n + ((int)a.cols[pos] & (a.tile_n - 1)));  // tile_n is a power of two
    key = (uint32_t)k;
    hb = (uint32_t)reinterpret_cast<const uint16_t*>(a.vals)[pos] << 16;
  }
  __device__ int base(int64_t i, int g) const { return a.gbase[(size_t)g * a.N + i]; }
  __device__ void store(int64_t i, int g, uint32_t cg, uint32_t key, float h, int pos, float v) const {
    const size_t L = (size_t)a.n_tiles * a.slots;
    a.zlist[(size_t)i * L + pos] = make_uint2((uint32_t)(c0(g) + (int)cg), __float_as_uint(h * v));
    if (a.a_save) a.a_save[((size_t)(g * kTG + (int)cg / a.tile_n) * a.slots + key) * a.N + i] = v;
  }
};

using UpBlk = blk::Default;

__global__ __launch_bounds__(UpBlk::NT, 1) void ffn_up_blocked(FwdArgs a, int n_groups, int64_t n_tblocks) {
  blk::sddmm_block<UpBlk>(UpPolicy{a}, n_groups, n_tblocks);
}

}  // namespace

// Only where the (token block, group) pairs fill the CUs: with fewer (the
// 4096 x 2048 x 5632 forward has 8 x 11) the blocked form took 132 us against
// 67 us for the wave-per-token kernel.
bool up_blocked_applies(const FwdArgs& a) {
  const int64_t pairs = ((a.N + UpBlk::T - 1) / UpBlk::T) * ((a.n_tiles + kTG - 1) / kTG);
  return a.is_bf16 && a.N > 64 && a.D % 32 == 0 && a.tile_n <= 128 && a.slots < 1024 && pairs >= blk::kCus;
}

// The ordering kernel has one thread per up_rows workgroup.
bool down_order_applies(const FwdArgs& a) {
  return up_blocked_applies(a) && a.rb_order != nullptr && a.rb_code != nullptr && a.rb_hist != nullptr &&
         blkord::order_fits(a.N);
}

hipError_t launch_up_blocked(const FwdArgs& a, hipStream_t s) {
  if (!up_blocked_applies(a)) return hipErrorInvalidValue;
  const bool order = down_order_applies(a);
  TWELL_LAUNCH("up_rows", up_rows, dim3((unsigned)((a.N + 255) / 256)), 256, 0, s, a.counts, a.N, a.n_tiles, a.slots,
               a.offs, a.gbase, order ? a.rb_code : nullptr, a.rb_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (order) {
    TWELL_LAUNCH("order_blocks", blkord::order_blocks, 1, 1024, 0, s, a.N, a.rb_code, a.rb_hist, a.rb_order);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int n_groups = (a.n_tiles + kTG - 1) / kTG;
  const int64_t ntb = (a.N + UpBlk::T - 1) / UpBlk::T;
  TWELL_LAUNCH("ffn_up_blocked", ffn_up_blocked, dim3((unsigned)blk::grid_blocks(ntb, n_groups)), UpBlk::NT, 0, s, a,
               n_groups, ntb);
  return hipGetLastError();
}

}  // namespace twell
