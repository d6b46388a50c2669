// Up projection of large batches with weight-row reuse through LDS.
//
// "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me), second paragraph:
// the inference kernel takes the activations in TwELL and does the up
// projection (then the down projection) without writing the hidden state.
// Here: a = x_i . W_up^T[c] at every packed entry (i, c), z = h * a into the
// token's (column, z) list (the sparse intermediate the down projection reads).
//
// Gathering one W_up row per entry moves nnz * 2 * d_model bytes out of L2,
// about 15 GB on a 16384 x 4096 x 11008 layer at 1 % density. A workgroup here
// owns 512 tokens and a group of kUpGroupTiles TwELL tiles (C columns) and
// walks d_model in 32-element stages: each stage brings the 512 x rows and
// the group's C W_up rows into LDS once (global_load_lds, double buffered),
// so a staged W_up row serves 512 * p entries at density p and a staged x row
// C * p, and L2 delivers (N / 512 + F / C) * d_model * 2 bytes per row pair
// instead of one W_up row per entry.
//
// Lanes own entries, not tokens: the block's entries are split evenly over
// the threads in runs of consecutive entries, so the load is even whatever
// the per-token counts are. Each entry reads its W_up row (and, when it
// starts a token, the x row) from LDS per stage and sums 16 v_dot2_f32_bf16
// in a fixed order (ascending d_model), so the result is deterministic. A block with more entries than one pass holds takes
// further passes over d_model.
//
// up_rows, a small pass before, gives every token its list length (-1 for an
// overflow row, which the dense-row path handles) and the list position of
// each tile group's first entry.
#include "row_ops.h"
#include "twell_host.h"
#include "twell_kernels.h"
#include "twell_trace.h"

namespace twell {
namespace {

constexpr int kTG = kUpGroupTiles;

// Thread per token: list length (offs, -1 for an overflow row) and the list
// position of every kTG-tile group's first entry (gbase).
__global__ __launch_bounds__(256) void up_rows(const uint16_t* __restrict__ counts, int64_t N, int n_tiles, int slots,
                                               int32_t* __restrict__ offs, int32_t* __restrict__ gbase) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
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
}

// Super-tile of the workgroup order: token blocks x column groups that one
// XCD runs at a time (32 workgroups, one per CU of the XCD).
constexpr int kSupT = 4, kSupG = 8;

template <int T_, int ST_, int EPT_>
struct UpBlkCfg {
  static constexpr int T = T_, ST = ST_, EPT = EPT_;
  static constexpr int NT = 512, NW = NT / 64;
  static constexpr int KU = 2;                     // entries whose row reads are issued together
  static constexpr int ROWB = 64;                  // bytes of a staged row: 32 bf16 of d_model
  static constexpr int CMAX = kUpGroupTiles * 128; // columns of a group at the widest tile
  static constexpr int STAGE = (T + CMAX) * ROWB;  // x rows, then W_up rows
  static constexpr int RING = ST * STAGE;
  static constexpr int CAP = NT * EPT;             // entries of one pass
  static constexpr int XG = T / 16 / NW;           // 1 KB DMA groups of x per wave and stage
  static constexpr int WG = CMAX / 16 / NW;        // of W_up
  static constexpr int META = 2 * (T + 1) * 4;     // each token's first list index and list base
  static constexpr int LDS = RING + META + CAP * 8;
  static_assert(T % 128 == 0 && T <= NT, "one token per thread while listing, whole DMA groups per wave");
  static_assert(EPT % KU == 0, "whole read batches");
  static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// Inclusive sum over the 512 threads of the block (wsum: LDS for the 8 wave
// totals); *total gets the block's sum.
__device__ __forceinline__ int block_scan_512(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int s = wsum[w];
    before += w < wave ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// One workgroup: T tokens x one group of kUpGroupTiles TwELL tiles. The
// block's entries are listed token-major (token, tile, slot: the order of the
// token's list) and split into 512 runs of consecutive entries, one per
// thread, so every thread has the same number (one more for some) whatever
// the per-token counts, and a thread's entries mostly share a token. Per
// 32-element stage of d_model the T x rows and the group's W_up rows come
// into LDS by DMA (double buffered); each entry then reads its W_up row there
// (and, when it starts a token, the token's x row, kept in registers for the
// next entries) and takes 16 v_dot2_f32_bf16. Lanes start at different
// 16-byte chunks of their rows (chunk (q + lane) & 3 at step q), which
// spreads reads of random rows over the LDS banks (measured on gfx950: a wave
// reading 16 bytes per lane from random 64-byte rows takes about 5.4 ns per
// CU this way, 10.6 ns with every lane on the same chunk, 3.3 ns for a
// broadcast).
template <class C>
__global__ __launch_bounds__(C::NT, 1) void ffn_up_blocked(FwdArgs a, int n_groups, int64_t n_tblocks) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  __shared__ int wsum[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroup b runs on XCD b % 8. The (token block, group) pairs are cut
  // into super-tiles of kSupT token blocks x kSupG groups, dealt to the XCDs
  // round-robin; the 32 workgroups an XCD runs at a time are one super-tile,
  // so each staged x chunk is read by kSupG of them and each W_up chunk by
  // kSupT, at about the same time, out of the XCD's L2.
  const int xcd = blockIdx.x % 8;
  const int64_t kb = blockIdx.x / 8;
  const int64_t st = xcd + 8 * (kb / (kSupT * kSupG));
  const int in = (int)(kb % (kSupT * kSupG));
  const int64_t sup_g = (n_groups + kSupG - 1) / kSupG;
  const int64_t tb = (st % ((n_tblocks + kSupT - 1) / kSupT)) * kSupT + in / kSupG;
  const int64_t gg = (st / ((n_tblocks + kSupT - 1) / kSupT)) * kSupG + in % kSupG;
  if (tb >= n_tblocks || gg >= n_groups || st >= sup_g * ((n_tblocks + kSupT - 1) / kSupT)) return;
  const int g = (int)gg;
  const int64_t i0 = tb * C::T;
  const int64_t N = a.N;
  const int S = a.slots, Tn = a.tile_n, D = a.D;
  const int j0 = g * kUpGroupTiles, ntg = min(kUpGroupTiles, a.n_tiles - j0);
  const int c0 = j0 * Tn;
  const int ntok = (int)min<int64_t>(C::T, N - i0);
  const size_t L = (size_t)a.n_tiles * S;
  const uint16_t* __restrict__ xb = reinterpret_cast<const uint16_t*>(a.x);
  const uint16_t* __restrict__ wb = reinterpret_cast<const uint16_t*>(a.w_up);
  const uint16_t* __restrict__ vals = reinterpret_cast<const uint16_t*>(a.vals);

  int* tok_first = reinterpret_cast<int*>(smem + C::RING);  // [T + 1] first list index of each token
  int* tok_base = tok_first + (C::T + 1);                    // [T] list position of its first entry here
  uint2* list = reinterpret_cast<uint2*>(smem + C::RING + C::META);

  // DMA sources of this wave: x rows past the batch and W_up rows past d_ff
  // read row 0 (never used by an entry). A 1 KB group is 16 rows x 4 chunks;
  // lane l moves chunk l & 3 of row l >> 2 of its group.
  const char* src[C::XG + C::WG];
  uint32_t dst[C::XG + C::WG];
  {
    const int rin = lane >> 2, q = lane & 3;
#pragma unroll
    for (int t = 0; t < C::XG; ++t) {
      const int row = (wave + C::NW * t) * 16 + rin;
      const int64_t tok = i0 + row < N ? i0 + row : 0;
      src[t] = reinterpret_cast<const char*>(xb + tok * D) + q * 16;
      dst[t] = (uint32_t)((row - rin) * C::ROWB);
    }
#pragma unroll
    for (int t = 0; t < C::WG; ++t) {
      const int row = (wave + C::NW * t) * 16 + rin;
      const int col = c0 + row < a.F ? c0 + row : 0;
      src[C::XG + t] = reinterpret_cast<const char*>(wb + (int64_t)col * D) + q * 16;
      dst[C::XG + t] = (uint32_t)((C::T + row - rin) * C::ROWB);
    }
  }
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(smem));
  const int KT = D / 32;
  auto issue = [&](int kt) {
    const uint32_t sb = lds0 + (uint32_t)((kt % C::ST) * C::STAGE);
#pragma unroll
    for (int t = 0; t < C::XG + C::WG; ++t) dma_16B(src[t] + (size_t)kt * 64, sb + dst[t]);
  };

  // ---- the block's entries: thread t lists token i0 + t (none for an overflow row)
  int cnt[kUpGroupTiles];
  int tot = 0, base = 0;
  {
    const int64_t i = i0 + tid;
    const bool own = tid < ntok && a.offs[i < N ? i : 0] >= 0;
#pragma unroll
    for (int tj = 0; tj < kUpGroupTiles; ++tj) {
      const int c = own && tj < ntg ? (int)a.counts[(size_t)(j0 + tj) * N + i] : 0;
      cnt[tj] = min(c, S);
      tot += cnt[tj];
    }
    if (own) base = a.gbase[(size_t)g * N + i];
  }
  int total;
  const int first = block_scan_512(tot, wsum, &total) - tot;
  if (tid < C::T) {
    tok_first[tid] = first;
    tok_base[tid] = base;
  }
  for (int pass0 = 0; pass0 < total; pass0 += C::CAP) {
    // prefetch the first stages while the list is built
#pragma unroll
    for (int st = 0; st < C::ST - 1; ++st)
      if (st < KT) issue(st);
    // list entries [pass0, pass0 + CAP): (token | column in group << 10 | slot << 22, h as fp32 bits)
    {
      const int64_t i = i0 + tid;
      int e = first;
#pragma unroll
      for (int tj = 0; tj < kUpGroupTiles; ++tj) {
        const int n = cnt[tj];
        const int nmax = wave_max_int(n);
        for (int sl = 0; sl < nmax; ++sl) {
          const int le = e + sl - pass0;
          if (sl < n && le >= 0 && le < C::CAP) {
            const size_t pos = ((size_t)(j0 + tj) * S + sl) * N + i;
            const int cg = tj * Tn + ((int)a.cols[pos] & (Tn - 1));  // tile_n is a power of two
            list[le] = make_uint2((uint32_t)tid | ((uint32_t)cg << 10) | ((uint32_t)sl << 22),
                                  (uint32_t)vals[pos] << 16);
          }
        }
        e += n;
      }
    }
    __syncthreads();
    // this thread's entries of the pass: EPT consecutive ones of the
    // token-major list, so they mostly share a token and its x chunks stay
    // in registers from one entry to the next (lanes past the pass read row 0
    // and drop the result)
    const int npass = min(C::CAP, total - pass0);
    const int first_le = tid * npass / C::NT;  // an even split: floor or ceil of npass / NT each
    const int nmine = (tid + 1) * npass / C::NT - first_le;
    const int nmw = wave_max_int(nmine);
    uint2 desc[C::EPT];
    uint32_t xo[C::EPT], wo[C::EPT];
    uint32_t newx = 0;  // bit k: entry k starts a token (its x row is read)
    float acc[C::EPT];
#pragma unroll
    for (int k = 0; k < C::EPT; ++k) {
      desc[k] = k < nmine ? list[first_le + k] : make_uint2(0u, 0u);
      xo[k] = (desc[k].x & 1023u) * C::ROWB;
      wo[k] = (uint32_t)(C::T + ((desc[k].x >> 10) & 4095u)) * C::ROWB;
      if (k < nmine && (k == 0 || xo[k] != xo[k - 1])) newx |= 1u << k;
      acc[k] = 0.f;
    }
    const int rot = lane & 3;

    for (int kt = 0; kt < KT; ++kt) {
      if (C::ST >= 3 && kt + 1 < KT) wait_vmcnt<(C::XG + C::WG)>();
      else wait_vmcnt<0>();
      lds_barrier();  // stage kt is in LDS for every wave; the buffer refilled below is no longer read
      if (kt + C::ST - 1 < KT) issue(kt + C::ST - 1);
      const char* stg = smem + (kt % C::ST) * C::STAGE;
      u32x4_t xcur[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) xcur[q] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int k0 = 0; k0 < C::EPT; k0 += C::KU) {
        if (k0 < nmw) {
          u32x4_t xv[C::KU][4], wv[C::KU][4];
#pragma unroll
          for (int u = 0; u < C::KU; ++u) {
            const int k = k0 + u;
            if (newx & (1u << k)) {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                xv[u][q] = *reinterpret_cast<const u32x4_t*>(stg + xo[k] + ((q + rot) & 3) * 16);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
              wv[u][q] = *reinterpret_cast<const u32x4_t*>(stg + wo[k] + ((q + rot) & 3) * 16);
          }
#pragma unroll
          for (int u = 0; u < C::KU; ++u) {
            const int k = k0 + u;
            const bool nx = (newx >> k) & 1u;
#pragma unroll
            for (int q = 0; q < 4; ++q) xcur[q] = nx ? xv[u][q] : xcur[q];
            float s = acc[k];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              s = dot2_bf16(xcur[q].x, wv[u][q].x, s);
              s = dot2_bf16(xcur[q].y, wv[u][q].y, s);
              s = dot2_bf16(xcur[q].z, wv[u][q].z, s);
              s = dot2_bf16(xcur[q].w, wv[u][q].w, s);
            }
            acc[k] = s;
          }
        }
      }
    }
    // z = h * a into the token's list; a at the entry's TwELL slot (training)
#pragma unroll
    for (int k = 0; k < C::EPT; ++k) {
      if (k < nmine) {
        const int le = first_le + k;
        const int t = (int)(desc[k].x & 1023u), cg = (int)((desc[k].x >> 10) & 4095u), sl = (int)(desc[k].x >> 22);
        const int64_t i = i0 + t;
        const int pos = tok_base[t] + (pass0 + le - tok_first[t]);
        const float av = acc[k];
        a.zlist[(size_t)i * L + pos] =
            make_uint2((uint32_t)(c0 + cg), __float_as_uint(__uint_as_float(desc[k].y) * av));
        if (a.a_save) a.a_save[((size_t)(j0 + cg / Tn) * S + sl) * N + i] = av;
      }
    }
    __syncthreads();  // the list and the ring are refilled by the next pass
  }
}

// Configuration: 512 tokens x 4 tiles per workgroup, two stages of 64 KB,
// up to 3072 entries per pass (2621 expected at 1 % density).
using UpBlk = UpBlkCfg<512, 2, 6>;

}  // namespace

bool up_blocked_applies(const FwdArgs& a) { return a.is_bf16 && a.N > 64 && a.D % 32 == 0 && a.tile_n <= 128; }

hipError_t launch_up_blocked(const FwdArgs& a, hipStream_t s) {
  if (!up_blocked_applies(a)) return hipErrorInvalidValue;
  TWELL_LAUNCH("up_rows", up_rows, dim3((unsigned)((a.N + 255) / 256)), 256, 0, s, a.counts, a.N, a.n_tiles, a.slots,
               a.offs, a.gbase);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_groups = (a.n_tiles + kTG - 1) / kTG;
  const int64_t ntb = (a.N + UpBlk::T - 1) / UpBlk::T;
  const int64_t n_super = ((ntb + kSupT - 1) / kSupT) * ((n_groups + kSupG - 1) / kSupG);
  const int64_t blocks = 8 * ((n_super + 7) / 8) * (kSupT * kSupG);
  TWELL_LAUNCH("ffn_up_blocked", ffn_up_blocked<UpBlk>, dim3((unsigned)blocks), UpBlk::NT, 0, s, a, n_groups, ntb);
  return hipGetLastError();
}

}  // namespace twell
