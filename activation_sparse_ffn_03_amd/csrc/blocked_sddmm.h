// Sampled dense-dense product through LDS: out(i, c) = A_i . B_c (A [N][D],
// B [F][D], both bf16 and d_model-contiguous) at the active entries (i, c) of
// a sparse pattern, with weight-row reuse.
//
// A workgroup owns T tokens and a group of up to kGroupCols columns and walks
// d_model in 32-element stages: each stage brings the T rows of A and the
// group's rows of B into LDS once (global_load_lds, double buffered), so a
// staged B row serves T * p entries at density p and a staged A row C * p,
// and L2 delivers (N / T + F / C) * d_model * 2 bytes per row pair instead of
// one B row per entry.
//
// Lanes own entries, not tokens: the block's entries are listed token-major
// (the order of a token's own entries) and split evenly over the threads in
// runs of consecutive entries, so the load is even whatever the per-token
// counts are. Each entry reads its B row (and, when it starts a token, the A
// row, kept in registers for the next entries) from LDS per stage and sums
// 16 v_dot2_f32_bf16 in a fixed order (ascending d_model), so the result is
// deterministic. Lanes start at different 16-byte chunks of their rows
// (chunk (q + lane) & 3 at step q), which spreads reads of random rows over
// the LDS banks (measured on gfx950: a wave reading 16 bytes per lane from
// random 64-byte rows takes about 5.4 ns per CU this way, 10.6 ns with every
// lane on the same chunk, 3.3 ns for a broadcast). A block with more entries
// than one pass holds takes further passes over d_model.
//
// What the pattern is and where results go is a policy P (the forward's
// TwELL tiles, the backward's row-ELL):
//   const uint16_t* rows_a() const, rows_b() const
//   int64_t n() const; int d() const; int f() const
//   int c0(int g) const                        first column of group g
//   bool own(int64_t i) const                  token i's entries are in the pattern
//   static constexpr int kSub                  sub-ranges per token and group
//   int count(int64_t i, int g, int s) const   entries of token i in sub-range s
//   void entry(int64_t i, int g, int s, int k, uint32_t& cg, uint32_t& key, uint32_t& hbits) const
//                                              its k-th: column - c0(g) (< 4096),
//                                              a key (< 1024) handed back to store,
//                                              the stored activation as fp32 bits
//   int base(int64_t i, int g) const          output position of the token's
//                                              first entry of the group
//   void store(int64_t i, int g, uint32_t cg, uint32_t key, float h, int pos, float v) const
#pragma once

#include "twell_device.h"

namespace twell {
namespace blk {

constexpr int kGroupCols = 512;  // columns of a group at most
constexpr int kCus = 256;        // compute units of an MI355X: the blocked form needs this many workgroups

// Super-tile of the workgroup order: token blocks x column groups that one
// XCD runs at a time (32 workgroups, one per CU of the XCD).
constexpr int kSupT = 4, kSupG = 8;

template <int T_, int ST_, int EPT_>
struct Cfg {
  static constexpr int T = T_, ST = ST_, EPT = EPT_;
  static constexpr int NT = 512, NW = NT / 64;
  static constexpr int KU = 2;                     // entries whose row reads are issued together
  static constexpr int ROWB = 64;                  // bytes of a staged row: 32 bf16 of d_model
  static constexpr int CMAX = kGroupCols;
  static constexpr int STAGE = (T + CMAX) * ROWB;  // A rows, then B rows
  static constexpr int RING = ST * STAGE;
  static constexpr int CAP = NT * EPT;             // entries of one pass
  static constexpr int XG = T / 16 / NW;           // 1 KB DMA groups of A per wave and stage
  static constexpr int WG = CMAX / 16 / NW;        // of B
  static constexpr int META = 2 * (T + 1) * 4;     // each token's first list index and output base
  static constexpr int LDS = RING + META + CAP * 8;
  static_assert(T % 128 == 0 && T <= NT, "one token per thread while listing, whole DMA groups per wave");
  static_assert(EPT % KU == 0, "whole read batches");
  static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// 512 tokens x 512 columns per workgroup, two stages of 64 KB, up to 3072
// entries per pass (2621 expected at 1 % density).
using Default = Cfg<512, 2, 6>;

// Workgroups of a grid over n_tblocks token blocks x n_groups column groups.
inline int64_t grid_blocks(int64_t n_tblocks, int n_groups) {
  const int64_t n_super = ((n_tblocks + kSupT - 1) / kSupT) * ((n_groups + kSupG - 1) / kSupG);
  return 8 * ((n_super + 7) / 8) * (kSupT * kSupG);
}

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

// The workgroup body (called by a __global__ of launch bounds (C::NT, 1)).
template <class C, class P>
__device__ __forceinline__ void sddmm_block(const P& p, int n_groups, int64_t n_tblocks) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  __shared__ int wsum[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroup b runs on XCD b % 8. The (token block, group) pairs are cut
  // into super-tiles of kSupT token blocks x kSupG groups, dealt to the XCDs
  // round-robin; the 32 workgroups an XCD runs at a time are one super-tile,
  // so each staged A chunk is read by kSupG of them and each B chunk by
  // kSupT, at about the same time, out of the XCD's L2.
  const int xcd = blockIdx.x % 8;
  const int64_t kb = blockIdx.x / 8;
  const int64_t st = xcd + 8 * (kb / (kSupT * kSupG));
  const int in = (int)(kb % (kSupT * kSupG));
  const int64_t sup_g = (n_groups + kSupG - 1) / kSupG;
  const int64_t tsup = (n_tblocks + kSupT - 1) / kSupT;
  const int64_t tb = (st % tsup) * kSupT + in / kSupG;
  const int64_t gg = (st / tsup) * kSupG + in % kSupG;
  if (tb >= n_tblocks || gg >= n_groups || st >= sup_g * tsup) return;
  const int g = (int)gg;
  const int64_t i0 = tb * C::T;
  const int64_t N = p.n();
  const int D = p.d(), F = p.f();
  const int c0 = p.c0(g);
  const int ntok = (int)min<int64_t>(C::T, N - i0);

  int* tok_first = reinterpret_cast<int*>(smem + C::RING);  // [T + 1] first list index of each token
  int* tok_base = tok_first + (C::T + 1);                    // [T] output position of its first entry here
  uint2* list = reinterpret_cast<uint2*>(smem + C::RING + C::META);

  // DMA sources of this wave: A rows past the batch and B rows past d_ff read
  // row 0 (never used by an entry). A 1 KB group is 16 rows x 4 chunks; lane l
  // moves chunk l & 3 of row l >> 2 of its group.
  const char* src[C::XG + C::WG];
  uint32_t dst[C::XG + C::WG];
  {
    const int rin = lane >> 2, q = lane & 3;
#pragma unroll
    for (int t = 0; t < C::XG; ++t) {
      const int row = (wave + C::NW * t) * 16 + rin;
      const int64_t tok = i0 + row < N ? i0 + row : 0;
      src[t] = reinterpret_cast<const char*>(p.rows_a() + tok * D) + q * 16;
      dst[t] = (uint32_t)((row - rin) * C::ROWB);
    }
#pragma unroll
    for (int t = 0; t < C::WG; ++t) {
      const int row = (wave + C::NW * t) * 16 + rin;
      const int col = c0 + row < F ? c0 + row : 0;
      src[C::XG + t] = reinterpret_cast<const char*>(p.rows_b() + (int64_t)col * D) + q * 16;
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

  // ---- the block's entries: thread t lists token i0 + t
  int cnt[P::kSub];
  int tot = 0, base = 0;
  {
    const int64_t i = i0 + tid;
    const bool mine = tid < ntok && p.own(i);
#pragma unroll
    for (int s = 0; s < P::kSub; ++s) {
      cnt[s] = mine ? p.count(i, g, s) : 0;
      tot += cnt[s];
    }
    if (mine && tot > 0) base = p.base(i, g);
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
    // list entries [pass0, pass0 + CAP): (token | column in group << 10 | key << 22, h as fp32 bits)
    {
      const int64_t i = i0 + tid;
      int e = first;
#pragma unroll
      for (int s = 0; s < P::kSub; ++s) {
        const int n = cnt[s];
        const int nmax = wave_max_int(n);
        for (int k = 0; k < nmax; ++k) {
          const int le = e + k - pass0;
          if (k < n && le >= 0 && le < C::CAP) {
            uint32_t cg, key, hb;
            p.entry(i, g, s, k, cg, key, hb);
            list[le] = make_uint2((uint32_t)tid | (cg << 10) | (key << 22), hb);
          }
        }
        e += n;
      }
    }
    __syncthreads();
    // this thread's entries of the pass: EPT consecutive ones of the
    // token-major list, so they mostly share a token and its A chunks stay in
    // registers from one entry to the next (lanes past the pass read row 0 and
    // drop the result)
    const int npass = min(C::CAP, total - pass0);
    const int first_le = tid * npass / C::NT;  // an even split: floor or ceil of npass / NT each
    const int nmine = (tid + 1) * npass / C::NT - first_le;
    const int nmw = wave_max_int(nmine);
    uint2 desc[C::EPT];
    uint32_t xo[C::EPT], wo[C::EPT];
    uint32_t newx = 0;  // bit k: entry k starts a token (its A row is read)
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
    // results, at the token's output base + the entry's rank among its entries of the group
#pragma unroll
    for (int k = 0; k < C::EPT; ++k) {
      if (k < nmine) {
        const int le = first_le + k;
        const int t = (int)(desc[k].x & 1023u);
        const int pos = tok_base[t] + (pass0 + le - tok_first[t]);
        p.store(i0 + t, g, (desc[k].x >> 10) & 4095u, desc[k].x >> 22, __uint_as_float(desc[k].y), pos, acc[k]);
      }
    }
    __syncthreads();  // the list and the ring are refilled by the next pass
  }
}

}  // namespace blk
}  // namespace twell
