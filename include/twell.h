/*
 * libtwell — activation-sparse ReLU-gated FFN with TwELL-packed activations,
 * for AMD Instinct MI355X (gfx950).
 *
 * The block computed is  y = (ReLU(x·W_gate − t) ⊙ (x·W_up))·W_down  where the
 * gate output is 95–99% zeros. The pages this follows describe three stages
 * ("Sakana AI and NVIDIA present TwELL", edge.aivizor.me, second paragraph):
 *   1. the gate projection packs its ReLU output into TwELL — d_ff cut into
 *      horizontal tiles of width T_n matched to the matmul tile, nonzeros
 *      packed locally inside each tile — in the GEMM epilogue;
 *   2. one fused kernel reads TwELL and does the up and down projections
 *      without writing the hidden state to global memory;
 *   3. for training, a hybrid format routes each row either to a compact ELL
 *      matrix or to a dense backup for overflows.
 * TwELL means tile-wise ELLPACK ("How TwELL by Sakana AI and NVIDIA
 * Accelerates LLMs by 20%", aimodelsnavi.com, "Technical Explanation" and
 * "Core of TwELL").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - N = n_tokens, D = d_model, F = d_ff, T_n = tile_n, S = slots,
 *    K = row_cap, n_t = ceil(F / T_n).
 *  - All array pointers are DEVICE pointers except the twell_dims / twell_sizes
 *    structs and the struct arguments themselves (host memory, read during the
 *    call only). The caller owns every buffer; the library allocates no device
 *    memory and keeps no per-call state.
 *  - Dense matrices are row-major and contiguous: x, y, dy, dx are [N][D];
 *    every weight is stored [F][D] (W_gate^T, W_up^T and W_down alike), so row
 *    c of each weight belongs to hidden unit c.
 *  - Storage dtype (twell_dtype) applies to x, the three weights, dy, TwELL
 *    vals, ovf_h, ell_vals and dense_h. Accumulation is always fp32; y, a_save,
 *    ell_a, dx and the weight gradients are fp32.
 *  - Every base pointer must be 16-byte aligned.
 *  - Supported shapes: D a multiple of 64 with 64 <= D <= 8192 (<= 4096 for
 *    TWELL_F32); T_n in {16, 32, 64, 128}; 0 <= S <= T_n; F >= 1 (the last tile
 *    may be partial); N >= 0 (N == 0 is a no-op); F <= 65535.
 *  - Each call validates every argument on the host first. On error it returns
 *    the code and enqueues nothing. On success it enqueues its kernels on
 *    `stream` (a hipStream_t; NULL = the null stream) and returns without
 *    synchronising. Nothing aborts or prints.
 *  - Capacity overflow detected on the device (more overflow rows than
 *    ovf_cap, more dense rows than dense_cap) is reported through the call's
 *    device `status` word (TWELL_DEV_* bits) together with the true count; rows
 *    beyond the capacity are not computed. Check `status` after synchronising.
 *  - Calls that share output buffers must not overlap on different streams.
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum twell_status {
  TWELL_OK = 0,
  TWELL_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad shape, negative size */
  TWELL_ERR_UNSUPPORTED = 2, /* valid but outside the supported shape range */
  TWELL_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required */
  TWELL_ERR_CAPACITY = 4,    /* host-detectable capacity problem (e.g. index overflow) */
  TWELL_ERR_HIP = 5          /* a HIP runtime call failed; see twell_last_error() */
} twell_status;

typedef enum twell_dtype {
  TWELL_BF16 = 0, /* bfloat16 storage, round-to-nearest-even on store */
  TWELL_F32 = 1   /* IEEE fp32 storage */
} twell_dtype;

/* Device status bits written to the `status` words below. */
#define TWELL_DEV_OVF_CAPACITY 1u   /* n_ovf > ovf_cap: extra overflow rows were not computed */
#define TWELL_DEV_DENSE_CAPACITY 2u /* n_dense > dense_cap: extra dense rows were not routed */

/* Problem shape. Host memory. */
typedef struct twell_dims {
  int64_t n_tokens;  /* N */
  int32_t d_model;   /* D */
  int32_t d_ff;      /* F */
  int32_t tile_n;    /* T_n: TwELL tile width (columns of d_ff per tile) */
  int32_t slots;     /* S: ELL slots per (token, tile) */
  int32_t row_cap;   /* K: width of the training row-ELL (0 when no training call is made) */
  int32_t ovf_cap;   /* rows of ovf_rows / ovf_h (forward overflow capacity) */
  int32_t dense_cap; /* rows of dense_rows / dense_h (training dense-backup capacity) */
} twell_dims;

/* TwELL activation produced by twell_gate_pack / twell_pack_preact.
 * For token i and tile j the active columns c (g[i,c] > t_i, strict) of the
 * tile, in ascending order, fill slots s = 0,1,...; slot s < min(cnt,S) holds
 * vals = Q(fl32(g − t_i)) (Q = the storage rounding) and cols = c − j·T_n.
 * Slots at or beyond min(cnt,S) are don't-care. counts holds the TRUE count
 * (it may exceed S). A row overflows when any of its tile counts exceeds S;
 * overflow rows are listed in ascending order and their whole activation row
 * is kept densely in ovf_h. */
typedef struct twell_pack {
  void* vals;         /* [n_t][S][N] storage dtype (slot-major, token-minor) */
  uint16_t* cols;     /* [n_t][S][N] column offset inside the tile */
  uint16_t* counts;   /* [n_t][N]    true active count per (tile, token) */
  uint8_t* ovf_flag;  /* [N]         1 iff some tile count of the row exceeds S */
  int32_t* ovf_rows;  /* [ovf_cap]   overflow rows, ascending */
  void* ovf_h;        /* [ovf_cap][F] dense Q(ReLU(g − t)) of each overflow row, storage dtype */
  int32_t* n_ovf;     /* [1]         true number of overflow rows (may exceed ovf_cap) */
  uint32_t* status;   /* [1]         overwritten by twell_gate_pack / twell_pack_preact */
} twell_pack;

/* Hybrid training format produced by twell_route_hybrid.
 * row_nnz[i] = sum_j counts[j][i]. Row i is dense iff row_nnz[i] > K or it
 * overflowed a tile; otherwise its active columns, in ascending global order,
 * fill ELL positions 0..row_nnz[i]−1 (positions beyond are don't-care). */
typedef struct twell_hybrid {
  void* ell_vals;      /* [K][N] storage dtype: stored activation h */
  int32_t* ell_cols;   /* [K][N] global column c */
  float* ell_a;        /* [K][N] saved up activation a = x_i · W_up^T[c] */
  int32_t* row_nnz;    /* [N] true active count of every row */
  uint8_t* is_dense;   /* [N] 1 iff the row went to the dense backup */
  int32_t* dense_rows; /* [dense_cap] dense rows, ascending */
  void* dense_h;       /* [dense_cap][F] storage dtype: dense activation rows */
  int32_t* n_dense;    /* [1] true number of dense rows (may exceed dense_cap) */
  uint32_t* status;    /* [1] overwritten by twell_route_hybrid */
} twell_hybrid;

/* Largest token count the small-batch gate of twell_gate_pack_ws serves. */
#define TWELL_SMALL_BATCH_MAX 64

/* Byte sizes of every buffer for a given shape (host-only query). */
typedef struct twell_sizes {
  size_t vals, cols, counts, ovf_flag, ovf_rows, ovf_h, n_ovf, status;
  size_t ell_vals, ell_cols, ell_a, row_nnz, is_dense, dense_rows, dense_h, n_dense;
  size_t a_save;    /* [n_t][S][N] fp32 */
  size_t ws_fwd;    /* workspace of twell_ffn_fwd */
  size_t ws_bwd;    /* workspace of twell_ffn_bwd */
  size_t ws_gate;   /* workspace of twell_gate_pack_ws: N * F * 4 for bf16 and
                       1 <= N <= TWELL_SMALL_BATCH_MAX, else 0 */
} twell_sizes;

/* Human-readable name of a status code (static string, never NULL). */
const char* twell_status_str(int status);

/* Message of the last TWELL_ERR_* returned on the calling thread ("" if none). */
const char* twell_last_error(void);

/* n_t = ceil(d_ff / tile_n), or -1 when dims is NULL or d_ff / tile_n are not positive. */
int32_t twell_n_tiles(const twell_dims* dims);

/* Validate a shape and fill `out` with the byte size of every buffer and
 * workspace. Host-only; touches no device. */
twell_status twell_query_sizes(const twell_dims* dims, twell_dtype dtype, twell_sizes* out);

/* Stage 1: gate projection with the TwELL pack in its epilogue.
 *   g[i,c] = sum_k x[i,k] · w_gate_t[c,k]   (fp32 accumulation, MFMA for bf16)
 *   then the TwELL pack described at twell_pack, the overflow-row list, and the
 *   dense activation rows of the overflow rows (recomputed with the same
 *   arithmetic, so they are bit-identical to the values the epilogue saw).
 * x: [N][D], w_gate_t: [F][D] (storage dtype); t: [N] fp32 per-token threshold.
 * g_dump: optional [N][F] fp32 copy of g (debug/testing; NULL to skip).
 * Writes every field of *out. Needs no workspace. */
twell_status twell_gate_pack(const twell_dims* dims, twell_dtype dtype, const void* x,
                             const void* w_gate_t, const float* t, const twell_pack* out,
                             float* g_dump, void* stream);

/* twell_gate_pack for small batches (the decode regime), with a workspace.
 * For bf16 and 1 <= N <= TWELL_SMALL_BATCH_MAX the gate runs as a GEMV over
 * all CUs (each workgroup owns 16 hidden units, d_model split in 8 ranges
 * whose partial sums are added in a fixed order) and writes g to ws (or to
 * g_dump when given), from which the pack epilogue and the overflow rows both
 * read; the outputs are those of twell_gate_pack for that g. g is
 * deterministic but may
 * differ in its last bits from the large-batch GEMM's (a different fp32
 * summation order over d_model). Otherwise (fp32, larger N, or
 * twell_sizes.ws_gate == 0) this is exactly twell_gate_pack.
 * ws: at least twell_sizes.ws_gate bytes, 16-byte aligned device memory owned
 * by the caller (NULL allowed when ws_gate is 0). Errors as twell_gate_pack,
 * plus TWELL_ERR_WORKSPACE when ws is too small. */
twell_status twell_gate_pack_ws(const twell_dims* dims, twell_dtype dtype, const void* x,
                                const void* w_gate_t, const float* t, const twell_pack* out,
                                float* g_dump, void* ws, size_t ws_bytes, void* stream);

/* Test entry: the same pack epilogue fed from a given pre-activation g [N][F]
 * fp32 instead of the GEMM. Produces exactly what twell_gate_pack would for
 * that g. */
twell_status twell_pack_preact(const twell_dims* dims, twell_dtype dtype, const float* g,
                               const float* t, const twell_pack* out, void* stream);

/* 8-bit gate operands ("How TwELL by Sakana AI and NVIDIA Accelerates LLMs by
 * 20% Using Unstructured Sparsity", "Long-term Impact": TwELL combined with
 * 8-bit quantisation). Per-row FP8 E4M3 quantisation:
 *   scale[r] = max_k |in[r,k]| / 448 in fp32 (1 for an all-zero row and
 *              for a row holding NaN; inf in a row gives scale inf),
 *   q[r,k]   = E4M3(in[r,k] / scale[r]), nearest value with ties to even,
 *              magnitudes of 448 and above saturated to 448.
 * in: [rows][cols] bf16 or fp32; q: [rows][cols] bytes (codes: sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9, 0x7F NaN);
 * scale: [rows] fp32. Device pointers, 16-byte aligned; the caller owns them.
 * Use it on x for every call and once on w_gate_t. */
twell_status twell_quantize_e4m3(int64_t rows, int32_t cols, twell_dtype dtype, const void* in, uint8_t* q,
                                 float* scale, void* stream);

/* Stage 1 with FP8 gate operands: g[i,c] = x_scale[i] · w_scale[c] · sum_k
 * E4M3(x_q[i,k]) · E4M3(w_q[c,k]) on the matrix cores: products exact, each
 * run of 8 consecutive k summed in fixed point with every product truncated
 * toward zero below 2^-14 of the run's largest (the gfx950 FP8 instruction's
 * own arithmetic), the runs' sums accumulated in fp32, then the two scales
 * applied in fp32. Then exactly the TwELL pack, overflow list and overflow rows
 * of twell_gate_pack (recomputed by the same kernel, so bit-identical). The
 * pack buffers are those of dtype TWELL_BF16 (twell_query_sizes with
 * TWELL_BF16); d_model must be a multiple of 64. x_q [N][D], w_q [F][D] bytes;
 * x_scale [N], w_scale [F] fp32 (from twell_quantize_e4m3). The up / down
 * projection and the backward take the bf16 x and weights as before. */
twell_status twell_gate_pack_fp8(const twell_dims* dims, const uint8_t* x_q, const float* x_scale,
                                 const uint8_t* w_q, const float* w_scale, const float* t,
                                 const twell_pack* out, float* g_dump, void* stream);

/* twell_gate_pack_fp8 for small batches, with a workspace: for
 * 1 <= N <= TWELL_SMALL_BATCH_MAX the FP8 gate runs as the split GEMV of
 * twell_gate_pack_ws (same instruction and per-step k split as the GEMM,
 * 8 d_model ranges added in a fixed order, then the two scales), g goes
 * through ws (or g_dump when given) into the same pack and overflow rows.
 * ws: at least twell_sizes.ws_gate bytes of the TWELL_BF16 sizes. Otherwise
 * exactly twell_gate_pack_fp8; errors as there, plus TWELL_ERR_WORKSPACE. */
twell_status twell_gate_pack_fp8_ws(const twell_dims* dims, const uint8_t* x_q, const float* x_scale,
                                    const uint8_t* w_q, const float* w_scale, const float* t,
                                    const twell_pack* out, float* g_dump, void* ws, size_t ws_bytes,
                                    void* stream);

/* Stage 2: fused up + down projection from TwELL.
 *   y_i = sum over active (i,c) of h_ic · (x_i · w_up_t[c]) · w_down[c]
 * with h read from TwELL (or from ovf_h for overflow rows); z = h·a is kept in
 * fp32 and the hidden state is never written to memory.
 * y: [N][D] fp32, fully overwritten (rows beyond the overflow capacity are
 * left unwritten; the pack's status says so).
 * a_save: optional [n_t][S][N] fp32; when given, a = x_i · w_up_t[c] is stored
 * at the slot of every packed entry of non-overflow rows (training).
 * ws: workspace of at least twell_sizes.ws_fwd bytes: per-row entry totals,
 * the (column, z = h·a) pair of every packed entry in row-major order (the
 * sparse intermediate between the up and the down projection, never a dense
 * hidden state), for large d_model x d_ff the partial a of every entry over
 * each of a few d_model ranges, the partial rows of the overflow-row
 * chunks, for bf16 the overflow rows' z = h·a (as bf16 high and low parts),
 * and the list position of each group of tiles' first entry per row. */
twell_status twell_ffn_fwd(const twell_dims* dims, twell_dtype dtype, const twell_pack* pack,
                           const void* x, const void* w_up_t, const void* w_down, float* y,
                           float* a_save, void* ws, size_t ws_bytes, void* stream);

/* Stages 1 and 2 in one call ("Sakana AI and NVIDIA present TwELL",
 * edge.aivizor.me, second paragraph: the gate projection's epilogue forms
 * TwELL and one inference kernel consumes it for the up and down
 * projections). Same outputs as twell_gate_pack (or twell_gate_pack_ws when
 * gate_ws is not NULL) followed by twell_ffn_fwd on the same stream: the
 * TwELL pack, the overflow list and rows in *pack, y, and a_save when given.
 * Within one call the overflow branch (the ascending overflow list, the
 * overflow rows' dense activations and their up / down products) is
 * enqueued on a side stream beside the up / down projection of the other
 * rows, which reads only the pack and the overflow flags, and is joined back
 * into `stream` before the call returns; the two separate calls must each
 * finish their part before returning. The library keeps one side stream (and
 * one pair of events) per caller stream and device, created on that caller
 * stream's first call and kept until the process ends (at most 16 per
 * device); a caller stream that is being captured into a graph before it has
 * one, or one beyond that limit, gets the branch in order on `stream`
 * instead, with the same results. No g_dump.
 * x, w_gate_t, w_up_t, w_down: as in the two calls; ws: the forward
 * workspace (twell_sizes.ws_fwd bytes); gate_ws: the small-batch gate
 * workspace (twell_sizes.ws_gate bytes) or NULL. Validation covers every
 * argument of both calls before anything is enqueued; errors as there. */
twell_status twell_ffn_forward(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                               const float* t, const twell_pack* pack, const void* w_up_t, const void* w_down,
                               float* y, float* a_save, void* ws, size_t ws_bytes, void* gate_ws,
                               size_t gate_ws_bytes, void* stream);

/* twell_ffn_forward with the FP8 gate: twell_gate_pack_fp8 (or
 * twell_gate_pack_fp8_ws when gate_ws is not NULL) followed by twell_ffn_fwd
 * (bf16 x and weights) on the same stream, in one call, with the same
 * outputs and the same overlap of the overflow branch. Arguments as in those
 * calls; the pack buffers are those of TWELL_BF16. */
twell_status twell_ffn_forward_fp8(const twell_dims* dims, const uint8_t* x_q, const float* x_scale,
                                   const uint8_t* w_q, const float* w_scale, const float* t, const twell_pack* pack,
                                   const void* x, const void* w_up_t, const void* w_down, float* y, float* a_save,
                                   void* ws, size_t ws_bytes, void* gate_ws, size_t gate_ws_bytes, void* stream);

/* Size of the library's static device scratch used by
 * twell_ffn_forward_noalloc (one copy per GPU, held until the process ends). */
#define TWELL_NOALLOC_SCRATCH_BYTES (128u << 20)

/* twell_ffn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments (minus the two workspaces), outputs and results as
 * twell_ffn_forward (with gate_ws given whenever twell_sizes.ws_gate > 0);
 * the workspaces are carved out of a static device array of
 * TWELL_NOALLOC_SCRATCH_BYTES that the library owns, one per GPU. The call
 * allocates nothing, frees nothing and creates no stream: every kernel is
 * enqueued on `stream` in order (the overflow branch does not run beside the
 * up / down projection). On a device's first call the array's device address
 * is looked up (hipGetSymbolAddress) and kept.
 * The scratch keeps the last call's contents; every call writes what it reads.
 * Calls that overlap on one GPU (different streams, or different host
 * threads, without ordering between them) share that GPU's scratch and race:
 * the caller must order them.
 * Errors as twell_ffn_forward, plus TWELL_ERR_WORKSPACE when the shape needs
 * more than TWELL_NOALLOC_SCRATCH_BYTES of workspace
 * (align256(twell_sizes.ws_fwd) + twell_sizes.ws_gate), checked on the host
 * before anything is enqueued. */
twell_status twell_ffn_forward_noalloc(const twell_dims* dims, twell_dtype dtype, const void* x,
                                       const void* w_gate_t, const float* t, const twell_pack* pack,
                                       const void* w_up_t, const void* w_down, float* y, float* a_save,
                                       void* stream);

/* Stage 3a: route every row to the row-ELL (width K = dims->row_cap >= 1) or to
 * the dense backup (rule at twell_hybrid). a_save is the array filled by
 * twell_ffn_fwd. Writes every field of *out. */
twell_status twell_route_hybrid(const twell_dims* dims, twell_dtype dtype, const twell_pack* pack,
                                const float* a_save, const twell_hybrid* out, void* stream);

/* Stage 3b: backward through the hybrid format, for
 *   L = sum(dy ⊙ y) + l1_lambda · sum(h)
 * with M the active mask, h the stored activation and a = x·W_up:
 *   dz = dy·W_down^T (at active units), da = dz·h, dg = dz·a + l1_lambda,
 *   dx = sum_c da·W_up^T[c] + dg·W_gate^T[c],
 *   dW_up^T[c] = sum_i da_ic x_i,  dW_gate^T[c] = sum_i dg_ic x_i,
 *   dW_down[c] = sum_i h_ic a_ic dy_i.
 * dy: [N][D] storage dtype. dx: [N][D] fp32; dw_*: [F][D] fp32; all four are
 * fully overwritten (deterministic: no floating-point atomics). For dense rows
 * a is recomputed from x. Dense rows beyond dense_cap (status bit set by
 * twell_route_hybrid) contribute nothing and get dx = 0.
 * ws: at least twell_sizes.ws_bwd bytes.
 * Returns TWELL_ERR_UNSUPPORTED for d_ff > 32768. */
twell_status twell_ffn_bwd(const twell_dims* dims, twell_dtype dtype, const twell_hybrid* hyb,
                           const void* x, const void* dy, const void* w_gate_t,
                           const void* w_up_t, const void* w_down, float l1_lambda, float* dx,
                           float* dw_gate_t, float* dw_up_t, float* dw_down, void* ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Tracing (diagnostics). When started, every kernel launched by the calls
 * above is bracketed by two HIP events recorded on the call's stream, so the
 * device time of each kernel can be read back afterwards. Events are created
 * by twell_trace_start (capacity = launches that can be recorded; later
 * launches are counted as dropped); recording itself allocates nothing.
 * Not meant to be used from several threads at once.
 * ------------------------------------------------------------------------- */

/* Start (or restart) recording with room for `capacity` launches (1..2^20). */
twell_status twell_trace_start(int32_t capacity);
/* Stop recording; the records stay readable. */
twell_status twell_trace_stop(void);
/* Number of launches recorded / dropped since the last start. */
int32_t twell_trace_count(void);
int32_t twell_trace_dropped(void);
/* Kernel name (static string) and device time in ms of record i; waits for
 * that launch to finish. */
twell_status twell_trace_get(int32_t i, const char** name, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
