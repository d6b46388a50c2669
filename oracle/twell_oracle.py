"""CPU oracle for the activation-sparse gated FFN and its TwELL formats.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or call it. It shares no code with the HIP library (no kernels, no
headers, no helpers); its only common dependency is the seeded input
generator, which holds none of the method's arithmetic.

Everything is plain NumPy in float64 on inputs that are exact bf16 (or fp32)
values upcast to float64. Library primitives (matmul, sort, cumsum) serve as
steps; there is no blocking, fusion or reordering beyond what each definition
states.

Sources (the three pages on TwELL; no section numbers exist on them, so each
cite names the page and its paragraph or heading):

* "Sakana AI and NVIDIA present TwELL" (edge.aivizor.me community post),
  second paragraph: the gated FFN with "gate", "up" and "down" projections;
  horizontal tiles of width T_n matched to the matmul tile; nonzeros packed
  locally inside each tile; the format built in the gate projection's
  epilogue; a fused up+down inference kernel that never writes the hidden
  state; a hybrid training format that routes each row either to a compact
  ELL matrix or to a dense backup for overflows. Fourth paragraph: the
  maximum number of nonzeros per row can far exceed the mean.
* "How TwELL by Sakana AI and NVIDIA Accelerates LLMs by 20%"
  (aimodelsnavi.com), "Technical Explanation": ReLU with L1 regularisation
  gives >95% zeros; TwELL = Tile-wise ELLPACK. "Core of TwELL": fixed-size
  tiles with nonzeros packed inside each tile.

Readings where the pages are silent (each is also listed in the design notes):
stored value is ReLU(g - t) with a per-token threshold t_i; a unit is active iff
g > t (strict); slots inside a tile hold the active columns in ascending order;
counts hold the true per-tile count even when it exceeds the slot capacity S;
slots at or beyond min(count, S) are don't-care; a row overflows when any tile
count exceeds S; overflow rows are listed in ascending order; the hybrid format
sends a row to the dense backup iff its total count exceeds the ELL width K or
it overflowed a tile; the L1 term is lambda * sum(h); the stored activation is
rounded to the storage dtype (bf16 round-to-nearest-even, or fp32) and that
rounded value is what the up/down products and the backward use.

Parity status: every function here is pinned by the CPU test suite against
closed forms, torch float64 autograd, finite differences, brute-force
enumeration or hand-worked fixtures (the FP8 quantiser and FP8 gate by the
hand-worked tests/golden/fp8_handworked.json); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# Storage rounding
# ---------------------------------------------------------------------------


def round_bf16(a) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even, in float64.

    bfloat16 keeps 8 significant bits and the fp32 exponent range. For a
    normal float64 value m * 2**e with m in [0.5, 1), the nearest bf16 value
    is rint(m * 2**8) * 2**(e - 8), where rint rounds half to even. Zero maps
    to zero (sign kept). Values outside the normal fp32 range are rejected:
    the activations here are O(1).
    """
    a = np.asarray(a, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("round_bf16: non-finite input")
    nz = a != 0
    if np.any(np.abs(a[nz]) < 2.0 ** -126) or np.any(np.abs(a) >= 2.0 ** 127):
        raise ValueError("round_bf16: value outside the normal fp32 range")
    m, e = np.frexp(a)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_f32(a) -> np.ndarray:
    """Round to the nearest fp32 value (numpy's cast is IEEE round-to-nearest-even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def store_round(a, store: str) -> np.ndarray:
    """The format's storage rounding Q: "bf16", "f32", or "exact" (identity)."""
    if store == "bf16":
        return round_bf16(a)
    if store == "f32":
        return round_f32(a)
    if store == "exact":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown store {store!r}")


def _f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("oracle inputs must be finite")
    return a


# ---------------------------------------------------------------------------
# Dense forward (the definition the sparse path must reproduce)
# ---------------------------------------------------------------------------


def n_tiles(d_ff: int, tile_n: int) -> int:
    """Number of TwELL tiles: d_ff split into horizontal tiles of width T_n (last one partial)."""
    if tile_n <= 0:
        raise ValueError("tile_n must be positive")
    return -(-int(d_ff) // int(tile_n))


def gate_preact(x, w_gate_t) -> np.ndarray:
    """g[i, c] = sum_k x[i, k] * W_gate^T[c, k]  (gate projection, weights stored [F][D])."""
    return _f64(x) @ _f64(w_gate_t).T


def ffn_forward(x, w_gate_t, w_up_t, w_down, t, store: str = "bf16", arith: str = "f64") -> dict:
    """Dense ReLU-gated FFN y = (Q(ReLU(x W_gate - t)) * (x W_up)) W_down, float64.

    g = x W_gate (gate projection), active mask M = g > t_i (strict),
    h = M * (g - t_i), hq = Q(h) the storage rounding of the activation,
    a = x W_up (up projection), z = hq * a, y = z W_down (down projection).

    arith="f32" forms the stored activation the way the packed format defines
    it, Q(fl32(g32 - t)) with g32 = fl32(g) and the compare and subtraction in
    IEEE fp32; everything else stays float64. arith="f64" uses g and g - t in
    float64.
    """
    x = _f64(x)
    t = _f64(t).reshape(-1)
    g = gate_preact(x, w_gate_t)
    if arith == "f32":
        g32 = g.astype(np.float32)
        t32 = t.astype(np.float32)
        mask = g32 > t32[:, None]
        h = np.where(mask, (g32 - t32[:, None]).astype(np.float64), 0.0)
    elif arith == "f64":
        mask = g > t[:, None]
        h = np.where(mask, g - t[:, None], 0.0)
    else:
        raise ValueError(f"unknown arith {arith!r}")
    hq = store_round(h, store)
    a = x @ _f64(w_up_t).T
    z = hq * a
    y = z @ _f64(w_down)
    return {"g": g, "mask": mask, "h": h, "hq": hq, "a": a, "z": z, "y": y}


# ---------------------------------------------------------------------------
# 8-bit gate operands (OCP FP8 E4M3)
# ---------------------------------------------------------------------------
# "How TwELL by Sakana AI and NVIDIA Accelerates LLMs by 20% Using Unstructured
# Sparsity", "Long-term Impact": TwELL combined with 8-bit quantisation is named
# as a direction. Reading taken here (the page fixes no scheme): only the gate
# projection's operands are quantised, to FP8 E4M3 with one fp32 scale per row
# (per token for x, per hidden unit for W_gate) equal to the row's largest
# magnitude / 448; g = s_x,i * s_w,c * sum_k q_x[i,k] q_w[c,k]; everything after
# g (threshold, TwELL, up/down, backward) is unchanged.

E4M3_MAX = 448.0


def e4m3_decode(q) -> np.ndarray:
    """FP8 E4M3 ("FN" variant) code -> value: sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; there
    are no infinities and S.1111.111 is NaN (so the largest value is 448)."""
    q = np.asarray(q, dtype=np.uint8).astype(np.int64)
    sign = np.where((q & 0x80) != 0, -1.0, 1.0)
    e = (q >> 3) & 0xF
    m = (q & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((q & 0x7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(v) -> np.ndarray:
    """Value -> FP8 E4M3 code, rounding to the nearest representable value with
    ties to the even code, and saturating magnitudes beyond 448 to 448 (NaN ->
    0x7F). The quantum of a magnitude a is 2^(e - 3) for 2^e <= a < 2^(e+1)
    (e >= -6) and 2^-9 below 2^-6 (subnormals)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)  # a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    e = np.clip(ex - 1, -6, 8).astype(np.float64)
    quantum = np.exp2(e - 3.0)
    r = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)  # np.rint: ties to even
    # encode the representable magnitude r
    _, er = np.frexp(np.where(r > 0, r, 1.0))
    er = (er - 1).astype(np.int64)
    sub = r < 2.0 ** -6
    m_sub = np.rint(r / 2.0 ** -9).astype(np.int64)
    m_nrm = np.rint((r / np.exp2(er.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    code = np.where(sub, m_sub, ((er + 7) << 3) | m_nrm)
    code = np.where(np.signbit(v), code | 0x80, code)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def quantize_rows_e4m3(a):
    """Per-row FP8 quantisation: scale = float32(max|row|) / 448 in float32,
    replaced by 1 when it is not > 0 (an all-zero row, a row holding NaN, or a
    maximum so small that the quotient underflows to 0: a zero scale would
    turn the row's zeros into NaN codes); q = e4m3(float32(a / scale)).
    Returns (q uint8, scale float32)."""
    a32 = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(a32), axis=1) if a32.shape[1] else np.zeros(a32.shape[0], np.float32)
    with np.errstate(invalid="ignore"):
        scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
        scaled = (a32 / scale[:, None]).astype(np.float32)
    return e4m3_encode(scaled), scale


def gate_preact_fp8(xq, x_scale, wq, w_scale) -> np.ndarray:
    """g[i, c] = s_x[i] * s_w[c] * sum_k e4m3(q_x[i, k]) * e4m3(q_w[c, k]), fp64."""
    return (_f64(x_scale)[:, None] * _f64(w_scale)[None, :]) * (e4m3_decode(xq) @ e4m3_decode(wq).T)


# ---------------------------------------------------------------------------
# TwELL: tile-wise ELLPACK pack / unpack
# ---------------------------------------------------------------------------


def pack(g, t, tile_n: int, slots: int, store: str = "bf16", arith: str = "f32") -> dict:
    """Pack ReLU(g - t) into TwELL.

    d_ff is cut into n_t = ceil(F / T_n) tiles of width T_n (last one partial).
    For every token i and tile j the active columns c (g[i, c] > t_i) of the
    tile, in ascending order, fill slots s = 0, 1, ...; slot s < min(cnt, S)
    holds val = Q(g - t) and col = c - j*T_n (offset inside the tile);
    counts[j, i] = cnt is the true number of active columns of the tile, even
    when it exceeds S. ovf_flag[i] is set when any tile of row i has cnt > S;
    ovf_rows lists those rows in ascending order.

    arith="f32" evaluates the compare and the subtraction in IEEE fp32 on fp32
    inputs (the precision the format is built in); arith="f64" in float64.
    Layout: vals / cols are [n_t][S][N] (slot-major, token-minor), counts is
    [n_t][N]. Slots at or beyond min(cnt, S) are left at val 0 / col -1
    (don't-care in the format).
    """
    if arith == "f32":
        g = np.asarray(g, dtype=np.float32)
        t = np.asarray(t, dtype=np.float32).reshape(-1)
        active = g > t[:, None]
        diff = (g - t[:, None]).astype(np.float64)  # IEEE fp32 subtraction
    elif arith == "f64":
        g = _f64(g)
        t = _f64(t).reshape(-1)
        active = g > t[:, None]
        diff = g - t[:, None]
    else:
        raise ValueError(f"unknown arith {arith!r}")
    N, F = g.shape
    if slots < 0:
        raise ValueError("slots must be >= 0")
    nt = n_tiles(F, tile_n)
    vals = np.zeros((nt, slots, N), dtype=np.float64)
    cols = np.full((nt, slots, N), -1, dtype=np.int64)
    counts = np.zeros((nt, N), dtype=np.int64)
    for j in range(nt):
        c0, c1 = j * tile_n, min((j + 1) * tile_n, F)
        act = active[:, c0:c1]
        counts[j] = act.sum(axis=1)
        rank = np.cumsum(act, axis=1) - 1          # slot each active column would take
        ii, cc = np.nonzero(act & (rank < slots))
        ss = rank[ii, cc]
        vals[j, ss, ii] = store_round(diff[ii, c0 + cc], store) if ii.size else 0.0
        cols[j, ss, ii] = cc
    ovf_flag = (counts > slots).any(axis=0)
    ovf_rows = np.nonzero(ovf_flag)[0].astype(np.int64)
    return {"vals": vals, "cols": cols, "counts": counts, "ovf_flag": ovf_flag,
            "ovf_rows": ovf_rows, "n_ovf": int(ovf_rows.size), "tile_n": int(tile_n),
            "slots": int(slots), "d_ff": int(F)}


def dense_activation(g, t, store: str = "bf16", arith: str = "f32") -> np.ndarray:
    """Q(ReLU(g - t)) as a dense [N][F] array, in the same arithmetic as pack()."""
    if arith == "f32":
        g = np.asarray(g, dtype=np.float32)
        t = np.asarray(t, dtype=np.float32).reshape(-1)
        h = np.where(g > t[:, None], (g - t[:, None]).astype(np.float64), 0.0)
    else:
        g = _f64(g)
        t = _f64(t).reshape(-1)
        h = np.where(g > t[:, None], g - t[:, None], 0.0)
    return store_round(h, store)


def unpack(packed: dict, ovf_h: Optional[np.ndarray] = None) -> np.ndarray:
    """Scatter TwELL slots back to a dense [N][F] activation.

    Rows that did not overflow are rebuilt from their slots alone; overflow
    rows are taken from ovf_h (dense rows in ovf_rows order) when given, and
    are left zero otherwise.
    """
    vals, cols, counts = packed["vals"], packed["cols"], packed["counts"]
    tile_n, slots, F = packed["tile_n"], packed["slots"], packed["d_ff"]
    nt, N = counts.shape
    out = np.zeros((N, F), dtype=np.float64)
    keep = ~packed["ovf_flag"]
    for j in range(nt):
        for s in range(slots):
            rows = np.nonzero(keep & (counts[j] > s))[0]
            out[rows, j * tile_n + cols[j, s, rows]] = vals[j, s, rows]
    if ovf_h is not None and packed["n_ovf"]:
        out[packed["ovf_rows"]] = np.asarray(ovf_h, dtype=np.float64)[: packed["n_ovf"]]
    return out


def sparse_forward(packed: dict, x, w_up_t, w_down, ovf_h: Optional[np.ndarray] = None) -> np.ndarray:
    """y from the packed activation: for each active (i, c) in the format,
    y_i += h_ic * (x_i . W_up^T[c]) * W_down[c]; overflow rows use their dense h."""
    hq = unpack(packed, ovf_h)
    x = _f64(x)
    return (hq * (x @ _f64(w_up_t).T)) @ _f64(w_down)


# ---------------------------------------------------------------------------
# Hybrid ELL + dense-backup format (training)
# ---------------------------------------------------------------------------


def route(packed: dict, row_cap: int, a=None, ovf_h: Optional[np.ndarray] = None) -> dict:
    """Route every row to a fixed-width row-ELL (width K) or to the dense backup.

    row_nnz[i] = sum_j counts[j, i]. Row i goes to the dense backup iff
    row_nnz[i] > K or it overflowed a TwELL tile; otherwise its active columns,
    in ascending global order (tile by tile, slot by slot), fill ELL positions
    0 .. row_nnz[i]-1 of ell_cols / ell_vals [K][N] (slot-major, token-minor).
    ell_a holds the saved up activation a[i, c] at the same positions when a
    dense a [N][F] is supplied. dense_rows lists backup rows in ascending order
    and dense_h their dense activation rows.
    """
    counts, vals, cols = packed["counts"], packed["vals"], packed["cols"]
    tile_n = packed["tile_n"]
    nt, N = counts.shape
    K = int(row_cap)
    row_nnz = counts.sum(axis=0)
    dense = (row_nnz > K) | packed["ovf_flag"]
    ell_vals = np.zeros((K, N), dtype=np.float64)
    ell_cols = np.full((K, N), -1, dtype=np.int64)
    ell_a = np.zeros((K, N), dtype=np.float64)
    a = None if a is None else np.asarray(a, dtype=np.float64)
    for i in np.nonzero(~dense)[0]:
        k = 0
        for j in range(nt):
            for s in range(int(counts[j, i])):
                c = j * tile_n + int(cols[j, s, i])
                ell_cols[k, i] = c
                ell_vals[k, i] = vals[j, s, i]
                if a is not None:
                    ell_a[k, i] = a[i, c]
                k += 1
    dense_rows = np.nonzero(dense)[0].astype(np.int64)
    full = unpack(packed, ovf_h)
    return {"row_nnz": row_nnz, "is_dense": dense, "ell_vals": ell_vals, "ell_cols": ell_cols,
            "ell_a": ell_a, "dense_rows": dense_rows, "n_dense": int(dense_rows.size),
            "dense_h": full[dense_rows], "row_cap": K}


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------


def ffn_backward(x, dy, w_gate_t, w_up_t, w_down, mask, hq, lam: float) -> dict:
    """Gradients of L = sum(dy * y) + lam * sum(h) for the gated FFN, float64.

    With a = x W_up and z = hq * a (hq the stored activation, whose rounding is
    passed through as the identity):
      dz = dy W_down^T;  da = M * dz * hq;  dg = M * (dz * a + lam)
      dx = da W_up^T^T + dg W_gate^T^T  (weights stored [F][D]: dx = da @ W_up^T + dg @ W_gate^T)
      dW_up^T = da^T x;  dW_gate^T = dg^T x;  dW_down = z^T dy.
    The threshold receives no gradient (it is an input).
    """
    x, dy = _f64(x), _f64(dy)
    wg, wu, wd = _f64(w_gate_t), _f64(w_up_t), _f64(w_down)
    m = np.asarray(mask, dtype=bool)
    hq = _f64(hq)
    a = x @ wu.T
    dz = dy @ wd.T
    da = np.where(m, dz * hq, 0.0)
    dg = np.where(m, dz * a + lam, 0.0)
    z = hq * a
    return {"dx": da @ wu + dg @ wg, "dw_gate_t": dg.T @ x, "dw_up_t": da.T @ x,
            "dw_down": z.T @ dy, "dz": dz, "da": da, "dg": dg, "a": a, "z": z}


# ---------------------------------------------------------------------------
# Test helpers
# ---------------------------------------------------------------------------


def margin_thresholds(g, p, window: float = 0.25) -> np.ndarray:
    """Per-row fp32 thresholds placed mid-way inside a wide gap of the row's g.

    For row i the target number of active units is k = round(p_i * F). Among
    the candidate cut points within +-window*k (at least +-2) of that rank, the
    one with the widest gap between adjacent sorted values is chosen, and t_i is
    the fp32 value nearest the midpoint of that gap. Every unit is then at least
    half a gap away from t_i, so a mask computed from g with any rounding much
    smaller than the gap agrees with the exact one.
    """
    g = _f64(g)
    N, F = g.shape
    p = np.broadcast_to(np.asarray(p, dtype=np.float64), (N,))
    s = np.sort(g, axis=1)
    t = np.empty(N, dtype=np.float32)
    for i in range(N):
        k = int(round(p[i] * F))
        k = min(max(k, 1), F - 1)
        w = max(2, int(window * k))
        lo, hi = max(1, F - k - w), min(F - 1, F - k + w)   # cut between s[q-1] and s[q]
        q = np.arange(lo, hi + 1)
        gaps = s[i, q] - s[i, q - 1]
        b = int(q[np.argmax(gaps)])
        mid = np.float32(0.5 * (s[i, b - 1] + s[i, b]))
        if not (s[i, b - 1] < float(mid) < s[i, b]):
            raise ValueError(f"row {i}: gap too narrow for an fp32 threshold")
        t[i] = mid
    return t


def bf16_ulp(a) -> np.ndarray:
    """Spacing of bf16 values at |a| (2^(e-7) for |a| in [2^e, 2^(e+1))); 0 at a == 0."""
    a = np.abs(_f64(a))
    _, e = np.frexp(a)
    return np.where(a > 0, np.ldexp(1.0, e - 8), 0.0)


def store_ulp(a, store: str) -> np.ndarray:
    """Spacing of storage values at |a|: bf16 (8 significant bits) or fp32 (24)."""
    a = np.abs(_f64(a))
    _, e = np.frexp(a)
    bits = {"bf16": 8, "f32": 24}[store]
    return np.where(a > 0, np.ldexp(1.0, e - bits), 0.0)


def rounding_ambiguous(h, delta, store: str = "bf16") -> np.ndarray:
    """Entries whose stored value Q(v) is not the same for every v within
    [h - delta, h + delta]: an implementation that evaluates h with an error up
    to delta may store either neighbour there, and both are correct results."""
    h = _f64(h)
    lo = store_round(np.maximum(h - delta, 0.0), store)
    hi = store_round(h + delta, store)
    return (h > 0) & (lo != hi)


def relative_margin(g, t) -> np.ndarray:
    """Per row: min_c |g - t| / sigma_i with sigma_i the row's rms of g."""
    g = _f64(g)
    t = _f64(t).reshape(-1)
    sig = np.sqrt(np.mean(g * g, axis=1))
    return np.min(np.abs(g - t[:, None]), axis=1) / np.maximum(sig, 1e-300)


def row_rms(a) -> np.ndarray:
    a = _f64(a)
    return np.sqrt(np.mean(a * a, axis=1))


def rowwise_rel_err(got, ref) -> np.ndarray:
    """max|got - ref| / rms(ref) per row (inf where ref is zero but got is not)."""
    got, ref = _f64(got), _f64(ref)
    err = np.max(np.abs(got - ref), axis=1)
    rms = row_rms(ref)
    out = np.where(rms > 0, err / np.where(rms > 0, rms, 1.0), np.where(err > 0, np.inf, 0.0))
    return out


def flops_dense_ffn(N: int, D: int, F: int) -> float:
    """Dense gated FFN forward: three N x D x F products."""
    return 6.0 * N * D * F


__all__ = [name for name in dir() if not name.startswith("_") and name not in ("annotations", "math", "np", "Optional")]
