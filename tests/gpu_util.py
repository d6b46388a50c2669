"""Helpers shared by the GPU parity tests: device upload, the libtwell pipeline,
readback of the packed formats, and per-row comparisons against the oracle."""
from __future__ import annotations

import numpy as np
import torch

from activation_sparse_ffn_03_amd import twell as tw
from oracle import twell_oracle as orc


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    tw.lib()  # raises if libtwell.so is missing


def dev(a, dtype: str):
    """float32 numpy array holding exact storage values -> device tensor in the storage dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def f64(t: torch.Tensor) -> np.ndarray:
    # Unused TwELL slots and ELL positions keep whatever the buffer held (any
    # bit pattern, NaNs included); callers compare valid entries only.
    with np.errstate(invalid="ignore"):
        return t.detach().float().cpu().numpy().astype(np.float64)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16).astype(np.int64)


def code(dtype: str) -> int:
    return tw.BF16 if dtype == "bf16" else tw.F32


def check_pack(pk: tw.TwellPack, ref: dict, cap: int, exact_vals: bool = True, ulps: int = 1):
    """Bit-exact comparison of a GPU TwELL pack with the oracle's pack."""
    counts = u16(pk.counts)
    np.testing.assert_array_equal(counts, ref["counts"], err_msg="counts")
    S = ref["vals"].shape[1]
    valid = np.arange(S)[None, :, None] < np.minimum(ref["counts"], S)[:, None, :]
    cols = u16(pk.cols)
    np.testing.assert_array_equal(cols[valid], ref["cols"][valid], err_msg="cols")
    vals = f64(pk.vals)
    if exact_vals:
        np.testing.assert_array_equal(vals[valid], ref["vals"][valid], err_msg="vals")
    else:
        rv = ref["vals"][valid]
        ulp = np.abs(rv) * 2.0 ** -7
        assert np.all(np.abs(vals[valid] - rv) <= ulps * ulp), "vals beyond bf16 ulp tolerance"
    flag = pk.ovf_flag.cpu().numpy().astype(bool)
    np.testing.assert_array_equal(flag, ref["ovf_flag"], err_msg="ovf_flag")
    n_ovf = int(pk.n_ovf.item())
    assert n_ovf == ref["n_ovf"]
    k = min(n_ovf, cap)
    np.testing.assert_array_equal(pk.ovf_rows[:k].cpu().numpy(), ref["ovf_rows"][:k], err_msg="ovf_rows")
    status = int(pk.status.item())
    assert status == (tw.DEV_OVF_CAPACITY if n_ovf > cap else 0)


# Bound on |g32 - g| of an fp32 evaluation of the gate pre-activation,
# relative to the row's rms(g): about 100x the typical fp32 accumulation error
# at d_model <= 8192 (the gate GEMM test checks the GPU stays inside it).
DELTA_REL = 2.0 ** -17


def fp8_gate_err_bound(xq, sx, wq, sw, g):
    """Bound on |g_gpu - g| for the FP8 gate, elementwise.

    On gfx950, v_mfma_f32_32x32x64_f8f6f4 (the large-batch gate) and
    v_mfma_f32_16x16x32_fp8_fp8 (the small-batch GEMV) both sum each run of 8
    bytes a lane supplies (8 consecutive k in these kernels' layouts) in fixed
    point: every product is truncated toward zero on the grid 2^(E - 14),
    E = floor(log2) of the group's largest product (measured: 448*448 + 20 in
    one group gives 448*448 + 16, 448*448 - 5 gives 448*448, and products in
    different groups add with fp32 rounding). The group sums and the
    accumulator are added in fp32. The bound takes the grid one bit coarser,
    G = 2^(E - 13), which also covers a grid tied to the exponent sum of the
    operands, and allows per group the products' remainders on G plus G (a
    truncation of the group sum instead); the fp32 additions, one per group
    and one per instruction (4.5 per 32 k for the 64-k instruction, 5 for the
    32-k one), add at most 5 ulps of the running sum per 32 k; the epilogue's
    two scale multiplications add 2 ulps of g.
    """
    qx = orc.e4m3_decode(xq)
    qw = orc.e4m3_decode(wq)
    N, D = qx.shape
    F = qw.shape[0]
    bx = np.abs(qx).reshape(N, D // 8, 8)
    bw = np.abs(qw).reshape(F, D // 8, 8)
    out = np.empty((N, F))
    for i in range(N):
        p = bx[i][None] * bw                            # [F, D/8, 8] |products|, exact in fp64
        m = p.max(axis=2, keepdims=True)
        e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
        grid = np.where(m > 0, np.exp2(e - 13), 0.0)
        gs = np.where(grid > 0, grid, 1.0)
        rem = np.where(grid > 0, p - np.floor(p / gs) * gs, 0.0)  # exact: gs is a power of two
        trunc = (rem.sum(axis=2) + grid[..., 0]).sum(axis=1)
        rounding = 5 * (D // 32) * 2.0 ** -24 * p.sum(axis=(1, 2))
        out[i] = trunc + rounding
    s = np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    return s * out + 2.0 ** -22 * np.abs(g)


def h_flip(fw: dict, store: str) -> np.ndarray:
    """Per entry, how far the stored activation may legitimately differ from
    the oracle's: one storage ulp where rounding Q(fl32(g - t)) is ambiguous
    under an fp32 evaluation error of g (both neighbours are correct results),
    else 0."""
    g, h = fw["g"], fw["h"]
    rms = np.sqrt(np.mean(g * g, axis=1))
    delta = DELTA_REL * rms[:, None] + np.abs(h) * 2.0 ** -23
    amb = orc.rounding_ambiguous(h, delta, store)
    return np.where(amb, orc.store_ulp(h, store), 0.0)


def rowwise_ok(got: np.ndarray, ref: np.ndarray, tol: float, what: str, slack=None):
    """|err| <= tol * rms(ref row) (+ slack) per row; rows whose reference is all
    zero (and carry no slack) must be exactly zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = orc.row_rms(ref)
    bound = tol * rms[:, None] + (0.0 if slack is None else slack)
    ok = np.abs(got - ref) <= bound
    bad = np.nonzero(~ok.all(axis=1))[0]
    err = orc.rowwise_rel_err(got, ref)
    assert bad.size == 0, (f"{what}: {bad.size} rows beyond {tol}*rms(+slack); first bad row {int(bad[0])} "
                           f"rel err {err[bad[0]]:.3e}")
    return float(np.max(err[np.isfinite(err)])) if np.isfinite(err).any() else 0.0


class Pipeline:
    """Upload a workload and run the libtwell hot path on it."""

    def __init__(self, w, thresholds=None, ovf_cap=None, dense_cap=None, slots=None, tile_n=None, row_cap=None):
        require_gpu()
        self.w = w
        self.dtype = w.dtype
        self.code = code(w.dtype)
        S = w.slots if slots is None else slots
        T = w.tile_n if tile_n is None else tile_n
        K = w.row_cap if row_cap is None else row_cap
        self.ovf_cap = max(8, w.N // 8) if ovf_cap is None else ovf_cap
        self.dense_cap = (max(8, w.N // 8) if w.train or K else 0) if dense_cap is None else dense_cap
        self.dims = tw.make_dims(w.N, w.D, w.F, T, S, K, self.ovf_cap, self.dense_cap)
        self.t_np = (w.t if thresholds is None else thresholds).astype(np.float32)
        self.x = dev(w.x, w.dtype)
        self.wg = dev(w.w_gate_t, w.dtype)
        self.wu = dev(w.w_up_t, w.dtype)
        self.wd = dev(w.w_down, w.dtype)
        self.t = torch.from_numpy(self.t_np).cuda()
        self.dy = dev(w.dy, w.dtype) if w.dy is not None else None
        self.ffn = tw.TwellFFN(self.dims, self.code, train=bool(K) or w.train)

    def forward(self, g_dump=None):
        y = self.ffn.forward(self.x, self.wg, self.wu, self.wd, self.t, g_dump=g_dump)
        torch.cuda.synchronize()
        return y

    def backward(self, lam=None):
        lam = self.w.lam if lam is None else lam
        out = self.ffn.backward(self.x, self.dy, self.wg, self.wu, self.wd, lam)
        torch.cuda.synchronize()
        return out
