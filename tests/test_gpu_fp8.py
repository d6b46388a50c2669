"""FP8 (E4M3) gate operands against the oracle.

* quantisation: codes and row scales bit-exact (bf16 and fp32 inputs, widths
  with and without 4-byte groups, an all-zero row);
* the gate + TwELL pack on operands whose products and sums are exact in fp32
  (codes of multiples of 1/8 in [-2, 2], power-of-two scales): TwELL, the
  overflow list and the overflow rows bit-exact;
* the gate on random operands: g within the error bound of the FP8 matrix
  instruction (below) of the oracle's fp64 value;
* the forward with the FP8 gate and the bf16 up / down projections, thresholds
  placed in wide gaps of g so that the mask is unambiguous.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from activation_sparse_ffn_03_amd import twell as tw
from oracle import twell_oracle as orc

from gpu_util import check_pack, f64, fp8_gate_err_bound, require_gpu, rowwise_ok

pytestmark = pytest.mark.gpu


def _fp8_exact_rows(rng, rows, cols, m_lo, m_hi):
    """bf16-exact rows whose per-row E4M3 quantisation is exact: one element
    +-448 * 2^m, the others 16 k 2^m with |k| <= 15, so the scale is 2^m and
    every scaled element is an E4M3 value."""
    m = rng.integers(m_lo, m_hi + 1, rows)
    v = 16.0 * rng.integers(-15, 16, (rows, cols))
    v[np.arange(rows), rng.integers(0, cols, rows)] = 448.0 * rng.choice([-1.0, 1.0], rows)
    return (v * np.exp2(m)[:, None]).astype(np.float32)


def _bf16_exact(a):
    return orc.round_bf16(np.asarray(a, dtype=np.float64)).astype(np.float32)


@pytest.mark.parametrize("dtype,cols", [
    ("bf16", 1024),   # 16-byte loads, row held in registers
    ("bf16", 5120),   # 16-byte loads, rest of the row re-read
    ("f32", 640),
    ("f32", 3000),    # 16-byte loads, rest of the row re-read
    ("bf16", 999),    # width without 16-byte chunks: one element per lane
    ("f32", 1023),
])
def test_quantize_e4m3_bit_exact(dtype, cols):
    require_gpu()
    rng = np.random.default_rng(11)
    rows = 41
    a = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 12, (rows, 1)))).astype(np.float32)
    if dtype == "bf16":
        a = _bf16_exact(a)
    # special values (each exact in bf16)
    a[3] = 0.0
    a[7, 5] = 2.0 ** -100  # far below the smallest code of its row
    a[9, 17] = np.nan      # scale 1, NaN -> 0x7F, the rest saturates or rounds
    a[11, 2] = np.inf      # scale inf: finite elements -> +-0, inf -> 0x7F
    a[13] = -0.0           # sign of zero kept
    a[13, 1] = 0.0
    if dtype == "f32":
        # largest magnitude below 448 * 2^-126: the scale is subnormal (2^-149
        # here) and the largest quotient 512 saturates
        a[15] = 0.0
        a[15, :4] = np.array([2.0 ** -140, -(2.0 ** -141), 2.0 ** -149, 3 * 2.0 ** -145])
        # the quotient max / 448 underflows to 0: scale 1, every code +-0
        a[17] = 0.0
        a[17, :3] = np.array([2.0 ** -146, -(2.0 ** -147), 2.0 ** -149])
        # maximum just above and just below 448 * 2^-126 (normal scale or not)
        a[19] *= np.float32(448.0 * 2.0 ** -126) / np.float32(np.abs(a[19]).max())
        a[21] *= np.float32(447.0 * 2.0 ** -126) / np.float32(np.abs(a[21]).max())
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.from_numpy(a).cuda().to(tdt)
    q, s = tw.quantize_e4m3(dev)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        rq, rs = orc.quantize_rows_e4m3(a)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_quantize_e4m3_rejects_misaligned_rows():
    """Inputs must start on a 16-byte boundary: an error, and nothing written."""
    require_gpu()
    buf = torch.zeros(64 * 8 + 1, dtype=torch.bfloat16, device="cuda")
    q = torch.full((64, 8), 0x55, dtype=torch.uint8, device="cuda")
    sc = torch.full((64,), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(tw.TwellError):
        tw.quantize_e4m3(buf[1:].view(64, 8), out=(q, sc))
    torch.cuda.synchronize()
    assert bool((q == 0x55).all()) and bool((sc == 7.0).all())


def _grid_codes(rng, shape):
    """E4M3 codes of k/8 for k in [-16, 16]: at most 4 significant bits."""
    vals = rng.integers(-16, 17, shape) / 8.0
    return orc.e4m3_encode(vals)


def _run_fp8(xq, sx, wq, sw, t, tile_n, slots, ovf_cap, g_dump=False):
    N, D = xq.shape
    F = wq.shape[0]
    dims = tw.make_dims(N, D, F, tile_n, slots, 0, ovf_cap, 0)
    pack = tw.alloc_pack(dims, tw.BF16)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    gd = torch.empty((N, F), dtype=torch.float32, device="cuda") if g_dump else None
    tw.gate_pack_fp8(dims, cu(xq), cu(sx), cu(wq), cu(sw), cu(t.astype(np.float32)), pack, g_dump=gd)
    torch.cuda.synchronize()
    return dims, pack, gd


@pytest.mark.parametrize("N,D,F,tile_n,slots", [(300, 256, 1000, 128, 4), (130, 128, 384, 64, 2), (520, 192, 700, 32, 3)])
def test_gate_pack_fp8_exact_grid(N, D, F, tile_n, slots):
    require_gpu()
    rng = np.random.default_rng(N + D + F)
    xq, wq = _grid_codes(rng, (N, D)), _grid_codes(rng, (F, D))
    sx = np.exp2(rng.integers(-3, 3, N)).astype(np.float32)
    sw = np.exp2(rng.integers(-3, 3, F)).astype(np.float32)
    g = orc.gate_preact_fp8(xq, sx, wq, sw)  # exact in fp32 for these operands
    t = orc.margin_thresholds(g, 0.05)
    ovf_cap = N
    dims, pack, gd = _run_fp8(xq, sx, wq, sw, t, tile_n, slots, ovf_cap, g_dump=True)
    np.testing.assert_array_equal(gd.cpu().numpy().astype(np.float64), g)
    pk = orc.pack(g, t, tile_n, slots, store="bf16", arith="f32")
    check_pack(pack, pk, ovf_cap)
    assert pk["n_ovf"] > 0
    hq = orc.dense_activation(g, t, store="bf16", arith="f32")
    n = min(pk["n_ovf"], ovf_cap)
    np.testing.assert_array_equal(f64(pack.ovf_h[:n]), hq[pk["ovf_rows"][:n]])


def test_gate_fp8_random_within_fp32_bound():
    require_gpu()
    rng = np.random.default_rng(21)
    N, D, F = 192, 1024, 520
    x = _bf16_exact(rng.standard_normal((N, D)))
    w = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(D))
    xq, sx = tw.quantize_e4m3(torch.from_numpy(x).cuda().to(torch.bfloat16))
    wq, sw = tw.quantize_e4m3(torch.from_numpy(w).cuda().to(torch.bfloat16))
    rxq, rsx = orc.quantize_rows_e4m3(x)
    rwq, rsw = orc.quantize_rows_e4m3(w)
    np.testing.assert_array_equal(xq.cpu().numpy(), rxq)
    np.testing.assert_array_equal(wq.cpu().numpy(), rwq)
    g = orc.gate_preact_fp8(rxq, rsx, rwq, rsw)
    t = np.full(N, 1e30, np.float32)  # nothing active: this test checks g only
    _, _, gd = _run_fp8(rxq, rsx, rwq, rsw, t, 128, 16, 64, g_dump=True)
    err = np.abs(gd.cpu().numpy().astype(np.float64) - g)
    bound = fp8_gate_err_bound(rxq, rsx, rwq, rsw, g)
    assert (err <= bound).all(), float((err / bound).max())


def test_forward_with_fp8_gate():
    """Quantisation on the GPU, the FP8 gate with the TwELL pack, then the bf16
    up / down projections, on rows whose quantisation and gate are exact:
    codes, scales, TwELL and the overflow rows bit-exact, y to fp32 accuracy."""
    require_gpu()
    rng = np.random.default_rng(31)
    N, D, F = 512, 512, 1536
    x = _fp8_exact_rows(rng, N, D, -8, -4)
    wg = _fp8_exact_rows(rng, F, D, -14, -10)
    wu = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(D))
    wd = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(F))
    rxq, rsx = orc.quantize_rows_e4m3(x)
    rwq, rsw = orc.quantize_rows_e4m3(wg)
    np.testing.assert_array_equal(orc.e4m3_decode(rxq) * rsx[:, None], x)  # exact quantisation
    g = orc.gate_preact_fp8(rxq, rsx, rwq, rsw)
    t = orc.margin_thresholds(g, 0.02)
    tile_n, slots, ovf_cap = 128, 8, N
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xb = cu(x).to(torch.bfloat16)
    xq, sx = tw.quantize_e4m3(xb)
    wq, sw = tw.quantize_e4m3(cu(wg).to(torch.bfloat16))
    dims = tw.make_dims(N, D, F, tile_n, slots, 0, ovf_cap, 0)
    pack = tw.alloc_pack(dims, tw.BF16)
    gd = torch.empty((N, F), dtype=torch.float32, device="cuda")
    tw.gate_pack_fp8(dims, xq, sx, wq, sw, cu(t), pack, g_dump=gd)
    sizes = tw.query_sizes(dims, tw.BF16)
    y = torch.empty((N, D), dtype=torch.float32, device="cuda")
    ws = tw.alloc_workspace(sizes["ws_fwd"])
    tw.ffn_fwd(dims, tw.BF16, pack, xb, cu(wu).to(torch.bfloat16), cu(wd).to(torch.bfloat16), y, ws=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq.cpu().numpy(), rxq)
    np.testing.assert_array_equal(sx.cpu().numpy(), rsx)
    np.testing.assert_array_equal(wq.cpu().numpy(), rwq)
    np.testing.assert_array_equal(gd.cpu().numpy().astype(np.float64), g)
    pk = orc.pack(g, t, tile_n, slots, store="bf16", arith="f32")
    check_pack(pack, pk, ovf_cap)
    hq = orc.dense_activation(g, t, store="bf16", arith="f32")
    n = min(pk["n_ovf"], ovf_cap)
    np.testing.assert_array_equal(f64(pack.ovf_h[:n]), hq[pk["ovf_rows"][:n]])
    y_ref = orc.sparse_forward(pk, x, wu, wd, ovf_h=hq[pk["ovf_rows"]])
    rowwise_ok(f64(y), y_ref, 1e-4, "y (fp8 gate)")


def test_runner_fp8_gate_matches_calls():
    """TwellFFN(fp8_gate=True) runs quantisation, FP8 gate + pack and the
    forward into its own buffers: y equal to the oracle on exact rows."""
    require_gpu()
    rng = np.random.default_rng(41)
    N, D, F = 300, 256, 1024
    x = _fp8_exact_rows(rng, N, D, -8, -4)
    wg = _fp8_exact_rows(rng, F, D, -12, -8)
    wu = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(D))
    wd = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(F))
    rxq, rsx = orc.quantize_rows_e4m3(x)
    rwq, rsw = orc.quantize_rows_e4m3(wg)
    g = orc.gate_preact_fp8(rxq, rsx, rwq, rsw)
    t = orc.margin_thresholds(g, 0.03)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dims = tw.make_dims(N, D, F, 128, 4, 0, N, 0)
    ffn = tw.TwellFFN(dims, tw.BF16, fp8_gate=True)
    wgate = tw.quantize_e4m3(cu(wg).to(torch.bfloat16))
    xb = cu(x).to(torch.bfloat16)
    for _ in range(2):   # the second call reuses every buffer
        y = ffn.forward(xb, wgate, cu(wu).to(torch.bfloat16), cu(wd).to(torch.bfloat16), cu(t))
        torch.cuda.synchronize()
        pk = orc.pack(g, t, 128, 4, store="bf16", arith="f32")
        check_pack(ffn.pack, pk, N)
        hq = orc.dense_activation(g, t, store="bf16", arith="f32")
        rowwise_ok(f64(y), orc.sparse_forward(pk, x, wu, wd, ovf_h=hq[pk["ovf_rows"]]), 1e-4, "y (runner)")
    with pytest.raises(ValueError):
        tw.TwellFFN(dims, tw.F32, fp8_gate=True)


@pytest.mark.parametrize("N", [1, 7, 33, 64])
def test_small_batch_fp8_gate_exact_grid(N):
    """The split-GEMV FP8 gate (gate_pack_fp8 with a workspace) on operands
    whose FP8 gate is exact: g, TwELL and the overflow rows bit-exact."""
    require_gpu()
    D, F, tile_n, slots = 512, 1000, 128, 4
    rng = np.random.default_rng(100 + N)
    xq, wq = _grid_codes(rng, (N, D)), _grid_codes(rng, (F, D))
    sx = np.exp2(rng.integers(-3, 3, N)).astype(np.float32)
    sw = np.exp2(rng.integers(-3, 3, F)).astype(np.float32)
    g = orc.gate_preact_fp8(xq, sx, wq, sw)
    t = orc.margin_thresholds(g, 0.05)
    dims = tw.make_dims(N, D, F, tile_n, slots, 0, N, 0)
    ws = tw.alloc_workspace(tw.query_sizes(dims, tw.BF16)["ws_gate"])
    pack = tw.alloc_pack(dims, tw.BF16)
    gd = torch.empty((N, F), dtype=torch.float32, device="cuda")
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tw.gate_pack_fp8(dims, cu(xq), cu(sx), cu(wq), cu(sw), cu(t), pack, g_dump=gd, ws=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gd.cpu().numpy().astype(np.float64), g)
    pk = orc.pack(g, t, tile_n, slots, store="bf16", arith="f32")
    check_pack(pack, pk, N)
    hq = orc.dense_activation(g, t, store="bf16", arith="f32")
    n = min(pk["n_ovf"], N)
    np.testing.assert_array_equal(f64(pack.ovf_h[:n]), hq[pk["ovf_rows"][:n]])


@pytest.mark.parametrize("N", [1, 40])
def test_small_batch_fp8_gate_random_within_bound(N):
    require_gpu()
    rng = np.random.default_rng(200 + N)
    D, F = 1024, 520
    x = _bf16_exact(rng.standard_normal((N, D)))
    w = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(D))
    rxq, rsx = orc.quantize_rows_e4m3(x)
    rwq, rsw = orc.quantize_rows_e4m3(w)
    g = orc.gate_preact_fp8(rxq, rsx, rwq, rsw)
    dims = tw.make_dims(N, D, F, 128, 16, 0, N, 0)
    ws = tw.alloc_workspace(tw.query_sizes(dims, tw.BF16)["ws_gate"])
    pack = tw.alloc_pack(dims, tw.BF16)
    gd = torch.empty((N, F), dtype=torch.float32, device="cuda")
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tw.gate_pack_fp8(dims, cu(rxq), cu(rsx), cu(rwq), cu(rsw), cu(np.full(N, 1e30, np.float32)), pack,
                     g_dump=gd, ws=ws)
    torch.cuda.synchronize()
    err = np.abs(gd.cpu().numpy().astype(np.float64) - g)
    bound = fp8_gate_err_bound(rxq, rsx, rwq, rsw, g)
    assert (err <= bound).all(), float((err / bound).max())


def test_runner_fp8_gate_small_batch():
    """TwellFFN(fp8_gate=True) at one token uses the small-batch FP8 gate:
    y against the oracle on an exactly quantisable row."""
    require_gpu()
    rng = np.random.default_rng(43)
    N, D, F = 1, 512, 2048
    x = _fp8_exact_rows(rng, N, D, -8, -4)
    wg = _fp8_exact_rows(rng, F, D, -12, -8)
    wu = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(D))
    wd = _bf16_exact(rng.standard_normal((F, D)) / np.sqrt(F))
    rxq, rsx = orc.quantize_rows_e4m3(x)
    rwq, rsw = orc.quantize_rows_e4m3(wg)
    g = orc.gate_preact_fp8(rxq, rsx, rwq, rsw)
    t = orc.margin_thresholds(g, 0.03)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dims = tw.make_dims(N, D, F, 128, 128, 0, 8, 0)
    ffn = tw.TwellFFN(dims, tw.BF16, fp8_gate=True)
    assert ffn.ws_gate is not None
    y = ffn.forward(cu(x).to(torch.bfloat16), tw.quantize_e4m3(cu(wg).to(torch.bfloat16)),
                    cu(wu).to(torch.bfloat16), cu(wd).to(torch.bfloat16), cu(t))
    torch.cuda.synchronize()
    pk = orc.pack(g, t, 128, 128, store="bf16", arith="f32")
    check_pack(ffn.pack, pk, 8)
    rowwise_ok(f64(y), orc.sparse_forward(pk, x, wu, wd), 1e-4, "y (small-batch FP8 gate)")
