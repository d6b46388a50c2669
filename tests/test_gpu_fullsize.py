"""Parity at the full workload sizes, in the launch configuration bench.py
times (same shapes, thresholds, capacities and kernels): sampled outputs are
recomputed one by one by the oracle, and properties that hold at any size are
checked on everything."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from activation_sparse_ffn_03_amd import twell as tw
from bench import capacities, workload_inputs
from oracle import twell_oracle as orc

from gpu_util import DELTA_REL, dev, f64, fp8_gate_err_bound, h_flip, require_gpu, rowwise_ok, u16

pytestmark = pytest.mark.gpu
Y_TOL = 1e-2


def _setup(name):
    require_gpu()
    w, train, _fp8 = workload_inputs(name)
    return w, train


def _sample_rows(N, extra, k=48, seed=7):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(k, N), replace=False).tolist()) | {0, 1, N - 2, N - 1}
    rows |= set(int(r) for r in extra[:16])
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["c2", "c3_5", "c3_1", "c3_05", "c4"])
def test_fullsize_forward(name):
    w, _ = _setup(name)
    print(f"[fullsize] {name}: N={w.N} D={w.D} F={w.F}", flush=True)
    ovf_cap, _ = capacities(w, False)
    dims = tw.make_dims(w.N, w.D, w.F, w.tile_n, w.slots, 0, ovf_cap, 0)
    ffn = tw.TwellFFN(dims, tw.BF16)
    x, wg, wu, wd = dev(w.x, "bf16"), dev(w.w_gate_t, "bf16"), dev(w.w_up_t, "bf16"), dev(w.w_down, "bf16")
    t = torch.from_numpy(w.t).cuda()
    y = ffn.forward(x, wg, wu, wd, t)
    torch.cuda.synchronize()
    assert int(ffn.pack.status.item()) == 0
    n_ovf = int(ffn.pack.n_ovf.item())
    ovf_rows = ffn.pack.ovf_rows[:n_ovf].cpu().numpy()
    # any-size properties: counts sum to a plausible density, overflow flags agree with counts
    counts = u16(ffn.pack.counts)
    assert abs(counts.sum() / (w.N * w.F) - w.p.mean()) < 0.1 * w.p.mean()
    flag = ffn.pack.ovf_flag.cpu().numpy().astype(bool)
    np.testing.assert_array_equal(flag, (counts > w.slots).any(0))
    np.testing.assert_array_equal(ovf_rows, np.nonzero(flag)[0])

    rows = _sample_rows(w.N, ovf_rows)
    fw = orc.ffn_forward(w.x[rows], w.w_gate_t, w.w_up_t, w.w_down, w.t[rows], store="bf16", arith="f32")
    slack = (h_flip(fw, "bf16") * np.abs(fw["a"])) @ np.abs(w.w_down.astype(np.float64))
    rowwise_ok(f64(y[torch.from_numpy(rows).cuda()]), fw["y"], Y_TOL, f"{name} y", slack)

    # pack of the sampled rows: bit-exact wherever no unit lies within the fp32 error of its threshold
    g = fw["g"]
    rms = np.sqrt(np.mean(g * g, axis=1))
    clean = np.all(np.abs(g - w.t[rows, None]) > DELTA_REL * rms[:, None], axis=1)
    assert clean.mean() > 0.9
    ref = orc.pack(g[clean].astype(np.float32), w.t[rows][clean], w.tile_n, w.slots, store="bf16", arith="f32")
    cr = rows[clean]
    np.testing.assert_array_equal(counts[:, cr], ref["counts"])
    S = w.slots
    valid = np.arange(S)[None, :, None] < np.minimum(ref["counts"], S)[:, None, :]
    cols = u16(ffn.pack.cols)[:, :, cr]
    np.testing.assert_array_equal(cols[valid], ref["cols"][valid])
    # stored values: the GPU's fp32 g may differ from fl32(g64) by up to delta_i = DELTA_REL * rms_i,
    # so Q(fl32(g - t)) may differ by that plus one bf16 rounding step on either side
    vals = f64(ffn.pack.vals)[:, :, cr]
    delta = np.broadcast_to((DELTA_REL * rms[clean])[None, None, :], valid.shape)[valid]
    rv = ref["vals"][valid]
    assert np.all(np.abs(vals[valid] - rv) <= 1.01 * delta + (np.abs(rv) + delta) * 2.0 ** -7)


@pytest.mark.parametrize("name", ["c2_dec1", "c2_dec16", "c2_dec64", "c3_dec1", "c3_dec64"])
def test_fullsize_decode(name):
    """The small-batch workloads as the benchmark runs them (S = T_n: no row
    can overflow, the gate is the split GEMV): every row against the oracle."""
    w, _ = _setup(name)
    assert w.slots >= w.tile_n and w.N <= 64
    print(f"[fullsize] {name}: N={w.N} D={w.D} F={w.F} S={w.slots}", flush=True)
    ovf_cap, _ = capacities(w, False)
    dims = tw.make_dims(w.N, w.D, w.F, w.tile_n, w.slots, 0, ovf_cap, 0)
    ffn = tw.TwellFFN(dims, tw.BF16)
    assert ffn.ws_gate is not None
    x, wg, wu, wd = dev(w.x, "bf16"), dev(w.w_gate_t, "bf16"), dev(w.w_up_t, "bf16"), dev(w.w_down, "bf16")
    y = ffn.forward(x, wg, wu, wd, torch.from_numpy(w.t).cuda())
    torch.cuda.synchronize()
    assert int(ffn.pack.status.item()) == 0 and int(ffn.pack.n_ovf.item()) == 0
    assert not bool(ffn.pack.ovf_flag.any())
    fw = orc.ffn_forward(w.x, w.w_gate_t, w.w_up_t, w.w_down, w.t, store="bf16", arith="f32")
    slack = (h_flip(fw, "bf16") * np.abs(fw["a"])) @ np.abs(w.w_down.astype(np.float64))
    rowwise_ok(f64(y), fw["y"], Y_TOL, f"{name} y", slack)
    # counts of every row whose units all lie outside the fp32 error of their threshold
    g = fw["g"]
    rms = np.sqrt(np.mean(g * g, axis=1))
    clean = np.all(np.abs(g - w.t[:, None]) > DELTA_REL * rms[:, None], axis=1)
    ref = orc.pack(g[clean].astype(np.float32), w.t[clean], w.tile_n, w.slots, store="bf16", arith="f32")
    np.testing.assert_array_equal(u16(ffn.pack.counts)[:, clean], ref["counts"])


@pytest.mark.parametrize("name,k", [("c2_fp8", 48), ("c3_1_fp8", 16), ("c3_dec1_fp8", 0), ("c3_dec64_fp8", 0)])
def test_fullsize_forward_fp8(name, k):
    """The FP8-gate workloads as the benchmark runs them (x quantised on the
    GPU, W_gate quantised once): sampled rows against the oracle's FP8 gate.
    A unit within the FP8 gate's error bound of its threshold may take either
    side, and a stored value either bf16 neighbour where its rounding is
    ambiguous within that bound; the slack allows both."""
    w, train, fp8 = workload_inputs(name)
    require_gpu()
    assert fp8 and not train
    print(f"[fullsize] {name}: N={w.N} D={w.D} F={w.F}", flush=True)
    ovf_cap, _ = capacities(w, False)
    dims = tw.make_dims(w.N, w.D, w.F, w.tile_n, w.slots, 0, ovf_cap, 0)
    ffn = tw.TwellFFN(dims, tw.BF16, fp8_gate=True)
    x, wg, wu, wd = dev(w.x, "bf16"), dev(w.w_gate_t, "bf16"), dev(w.w_up_t, "bf16"), dev(w.w_down, "bf16")
    y = ffn.forward(x, tw.quantize_e4m3(wg), wu, wd, torch.from_numpy(w.t).cuda())
    torch.cuda.synchronize()
    assert int(ffn.pack.status.item()) == 0
    n_ovf = int(ffn.pack.n_ovf.item())
    rows = np.arange(w.N) if w.N <= 64 else _sample_rows(w.N, ffn.pack.ovf_rows[:n_ovf].cpu().numpy(), k=k)
    wq, wsc = orc.quantize_rows_e4m3(w.w_gate_t)
    xq, xsc = orc.quantize_rows_e4m3(w.x[rows])
    g = orc.gate_preact_fp8(xq, xsc, wq, wsc)
    t = w.t[rows].astype(np.float64)
    bound = fp8_gate_err_bound(xq, xsc, wq, wsc, g)
    g32, t32 = g.astype(np.float32), w.t[rows].astype(np.float32)
    h = np.where(g32 > t32[:, None], (g32 - t32[:, None]).astype(np.float64), 0.0)
    hq = orc.dense_activation(g, w.t[rows], store="bf16", arith="f32")
    a = w.x[rows].astype(np.float64) @ w.w_up_t.astype(np.float64).T
    y_ref = (hq * a) @ w.w_down.astype(np.float64)
    near = np.abs(g - t[:, None]) <= bound                    # may flip either way
    amb = orc.rounding_ambiguous(h, bound + np.abs(h) * 2.0 ** -23, "bf16")
    dev_h = np.where(near, np.abs(g - t[:, None]) + bound, np.where(amb, orc.store_ulp(h, "bf16"), 0.0))
    slack = (dev_h * np.abs(a)) @ np.abs(w.w_down.astype(np.float64))
    rowwise_ok(f64(y[torch.from_numpy(rows).cuda()]), y_ref, Y_TOL, f"{name} y", slack)


def test_fullsize_training_step():
    w, train = _setup("c5")
    assert train
    print(f"[fullsize] c5 train: N={w.N} D={w.D} F={w.F}", flush=True)
    g64 = orc.gate_preact(w.x, w.w_gate_t)
    t = orc.margin_thresholds(g64, w.p)    # unique mask: no unit near its threshold
    assert orc.relative_margin(g64, t).min() > 1e-4
    ovf_cap, dense_cap = capacities(w, True)
    dims = tw.make_dims(w.N, w.D, w.F, w.tile_n, w.slots, w.row_cap, ovf_cap, dense_cap)
    ffn = tw.TwellFFN(dims, tw.BF16, train=True)
    x, wg, wu, wd, dy = (dev(a, "bf16") for a in (w.x, w.w_gate_t, w.w_up_t, w.w_down, w.dy))
    ffn.forward(x, wg, wu, wd, torch.from_numpy(t).cuda())
    dx, dwg, dwu, dwd = ffn.backward(x, dy, wg, wu, wd, w.lam)
    torch.cuda.synchronize()
    assert int(ffn.pack.status.item()) == 0 and int(ffn.hyb.status.item()) == 0
    # routing of every row (exact: the mask is unique)
    mask = g64 > t[:, None]
    nnz = mask.sum(1)
    counts = u16(ffn.pack.counts)
    np.testing.assert_array_equal(counts.sum(0), nnz)
    np.testing.assert_array_equal(ffn.hyb.row_nnz.cpu().numpy(), nnz)
    dense = (nnz > w.row_cap) | (counts > w.slots).any(0)
    np.testing.assert_array_equal(ffn.hyb.is_dense.cpu().numpy().astype(bool), dense)
    nd = int(ffn.hyb.n_dense.item())
    np.testing.assert_array_equal(ffn.hyb.dense_rows[:nd].cpu().numpy(), np.nonzero(dense)[0])
    assert nd > 0

    # dx on sampled rows (including dense-backup rows)
    rows = _sample_rows(w.N, np.nonzero(dense)[0])
    fr = orc.ffn_forward(w.x[rows], w.w_gate_t, w.w_up_t, w.w_down, t[rows], store="bf16", arith="f32")
    br = orc.ffn_backward(w.x[rows], w.dy[rows], w.w_gate_t, w.w_up_t, w.w_down, fr["mask"], fr["hq"], w.lam)
    dh = h_flip(fr, "bf16")
    slack = (dh * np.abs(br["dz"])) @ np.abs(w.w_up_t.astype(np.float64))
    rowwise_ok(f64(dx[torch.from_numpy(rows).cuda()]), br["dx"], Y_TOL, "c5 dx", slack)

    # weight gradients on sampled columns (each depends on all tokens of its column only)
    rng = np.random.default_rng(11)
    cols = np.sort(rng.choice(w.F, size=32, replace=False))
    fc = orc.ffn_forward(w.x, w.w_gate_t[cols], w.w_up_t[cols], w.w_down[cols], t, store="bf16", arith="f32")
    bc = orc.ffn_backward(w.x, w.dy, w.w_gate_t[cols], w.w_up_t[cols], w.w_down[cols], fc["mask"], fc["hq"], w.lam)
    dhc = h_flip(fc, "bf16")
    ci = torch.from_numpy(cols).cuda()
    rowwise_ok(f64(dwg[ci]), bc["dw_gate_t"], Y_TOL, "c5 dW_gate")
    rowwise_ok(f64(dwu[ci]), bc["dw_up_t"], Y_TOL, "c5 dW_up",
               (dhc * np.abs(bc["dz"])).T @ np.abs(w.x.astype(np.float64)))
    rowwise_ok(f64(dwd[ci]), bc["dw_down"], Y_TOL, "c5 dW_down",
               (dhc * np.abs(fc["a"])).T @ np.abs(w.dy.astype(np.float64)))


def _hybrid_mask_h(ffn, w, rows=None, cols=None):
    """The GPU's own mask and stored activation, read back from the hybrid
    format the backward consumes: the row-ELL (positions < row_nnz) for ELL
    rows and the dense-backup rows (active iff the stored h > 0, the rule the
    backward applies to them). Returns (mask, hq) restricted to `rows` (all
    columns) or to `cols` (all rows)."""
    N, F = w.N, w.F
    K = w.row_cap
    row_nnz = ffn.hyb.row_nnz.cpu().numpy().astype(np.int64)
    is_dense = ffn.hyb.is_dense.cpu().numpy().astype(bool)
    nd = int(ffn.hyb.n_dense.item())
    dense_rows = ffn.hyb.dense_rows[:nd].cpu().numpy().astype(np.int64)
    pos = np.full(N, -1, dtype=np.int64)
    pos[dense_rows] = np.arange(nd)
    ell_cols = ffn.hyb.ell_cols.cpu().numpy().astype(np.int64)        # [K][N]
    ell_vals = f64(ffn.hyb.ell_vals)                                  # [K][N]
    valid = (np.arange(K)[:, None] < row_nnz[None, :]) & ~is_dense[None, :]
    if rows is not None:
        sel_rows, sel_cols = rows, np.arange(F)
    else:
        sel_rows, sel_cols = np.arange(N), cols
    colmap = np.full(F, -1, dtype=np.int64)
    colmap[sel_cols] = np.arange(sel_cols.size)
    rowmap = np.full(N, -1, dtype=np.int64)
    rowmap[sel_rows] = np.arange(sel_rows.size)
    hq = np.zeros((sel_rows.size, sel_cols.size))
    k_idx, i_idx = np.nonzero(valid)
    c_idx = ell_cols[k_idx, i_idx]
    assert ((c_idx >= 0) & (c_idx < F)).all()
    keep = (rowmap[i_idx] >= 0) & (colmap[c_idx] >= 0)
    hq[rowmap[i_idx[keep]], colmap[c_idx[keep]]] = ell_vals[k_idx[keep], i_idx[keep]]
    mask = np.zeros(hq.shape, dtype=bool)
    mask[rowmap[i_idx[keep]], colmap[c_idx[keep]]] = True
    dsel = [(r, pos[r]) for r in sel_rows if is_dense[r]]
    if dsel:
        dr = np.array([r for r, _ in dsel])
        dh = f64(ffn.hyb.dense_h[torch.from_numpy(np.array([p for _, p in dsel])).cuda()])[:, sel_cols]
        hq[rowmap[dr]] = dh
        mask[rowmap[dr]] = dh > 0
    # ascending global columns in every ELL row, and positive stored values
    assert (hq[mask] > 0).all()
    return mask, hq


def test_fullsize_training_step_benchmark_thresholds():
    """The training step exactly as bench.py times it: the generator's own
    per-token thresholds (units may sit arbitrarily close to them), the
    bench's capacities. The mask and the stored activation the backward uses
    are read back from the GPU's hybrid format and fed to the oracle's
    backward (ReLU' jumps at the threshold, so a near-threshold unit may fall
    on either side; its h there is tiny). Checked: routing of every row; the
    GPU mask against the oracle's fp64 g (disagreements only within the fp32
    evaluation error of the threshold); the hybrid against the TwELL pack on
    sampled rows; y and dx on sampled rows (dense-backup and overflow rows
    included) and dW_gate, dW_up, dW_down on sampled columns, each within
    1e-2 * rms of the oracle per row."""
    w, train = _setup("c5")
    assert train
    print(f"[fullsize] c5 train, benchmark thresholds: N={w.N} D={w.D} F={w.F}", flush=True)
    ovf_cap, dense_cap = capacities(w, True)
    dims = tw.make_dims(w.N, w.D, w.F, w.tile_n, w.slots, w.row_cap, ovf_cap, dense_cap)
    ffn = tw.TwellFFN(dims, tw.BF16, train=True)
    x, wg, wu, wd, dy = (dev(a, "bf16") for a in (w.x, w.w_gate_t, w.w_up_t, w.w_down, w.dy))
    y = ffn.forward(x, wg, wu, wd, torch.from_numpy(w.t).cuda())
    dx, dwg, dwu, dwd = ffn.backward(x, dy, wg, wu, wd, w.lam)
    torch.cuda.synchronize()
    assert int(ffn.pack.status.item()) == 0 and int(ffn.hyb.status.item()) == 0

    # routing of every row from the GPU's own counts
    counts = u16(ffn.pack.counts)                                     # [n_t][N]
    nnz = counts.sum(0)
    np.testing.assert_array_equal(ffn.hyb.row_nnz.cpu().numpy(), nnz)
    dense = (nnz > w.row_cap) | (counts > w.slots).any(0)
    np.testing.assert_array_equal(ffn.hyb.is_dense.cpu().numpy().astype(bool), dense)
    nd = int(ffn.hyb.n_dense.item())
    np.testing.assert_array_equal(ffn.hyb.dense_rows[:nd].cpu().numpy(), np.nonzero(dense)[0])
    assert nd > 0
    n_ovf = int(ffn.pack.n_ovf.item())
    ovf_rows = ffn.pack.ovf_rows[:n_ovf].cpu().numpy()
    assert n_ovf > 0

    rows = _sample_rows(w.N, np.concatenate([np.nonzero(dense)[0], ovf_rows]), k=40)
    mask_r, hq_r = _hybrid_mask_h(ffn, w, rows=rows)

    # the hybrid holds what the pack holds (ELL rows: slots in tile order, columns ascending)
    vals, cols = f64(ffn.pack.vals), u16(ffn.pack.cols)
    T, S = w.tile_n, w.slots
    for r_i, r in enumerate(rows):
        if dense[r]:
            continue
        want = np.zeros(w.F)
        for j in range(counts.shape[0]):
            c = int(counts[j, r])
            want[j * T + cols[j, :c, r]] = vals[j, :c, r]
        np.testing.assert_array_equal(hq_r[r_i], want, err_msg=f"hybrid vs pack, row {r}")

    # the GPU mask against the oracle's g: disagreements only within the fp32 error of the threshold
    g64 = orc.gate_preact(w.x[rows], w.w_gate_t)
    t64 = w.t[rows].astype(np.float64)
    ref_mask = g64 > t64[:, None]
    rms_g = np.sqrt(np.mean(g64 * g64, axis=1))
    near = np.abs(g64 - t64[:, None]) <= DELTA_REL * rms_g[:, None]
    flips = mask_r != ref_mask
    assert not (flips & ~near).any(), "mask differs from the oracle away from the threshold"
    print(f"[fullsize] c5 benchmark thresholds: {int(flips.sum())} near-threshold mask flips in "
          f"{rows.size} sampled rows, {int(near.sum())} units within the fp32 band", flush=True)
    # the stored activation where both agree: Q(fl32(g) - t), up to the fp32
    # evaluation error of g (relatively large where g - t is small) plus one
    # rounding to bf16
    fw = orc.ffn_forward(w.x[rows], w.w_gate_t, w.w_up_t, w.w_down, w.t[rows], store="bf16", arith="f32")
    both = mask_r & ref_mask
    dh = np.abs(hq_r - fw["hq"])
    allowed = DELTA_REL * rms_g[:, None] + orc.store_ulp(np.maximum(np.abs(hq_r), np.abs(fw["hq"])), "bf16")
    assert (dh[both] <= allowed[both]).all(), "stored activation beyond the fp32 error of g plus one bf16 ulp"
    print(f"[fullsize] c5 benchmark thresholds: stored h differs from the oracle's in {int((dh[both] > 0).sum())} "
          f"of {int(both.sum())} active units (largest {float((dh / allowed)[both].max()):.3f} of the bound)",
          flush=True)

    # y and dx of the sampled rows from the GPU's mask and h
    a_r = fw["a"]
    y_ref = (hq_r * a_r) @ w.w_down.astype(np.float64)
    rowwise_ok(f64(y[torch.from_numpy(rows).cuda()]), y_ref, Y_TOL, "c5 (benchmark thresholds) y")
    br = orc.ffn_backward(w.x[rows], w.dy[rows], w.w_gate_t, w.w_up_t, w.w_down, mask_r, hq_r, w.lam)
    rowwise_ok(f64(dx[torch.from_numpy(rows).cuda()]), br["dx"], Y_TOL, "c5 (benchmark thresholds) dx")

    # weight gradients on sampled columns, over every token, from the GPU's mask and h
    rng = np.random.default_rng(13)
    ccols = np.sort(rng.choice(w.F, size=24, replace=False))
    mask_c, hq_c = _hybrid_mask_h(ffn, w, cols=ccols)
    bc = orc.ffn_backward(w.x, w.dy, w.w_gate_t[ccols], w.w_up_t[ccols], w.w_down[ccols], mask_c, hq_c, w.lam)
    ci = torch.from_numpy(ccols).cuda()
    rowwise_ok(f64(dwg[ci]), bc["dw_gate_t"], Y_TOL, "c5 (benchmark thresholds) dW_gate")
    rowwise_ok(f64(dwu[ci]), bc["dw_up_t"], Y_TOL, "c5 (benchmark thresholds) dW_up")
    rowwise_ok(f64(dwd[ci]), bc["dw_down"], Y_TOL, "c5 (benchmark thresholds) dW_down")
