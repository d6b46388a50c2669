"""Pins for the CPU oracle, checked against things other than the oracle itself:
hand-worked fixtures, brute-force enumeration, torch float64 autograd, finite
differences, closed forms, metamorphic invariants and torch's bf16 cast."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import twell_oracle as orc
from synth import make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_bf16(a.astype(np.float64)), ref)


def test_round_bf16_ties_and_signs():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert orc.round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: the even one is 1+2^-6
    assert orc.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert orc.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -20)) == -(1.0 + 2.0 ** -7)
    assert orc.round_bf16(0.0) == 0.0
    # fp64 values between fp32 neighbours round directly (no double rounding):
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30   # just above the tie -> up
    assert orc.round_bf16(v) == 1.0 + 2.0 ** -7


# ----------------------------------------------------------------- dense forward

def test_forward_handworked():
    f = _load("ffn_handworked.json")
    out = orc.ffn_forward(f["x"], f["w_gate_t"], f["w_up_t"], f["w_down"], f["t"], store="exact")
    for k in ("g", "h", "a", "z", "y"):
        np.testing.assert_array_equal(out[k], np.array(f["expect"][k]), err_msg=k)


def test_backward_handworked():
    f = _load("ffn_handworked.json")
    fw = orc.ffn_forward(f["x"], f["w_gate_t"], f["w_up_t"], f["w_down"], f["t"], store="exact")
    bw = orc.ffn_backward(f["x"], f["dy"], f["w_gate_t"], f["w_up_t"], f["w_down"], fw["mask"], fw["hq"], f["lam"])
    loss = float(np.sum(np.array(f["dy"]) * fw["y"]) + f["lam"] * fw["h"].sum())
    assert loss == f["expect"]["loss"]
    for k in ("dx", "dw_gate_t", "dw_up_t", "dw_down"):
        np.testing.assert_array_equal(bw[k], np.array(f["expect"][k]), err_msg=k)


def _tiny(seed, N=5, D=6, F=9, p=0.4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, D))
    wg = rng.standard_normal((F, D)) / math.sqrt(D)
    wu = rng.standard_normal((F, D)) / math.sqrt(D)
    wd = rng.standard_normal((F, D)) / math.sqrt(F)
    dy = rng.standard_normal((N, D))
    g = x @ wg.T
    t = np.quantile(g, 1 - p, axis=1)
    return x, wg, wu, wd, dy, t


def test_forward_textbook_regelu_at_zero_threshold():
    # t = 0 reduces the block to a textbook ReLU-gated (ReGLU) FFN built from torch.nn.functional
    x, wg, wu, wd, _, _ = _tiny(2)
    out = orc.ffn_forward(x, wg, wu, wd, np.zeros(x.shape[0]), store="exact")
    X = torch.from_numpy(x)
    ref = torch.nn.functional.linear(
        torch.relu(torch.nn.functional.linear(X, torch.from_numpy(wg))) * torch.nn.functional.linear(X, torch.from_numpy(wu)),
        torch.from_numpy(wd).T)
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_forward_closed_forms():
    x, wg, wu, wd, _, _ = _tiny(3)
    # threshold above every g: nothing is active, y == 0 exactly
    out = orc.ffn_forward(x, wg, wu, wd, np.full(x.shape[0], 1e9), store="exact")
    assert not out["mask"].any() and np.all(out["y"] == 0)
    # threshold below every g: every unit active, h = g - t everywhere
    t = np.full(x.shape[0], -1e3)
    out = orc.ffn_forward(x, wg, wu, wd, t, store="exact")
    assert out["mask"].all()


def test_forward_metamorphic():
    x, wg, wu, wd, _, t = _tiny(4, N=6, D=7, F=11)
    y = orc.ffn_forward(x, wg, wu, wd, t, store="exact")["y"]
    # consistent permutation of the d_ff units leaves y unchanged
    perm = np.random.default_rng(0).permutation(wg.shape[0])
    yp = orc.ffn_forward(x, wg[perm], wu[perm], wd[perm], t, store="exact")["y"]
    np.testing.assert_allclose(yp, y, rtol=1e-12, atol=1e-12)
    # token permutation permutes rows of y
    tp = np.random.default_rng(1).permutation(x.shape[0])
    yt = orc.ffn_forward(x[tp], wg, wu, wd, t[tp], store="exact")["y"]
    np.testing.assert_allclose(yt, y[tp], rtol=1e-12, atol=1e-12)
    # linear in W_down and in W_up^T
    y2 = orc.ffn_forward(x, wg, 3.0 * wu, -2.0 * wd, t, store="exact")["y"]
    np.testing.assert_allclose(y2, -6.0 * y, rtol=1e-12, atol=1e-12)
    # (x, t) -> (alpha x, alpha t) scales y by alpha^2 (h and a both scale by alpha)
    y3 = orc.ffn_forward(2.5 * x, wg, wu, wd, 2.5 * t, store="exact")["y"]
    np.testing.assert_allclose(y3, 6.25 * y, rtol=1e-12, atol=1e-12)


def test_forward_brute_force_scalar_loops():
    x, wg, wu, wd, _, t = _tiny(5, N=3, D=4, F=6)
    y = orc.ffn_forward(x, wg, wu, wd, t, store="exact")["y"]
    N, D = x.shape
    F = wg.shape[0]
    for i in range(N):
        for d in range(D):
            acc = 0.0
            for c in range(F):
                gic = sum(x[i, k] * wg[c, k] for k in range(D))
                aic = sum(x[i, k] * wu[c, k] for k in range(D))
                acc += max(gic - t[i], 0.0) * aic * wd[c, d]
            assert abs(acc - y[i, d]) < 1e-12


# ----------------------------------------------------------------- backward

def _torch_grads(x, wg, wu, wd, dy, t, lam):
    X = torch.tensor(x, requires_grad=True)
    WG = torch.tensor(wg, requires_grad=True)
    WU = torch.tensor(wu, requires_grad=True)
    WD = torch.tensor(wd, requires_grad=True)
    h = torch.relu(X @ WG.T - torch.tensor(t)[:, None])
    y = (h * (X @ WU.T)) @ WD
    loss = (torch.tensor(dy) * y).sum() + lam * h.sum()
    loss.backward()
    return X.grad.numpy(), WG.grad.numpy(), WU.grad.numpy(), WD.grad.numpy()


@pytest.mark.parametrize("seed", [6, 7, 8])
def test_backward_matches_torch_autograd(seed):
    x, wg, wu, wd, dy, t = _tiny(seed, N=7, D=8, F=13)
    lam = 0.3
    fw = orc.ffn_forward(x, wg, wu, wd, t, store="exact")
    bw = orc.ffn_backward(x, dy, wg, wu, wd, fw["mask"], fw["hq"], lam)
    gx, gg, gu, gd = _torch_grads(x, wg, wu, wd, dy, t, lam)
    for got, ref in ((bw["dx"], gx), (bw["dw_gate_t"], gg), (bw["dw_up_t"], gu), (bw["dw_down"], gd)):
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_backward_finite_differences():
    x, wg, wu, wd, dy, _ = _tiny(9, N=4, D=5, F=7)
    g = x @ wg.T
    # threshold in the middle of a wide gap so no unit crosses it under the perturbation
    t = np.array([0.5 * (np.sort(r)[3] + np.sort(r)[4]) for r in g])
    assert np.min(np.abs(g - t[:, None])) > 1e-3
    lam = 0.2

    def loss(x_, wg_, wu_, wd_):
        fw = orc.ffn_forward(x_, wg_, wu_, wd_, t, store="exact")
        return float(np.sum(dy * fw["y"]) + lam * fw["h"].sum())

    fw = orc.ffn_forward(x, wg, wu, wd, t, store="exact")
    bw = orc.ffn_backward(x, dy, wg, wu, wd, fw["mask"], fw["hq"], lam)
    eps = 1e-6
    args = [x, wg, wu, wd]
    for idx, key in enumerate(("dx", "dw_gate_t", "dw_up_t", "dw_down")):
        base = args[idx]
        num = np.zeros_like(base)
        for pos in itertools.product(*[range(s) for s in base.shape]):
            up = [a.copy() for a in args]
            dn = [a.copy() for a in args]
            up[idx][pos] += eps
            dn[idx][pos] -= eps
            num[pos] = (loss(*up) - loss(*dn)) / (2 * eps)
        np.testing.assert_allclose(bw[key], num, rtol=1e-6, atol=1e-7, err_msg=key)


def test_backward_closed_forms():
    x, wg, wu, wd, dy, t = _tiny(10, N=6, D=5, F=8)
    lam = 0.7
    fw = orc.ffn_forward(x, wg, wu, wd, t, store="exact")
    m = fw["mask"].astype(np.float64)
    bw = orc.ffn_backward(x, np.zeros_like(dy), wg, wu, wd, fw["mask"], fw["hq"], lam)
    # with dy = 0 only the L1 term acts: dg = lam on active units
    np.testing.assert_allclose(bw["dw_gate_t"], lam * m.T @ x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(bw["dx"], lam * m @ wg, rtol=1e-13, atol=1e-13)
    assert np.all(bw["dw_up_t"] == 0) and np.all(bw["dw_down"] == 0)
    # nothing active: every gradient is zero
    fw0 = orc.ffn_forward(x, wg, wu, wd, np.full(x.shape[0], 1e9), store="exact")
    bw0 = orc.ffn_backward(x, dy, wg, wu, wd, fw0["mask"], fw0["hq"], lam)
    for k in ("dx", "dw_gate_t", "dw_up_t", "dw_down"):
        assert np.all(bw0[k] == 0)


# ----------------------------------------------------------------- TwELL pack

def test_pack_handworked():
    f = _load("twell_pack_handworked.json")
    pk = orc.pack(np.array(f["g"]), np.array(f["t"]), f["tile_n"], f["slots"], store="bf16")
    e = f["expect"]
    assert orc.n_tiles(6, f["tile_n"]) == e["n_tiles"]
    np.testing.assert_array_equal(pk["counts"], e["counts"])
    for j in range(e["n_tiles"]):
        for s in range(f["slots"]):
            for i in range(2):
                if e["vals"][j][s][i] is not None:
                    assert pk["vals"][j, s, i] == e["vals"][j][s][i]
                    assert pk["cols"][j, s, i] == e["cols"][j][s][i]
    np.testing.assert_array_equal(pk["ovf_flag"], e["ovf_flag"])
    np.testing.assert_array_equal(pk["ovf_rows"], e["ovf_rows"])
    dense = orc.dense_activation(np.array(f["g"]), np.array(f["t"]), "bf16")
    np.testing.assert_array_equal(dense, e["dense_h"])
    # round trip with the overflow row supplied densely
    np.testing.assert_array_equal(orc.unpack(pk, dense[pk["ovf_rows"]]), e["dense_h"])


def test_route_handworked():
    f = _load("twell_pack_handworked.json")
    g, t = np.array(f["g"]), np.array(f["t"])
    pk = orc.pack(g, t, 4, 2)
    dense = orc.dense_activation(g, t)
    r = orc.route(pk, 2, ovf_h=dense[pk["ovf_rows"]])
    np.testing.assert_array_equal(r["row_nnz"], f["route_k2"]["row_nnz"])
    np.testing.assert_array_equal(r["dense_rows"], f["route_k2"]["dense_rows"])
    np.testing.assert_array_equal(r["ell_cols"][:, 1], f["route_k2"]["ell_cols_row1"])
    np.testing.assert_array_equal(r["ell_vals"][:, 1], f["route_k2"]["ell_vals_row1"])
    np.testing.assert_array_equal(r["dense_h"], dense[[0]])
    pk4 = orc.pack(g, t, 4, 4)
    r4 = orc.route(pk4, 4)
    assert r4["n_dense"] == 0
    np.testing.assert_array_equal(r4["ell_cols"][:, 0], f["route_k4_s4"]["ell_cols_row0"])
    np.testing.assert_array_equal(r4["ell_vals"][:, 0], f["route_k4_s4"]["ell_vals_row0"])
    np.testing.assert_array_equal(r4["ell_cols"][:2, 1], f["route_k4_s4"]["ell_cols_row1"][:2])


def _expected_pack_by_loops(pattern, tile_n, slots):
    """Independent scalar construction: walk each row's columns left to right."""
    N, F = pattern.shape
    nt = -(-F // tile_n)
    entries = {}
    counts = np.zeros((nt, N), dtype=np.int64)
    for i in range(N):
        for j in range(nt):
            s = 0
            for c in range(j * tile_n, min(F, (j + 1) * tile_n)):
                if pattern[i, c]:
                    if s < slots:
                        entries[(j, s, i)] = c - j * tile_n
                    s += 1
            counts[j, i] = s
    return nt, counts, entries


@pytest.mark.parametrize("F", [1, 5, 8, 11])
def test_pack_brute_force_all_patterns(F):
    patterns = np.array(list(itertools.product([False, True], repeat=F)))
    # distinct positive gate values for active units, non-positive otherwise; t = 0
    base = 1.0 + np.arange(F) / 64.0
    g = np.where(patterns, base, -base * 0.5)
    t = np.zeros(len(patterns))
    for tile_n in (1, 2, 3, 4, 8):
        for slots in range(0, min(tile_n, 4) + 1):
            pk = orc.pack(g, t, tile_n, slots, store="bf16")
            nt, counts, entries = _expected_pack_by_loops(patterns, tile_n, slots)
            assert pk["vals"].shape[0] == nt == math.ceil(F / tile_n)
            np.testing.assert_array_equal(pk["counts"], counts)
            np.testing.assert_array_equal(pk["counts"].sum(0), patterns.sum(1))
            for (j, s, i), c in entries.items():
                assert pk["cols"][j, s, i] == c
                assert pk["vals"][j, s, i] == orc.round_bf16(g[i, j * tile_n + c])
            # every slot beyond min(cnt, S) stays at the don't-care marker
            filled = np.zeros_like(pk["cols"], dtype=bool)
            for (j, s, i) in entries:
                filled[j, s, i] = True
            assert np.all(pk["cols"][~filled] == -1)
            np.testing.assert_array_equal(pk["ovf_flag"], (counts > slots).any(0))
            np.testing.assert_array_equal(pk["ovf_rows"], np.nonzero((counts > slots).any(0))[0])
            dense = orc.dense_activation(g, t)
            np.testing.assert_array_equal(orc.unpack(pk, dense[pk["ovf_rows"]]), dense)


def test_pack_strict_threshold_and_signed_zero():
    g = np.array([[0.0, -0.0, 1e-30, -1e-30, 2.0, 2.0]], dtype=np.float32)
    t = np.array([0.0], dtype=np.float32)
    pk = orc.pack(g, t, 8, 8, store="f32")
    assert pk["counts"][0, 0] == 3   # 1e-30 and both 2.0 are above 0; +0 and -0 tie and stay inactive
    np.testing.assert_array_equal(pk["cols"][0, :3, 0], [2, 4, 5])
    t2 = np.array([2.0], dtype=np.float32)
    assert orc.pack(g, t2, 8, 8)["counts"][0, 0] == 0


def test_pack_fp32_subtraction_is_ieee():
    # vals are Q(fl32(g - t)): pick g, t whose exact difference is not an fp32 value
    g = np.array([[1.0 + 2.0 ** -23]], dtype=np.float32)
    t = np.array([2.0 ** -25], dtype=np.float32)
    pk = orc.pack(g, t, 4, 4, store="f32")
    ref = (np.float32(g[0, 0]) - np.float32(t[0]))
    assert pk["vals"][0, 0, 0] == float(ref)
    assert float(ref) != float(g[0, 0]) - float(t[0])


@pytest.mark.parametrize("tile_n,slots", [(16, 0), (16, 1), (16, 4), (64, 16), (7, 3), (300, 300)])
def test_sparse_path_equals_dense_path(tile_n, slots):
    w = make_inputs("c1", density=0.08, N=40, D=64, F=300)
    fw = orc.ffn_forward(w.x, w.w_gate_t, w.w_up_t, w.w_down, w.t, store="bf16")
    pk = orc.pack(fw["g"], w.t, tile_n, slots, store="bf16", arith="f64")
    ovf_h = fw["hq"][pk["ovf_rows"]]
    np.testing.assert_array_equal(orc.unpack(pk, ovf_h), fw["hq"])
    ys = orc.sparse_forward(pk, w.x, w.w_up_t, w.w_down, ovf_h)
    np.testing.assert_array_equal(ys, fw["y"])
    assert pk["counts"].sum() == fw["mask"].sum()
    if slots == 0:
        assert pk["n_ovf"] == int((fw["mask"].sum(1) > 0).sum())


def test_route_invariants():
    w = make_inputs("c5", N=64, D=64, F=512, row_cap=12)
    fw = orc.ffn_forward(w.x, w.w_gate_t, w.w_up_t, w.w_down, w.t)
    pk = orc.pack(fw["g"], w.t, 64, 4, arith="f64")
    r = orc.route(pk, w.row_cap, a=fw["a"], ovf_h=fw["hq"][pk["ovf_rows"]])
    ell = ~r["is_dense"]
    assert r["n_dense"] > 0 and ell.any()
    np.testing.assert_array_equal(r["dense_rows"], np.nonzero(r["is_dense"])[0])
    np.testing.assert_array_equal(r["row_nnz"], fw["mask"].sum(1))
    assert np.all(r["row_nnz"][ell] <= w.row_cap)
    assert np.all(r["is_dense"] >= pk["ovf_flag"])
    # ELL rows rebuild exactly, with ascending columns; saved a sits beside each entry
    for i in np.nonzero(ell)[0]:
        n = r["row_nnz"][i]
        c = r["ell_cols"][:n, i]
        assert np.all(np.diff(c) > 0)
        np.testing.assert_array_equal(c, np.nonzero(fw["mask"][i])[0])
        np.testing.assert_array_equal(r["ell_vals"][:n, i], fw["hq"][i, c])
        np.testing.assert_array_equal(r["ell_a"][:n, i], fw["a"][i, c])
    np.testing.assert_array_equal(r["dense_h"], fw["hq"][r["dense_rows"]])


# ----------------------------------------------------------------- generator and helpers

def test_generator_density_and_threshold():
    w = make_inputs("c2", N=256, D=2048, F=5632)
    g = orc.gate_preact(w.x, w.w_gate_t)
    nnz = (g > w.t[:, None].astype(np.float64)).sum(1)
    expect = w.p * w.F
    sd = np.sqrt(w.F * w.p * (1 - w.p))
    # mean over rows within 4 standard errors; ~56 active per token at 1% of 5632
    assert abs(nnz.mean() - expect.mean()) < 4 * sd.mean() / math.sqrt(len(nnz))
    assert 50 < nnz.mean() < 63


def test_generator_lognormal_moments():
    w = make_inputs("c4", N=20000, D=64, F=64)
    p = w.p
    assert p.min() >= 0.001 and p.max() <= 0.30
    assert abs(p.mean() - 0.01) < 0.0006
    assert abs(np.median(p) - math.exp(math.log(0.01) - 0.5)) < 0.0004


def test_generator_is_seeded_and_rounded():
    a = make_inputs("c1")
    b = make_inputs("c1")
    np.testing.assert_array_equal(a.x, b.x)
    c = make_inputs("c2", N=8, D=64, F=128)
    np.testing.assert_array_equal(orc.round_bf16(c.w_gate_t.astype(np.float64)), c.w_gate_t)


def test_margin_thresholds():
    w = make_inputs("c5", N=32, D=256, F=1024)
    g = orc.gate_preact(w.x, w.w_gate_t)
    t = orc.margin_thresholds(g, w.p)
    rm = orc.relative_margin(g, t)
    assert rm.min() > 1e-4
    nnz = (g > t[:, None]).sum(1)
    k = np.maximum(1, np.round(w.p * w.F))
    assert np.all(np.abs(nnz - k) <= np.maximum(2, 0.25 * k) + 1)


def test_rowwise_rel_err():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    got = np.array([[3.0, 4.1], [0.0, 0.0]])
    e = orc.rowwise_rel_err(got, ref)
    assert abs(e[0] - 0.1 / math.sqrt(12.5)) < 1e-12 and e[1] == 0
    assert orc.rowwise_rel_err(np.array([[0.0, 1e-9]]), np.zeros((1, 2)))[0] == np.inf


# ----------------------------------------------------------------- fp32-formed activation, rounding helpers

def test_forward_f32_arith_equals_f32_pack():
    # the dense activation formed as Q(fl32(fl32(g) - t)) equals the packed one (same definition, two codes)
    w = make_inputs("c2", N=50, D=128, F=300, density=0.1)
    fw = orc.ffn_forward(w.x, w.w_gate_t, w.w_up_t, w.w_down, w.t, store="bf16", arith="f32")
    pk = orc.pack(fw["g"].astype(np.float32), w.t, 64, 8, store="bf16", arith="f32")
    np.testing.assert_array_equal(orc.unpack(pk, fw["hq"][pk["ovf_rows"]]), fw["hq"])
    ys = orc.sparse_forward(pk, w.x, w.w_up_t, w.w_down, fw["hq"][pk["ovf_rows"]])
    np.testing.assert_array_equal(ys, fw["y"])
    # the two arithmetics differ only by fp32 rounding of g - t
    f64 = orc.ffn_forward(w.x, w.w_gate_t, w.w_up_t, w.w_down, w.t, store="exact", arith="f64")
    f32 = orc.ffn_forward(w.x, w.w_gate_t, w.w_up_t, w.w_down, w.t, store="exact", arith="f32")
    both = f64["mask"] & f32["mask"]
    assert np.all(np.abs(f64["h"][both] - f32["h"][both]) <= 2.0 ** -20 * (1 + np.abs(f64["g"][both])))


def test_grid_inputs_make_gate_exact_in_fp32():
    w = make_inputs("c5", N=64, D=8192, F=64, grid=True)
    g = orc.gate_preact(w.x, w.w_gate_t)
    # every partial sum is a multiple of 2^-9 below 2^21 in magnitude, so fp32 holds g exactly
    np.testing.assert_array_equal(g.astype(np.float32).astype(np.float64), g)
    np.testing.assert_array_equal(np.round(g * 512), g * 512)
    c = make_inputs("c5", N=4000, D=256, F=512, grid=True)
    gc = orc.gate_preact(c.x, c.w_gate_t)
    assert 0.008 < (gc > c.t[:, None]).mean() < 0.012   # thresholds still give ~1% density


def test_store_ulp_and_rounding_ambiguity():
    assert orc.store_ulp(1.0, "bf16") == 2.0 ** -7 and orc.store_ulp(1.5, "bf16") == 2.0 ** -7
    assert orc.store_ulp(2.0, "bf16") == 2.0 ** -6 and orc.store_ulp(0.75, "bf16") == 2.0 ** -8
    assert orc.store_ulp(1.0, "f32") == 2.0 ** -23 and orc.store_ulp(0.0, "bf16") == 0.0
    mid = 1.0 + 2.0 ** -8                        # half way between two bf16 neighbours
    assert orc.rounding_ambiguous(np.array([mid]), 1e-9)[0]
    assert not orc.rounding_ambiguous(np.array([1.0 + 2.0 ** -7]), 1e-9)[0]
    assert not orc.rounding_ambiguous(np.array([mid + 1e-6]), 1e-9)[0]
    assert orc.rounding_ambiguous(np.array([mid + 1e-6]), 2e-6)[0]
    assert not orc.rounding_ambiguous(np.array([0.0]), 1.0)[0]


# ----------------------------------------------------------------- FP8 E4M3 gate operands

def test_e4m3_decode_known_codes():
    """Values fixed by the format (sign, 4 exponent bits with bias 7, 3
    mantissa bits, subnormals m * 2^-9, S.1111.111 = NaN)."""
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x70: 128.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    codes = np.array(list(known), dtype=np.uint8)
    np.testing.assert_array_equal(orc.e4m3_decode(codes), np.array(list(known.values())))
    assert np.isnan(orc.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(orc.e4m3_decode(np.array([0x80], np.uint8)))[0]


def test_e4m3_encode_matches_torch_cast():
    """Independent implementation: torch's float8_e4m3fn cast (round to
    nearest even) on values spanning the subnormal and normal ranges."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(300000) * np.exp2(rng.integers(-14, 9, 300000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.e4m3_encode(x), ref)


def test_e4m3_round_trip_ties_and_saturation():
    codes = np.arange(256, dtype=np.uint8)
    v = orc.e4m3_decode(codes)
    ok = ~np.isnan(v)
    np.testing.assert_array_equal(orc.e4m3_encode(v[ok]), codes[ok])
    # ties go to the even code: 1 + 1/16 between 0x38 and 0x39, 1 + 3/16 between 0x39 and 0x3A,
    # half the smallest subnormal between 0 and 0x01, 1.5 x it between 0x01 and 0x02
    ties = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -1.0625])
    np.testing.assert_array_equal(orc.e4m3_encode(ties), np.array([0x38, 0x3A, 0x00, 0x02, 0xB8], np.uint8))
    # beyond the largest value: saturate
    np.testing.assert_array_equal(orc.e4m3_encode(np.array([460.0, 1e6, -1e6])), np.array([0x7E, 0x7E, 0xFE], np.uint8))
    assert orc.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_quantize_rows_e4m3():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal((37, 300)) * np.exp2(rng.integers(-6, 6, (37, 1)))).astype(np.float32)
    a[5] = 0.0
    q, s = orc.quantize_rows_e4m3(a)
    assert q.dtype == np.uint8 and s.dtype == np.float32
    assert s[5] == 1.0 and (q[5] == 0).all()
    deq = orc.e4m3_decode(q) * s[:, None].astype(np.float64)
    # each magnitude keeps 4 significant bits: error <= half a quantum = 2^-4 relative (plus the subnormal floor)
    err = np.abs(deq - a)
    assert (err <= 2.0 ** -4 * np.abs(a) + 2.0 ** -10 * s[:, None]).all()
    # the largest magnitude of each row maps to (about) 448
    big = np.abs(orc.e4m3_decode(q)).max(axis=1)
    assert np.all((big[np.arange(37) != 5] >= 416) & (big[np.arange(37) != 5] <= 448))


def test_gate_preact_fp8_closed_form():
    """With operands that are already E4M3 values and unit scales the FP8 gate
    is the plain product of the dequantised operands; scales factor out."""
    rng = np.random.default_rng(5)
    xq = rng.integers(0, 0x7F, (9, 64)).astype(np.uint8)
    wq = rng.integers(0, 0x7F, (13, 64)).astype(np.uint8)
    xq[xq == 0x7F] = 0
    wq[wq == 0x7F] = 0
    one_x, one_w = np.ones(9, np.float32), np.ones(13, np.float32)
    g = orc.gate_preact_fp8(xq, one_x, wq, one_w)
    ref = orc.e4m3_decode(xq) @ orc.e4m3_decode(wq).T
    np.testing.assert_array_equal(g, ref)
    sx = np.float32(2.0) ** rng.integers(-3, 3, 9).astype(np.float32)
    sw = np.float32(2.0) ** rng.integers(-3, 3, 13).astype(np.float32)
    np.testing.assert_allclose(orc.gate_preact_fp8(xq, sx, wq, sw), ref * np.outer(sx, sw), rtol=0, atol=0)


# ---------------------------------------------------------------- FP8: hand-worked fixture

def _fp8_fixture():
    with open(os.path.join(GOLD, "fp8_handworked.json")) as fh:
        return json.load(fh)


def _f32_from_bits(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


def _fp8_gate_operands(fx):
    from fractions import Fraction
    g = fx["gate"]
    D = g["d_model"]

    def codes(rows):
        out = np.zeros((len(rows), D), dtype=np.uint8)
        for r, nz in enumerate(rows):
            for k, c in nz.items():
                out[r, int(k)] = int(c, 16)
        return out

    xq, wq = codes(g["x_codes_nonzero"]), codes(g["w_codes_nonzero"])
    sx = np.array([float(Fraction(v)) for v in g["x_scale"]], dtype=np.float32)
    sw = np.array([float(Fraction(v)) for v in g["w_scale"]], dtype=np.float32)
    expect = np.array([[float(Fraction(v)) for v in row] for row in g["expect_g"]])
    return xq, sx, wq, sw, expect


def _check_quantize_fixture(quantize, fx):
    q = fx["quantize"]
    for bits, scale_bits, codes in zip(q["rows_f32_bits"], q["expect_scale_f32_bits"], q["expect_codes"]):
        row = _f32_from_bits(bits)[None, :]
        got_q, got_s = quantize(row)
        assert got_s.dtype == np.float32
        if got_s.view(np.uint32)[0] != int(scale_bits, 16):
            return False
        if not np.array_equal(got_q[0], np.array([int(c, 16) for c in codes], dtype=np.uint8)):
            return False
    return True


def test_quantize_rows_e4m3_handworked():
    """Rows quantised by hand (tests/golden/fp8_handworked.json): a
    non-power-of-two scale, ties to the even code in the normal and the
    subnormal range, a scale rounded up in fp32, a deep-subnormal maximum whose
    quotient saturates, and a maximum whose quotient underflows (scale 1)."""
    assert _check_quantize_fixture(orc.quantize_rows_e4m3, _fp8_fixture())


def test_gate_preact_fp8_handworked():
    """FP8 gate on hand-decoded codes (subnormal, negative, 0x7E) with
    non-power-of-two scales; g written out exactly by hand."""
    xq, sx, wq, sw, expect = _fp8_gate_operands(_fp8_fixture())
    np.testing.assert_array_equal(orc.gate_preact_fp8(xq, sx, wq, sw), expect)


def test_fp8_fixture_catches_planted_mistakes():
    """The fixture is sharp enough to fail plausible mistakes planted in copies
    of the oracle functions (on the CPU): the scale computed as
    max * fl32(1/448), the scale rule without the underflow case, the row and
    column scales swapped, a dropped subnormal decode and a lost sign."""
    fx = _fp8_fixture()

    def q_recip(a):
        a32 = np.asarray(a, dtype=np.float32)
        amax = np.max(np.abs(a32), axis=1)
        s = (amax * (np.float32(1.0) / np.float32(448.0))).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        return orc.e4m3_encode((a32 / s[:, None]).astype(np.float32)), s

    def q_no_underflow_rule(a):
        a32 = np.asarray(a, dtype=np.float32)
        amax = np.max(np.abs(a32), axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
            return orc.e4m3_encode((a32 / s[:, None]).astype(np.float32)), s

    assert not _check_quantize_fixture(q_recip, fx)
    assert not _check_quantize_fixture(q_no_underflow_rule, fx)

    xq, sx, wq, sw, expect = _fp8_gate_operands(fx)
    dec = orc.e4m3_decode
    swapped = np.outer(sw[:3], sx[:3]).astype(np.float64) * (dec(xq) @ dec(wq).T)
    assert not np.array_equal(swapped, expect)

    def dec_no_sub(q):
        v = dec(q)
        return np.where((np.asarray(q) & 0x78) == 0, 0.0, v)

    assert not np.array_equal(np.outer(sx, sw) * (dec_no_sub(xq) @ dec_no_sub(wq).T), expect)

    def dec_abs(q):
        return np.abs(dec(q))

    assert not np.array_equal(np.outer(sx, sw) * (dec_abs(xq) @ dec_abs(wq).T), expect)
