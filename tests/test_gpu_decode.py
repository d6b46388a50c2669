"""Small batches (the decode regime, 1 <= N <= TWELL_SMALL_BATCH_MAX = 64):
the split-GEMV gate of twell_gate_pack_ws, the whole forward at 1-64 tokens,
and the forward replayed from a HIP graph."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from activation_sparse_ffn_03_amd import twell as tw
from oracle import twell_oracle as orc
from synth import make_inputs

from gpu_util import DELTA_REL, Pipeline, check_pack, dev, f64, h_flip, require_gpu, rowwise_ok

pytestmark = pytest.mark.gpu

Y_TOL = 1e-2


def _gate(w, dims, ws=None, g_dump=None):
    pack = tw.alloc_pack(dims, tw.BF16)
    tw.gate_pack(dims, tw.BF16, dev(w.x, "bf16"), dev(w.w_gate_t, "bf16"),
                 torch.from_numpy(w.t.astype(np.float32)).cuda(), pack, g_dump=g_dump, ws=ws)
    torch.cuda.synchronize()
    return pack


@pytest.mark.parametrize("N", [1, 5, 16, 17, 48, 64])
def test_small_batch_gate_and_pack(N):
    """g within the fp32 accumulation bound; pack and overflow rows bit-exact
    against the oracle's pack of the GPU's own g; the run without g_dump
    (g through the workspace) bit-identical to the run with it."""
    require_gpu()
    D, F = 2048, 1000  # F ragged against 16-unit workgroups and 128-wide tiles
    w = make_inputs("c2", seed=N, N=N, D=D, F=F, density=0.06)
    dims = tw.make_dims(N, D, F, 128, 4, 0, N, 0)
    sizes = tw.query_sizes(dims, tw.BF16)
    assert sizes["ws_gate"] == N * F * 4
    ws = tw.alloc_workspace(sizes["ws_gate"])
    gd = torch.empty((N, F), dtype=torch.float32, device="cuda")
    pack = _gate(w, dims, ws=ws, g_dump=gd)
    g64 = orc.gate_preact(w.x, w.w_gate_t)
    rms = np.sqrt(np.mean(g64 * g64, axis=1))
    assert np.all(np.abs(f64(gd) - g64) <= DELTA_REL * rms[:, None])
    g_gpu = f64(gd)
    ref = orc.pack(g_gpu, w.t, 128, 4, store="bf16", arith="f32")
    check_pack(pack, ref, N)
    n = min(ref["n_ovf"], N)
    hq = orc.dense_activation(g_gpu, w.t, store="bf16", arith="f32")
    np.testing.assert_array_equal(f64(pack.ovf_h[:n]), hq[ref["ovf_rows"][:n]])
    pack2 = _gate(w, dims, ws=ws)
    for f in ("vals", "cols", "counts", "ovf_flag", "ovf_rows", "n_ovf", "status"):
        a, b = getattr(pack, f), getattr(pack2, f)
        if f == "ovf_rows":
            a, b = a[:n], b[:n]
        if f in ("vals", "cols"):  # slots past the count are don't-care
            S = dims.slots
            cnt = np.minimum(ref["counts"], S)
            valid = torch.from_numpy(np.arange(S)[None, :, None] < cnt[:, None, :]).cuda()
            a, b = a[valid], b[valid]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f


@pytest.mark.parametrize("N", [1, 64])
def test_small_batch_exact_gate_matches_large_batch_path(N):
    """On grid inputs every dot product is exact in fp32, so the split GEMV
    and the large-batch GEMM give the same g, and both packs equal the oracle's."""
    require_gpu()
    D, F = 1024, 640
    w = make_inputs("c2", seed=7, N=N, D=D, F=F, grid=True)
    dims = tw.make_dims(N, D, F, 128, 4, 0, N, 0)
    ws = tw.alloc_workspace(tw.query_sizes(dims, tw.BF16)["ws_gate"])
    p_small = _gate(w, dims, ws=ws)
    p_large = _gate(w, dims)
    g64 = orc.gate_preact(w.x, w.w_gate_t)
    ref = orc.pack(g64, w.t, 128, 4, store="bf16", arith="f32")
    check_pack(p_small, ref, N)
    check_pack(p_large, ref, N)


@pytest.mark.parametrize("name,N,kw", [
    ("c2", 1, {}), ("c2", 16, {}), ("c2", 64, {}),          # 1B-class layer, full size
    ("c3", 1, {}), ("c3", 33, {}),                           # 7B-class layer, full size
    ("c4", 64, dict(slots=8)),                               # lognormal density: overflow rows
])
def test_small_batch_forward(name, N, kw):
    require_gpu()
    w = make_inputs(name, seed=N, N=N)
    pl = Pipeline(w, ovf_cap=N, **kw)
    assert pl.ffn.ws_gate is not None
    y = f64(pl.forward())
    assert int(pl.ffn.pack.status.item()) == 0
    ref = orc.ffn_forward(w.x, w.w_gate_t, w.w_up_t, w.w_down, w.t, store=w.dtype, arith="f32")
    slack = (h_flip(ref, w.dtype) * np.abs(ref["a"])) @ np.abs(w.w_down.astype(np.float64))
    rowwise_ok(y, ref["y"], Y_TOL, "y", slack)


def test_small_batch_workspace_too_small():
    require_gpu()
    N, D, F = 8, 256, 512
    w = make_inputs("c2", seed=1, N=N, D=D, F=F)
    dims = tw.make_dims(N, D, F, 128, 4, 0, N, 0)
    pack = tw.alloc_pack(dims, tw.BF16)
    pack.counts.fill_(0x1234)
    ws = tw.alloc_workspace(N * F * 4 - 256)
    with pytest.raises(tw.TwellError) as ei:
        tw.gate_pack(dims, tw.BF16, dev(w.x, "bf16"), dev(w.w_gate_t, "bf16"),
                     torch.from_numpy(w.t).cuda(), pack, ws=ws)
    assert ei.value.status == 3  # TWELL_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((pack.counts == 0x1234).all())  # nothing was enqueued


@pytest.mark.parametrize("name,N", [("c2", 1), ("c2", 64), ("c4", 48)])
def test_forward_graph_replay(name, N):
    """The forward recorded into a HIP graph and replayed on new inputs: every
    replay equals the eager forward on the same inputs, bit for bit, with eager
    work and host synchronisations between replays."""
    require_gpu()
    w = make_inputs(name, seed=11, N=N)
    dims = tw.make_dims(N, w.D, w.F, w.tile_n, w.slots, 0, N, 0)
    ffn = tw.TwellFFN(dims, tw.BF16)
    x = dev(w.x, "bf16")
    wg, wu, wd = dev(w.w_gate_t, "bf16"), dev(w.w_up_t, "bf16"), dev(w.w_down, "bf16")
    t = torch.from_numpy(w.t).cuda()
    graph = ffn.capture(x, wg, wu, wd, t)
    eager = tw.TwellFFN(dims, tw.BF16)
    rng = np.random.default_rng(5)
    for rep in range(4):
        xn = orc.round_bf16(rng.standard_normal((N, w.D))).astype(np.float32)
        x.copy_(dev(xn, "bf16"))
        graph.replay()
        torch.cuda.synchronize()
        y_graph = ffn.y.clone()
        y_eager = eager.forward(x, wg, wu, wd, t).clone()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int32), y_eager.view(torch.int32)), rep
        assert torch.equal(ffn.pack.counts, eager.pack.counts), rep


def test_capture_refused_where_not_cleared():
    """capture() raises on the bf16 forward with d_model > 2048 and possible
    overflow rows (the path with the unexplained abort at process exit), and
    allows the small-batch and no-overflow forms of the same layer."""
    require_gpu()
    w = make_inputs("c4", seed=11, N=128, D=4096, F=1024)
    dims = tw.make_dims(128, 4096, 1024, 128, 16, 0, 32, 0)
    ffn = tw.TwellFFN(dims, tw.BF16)
    assert not ffn.capture_supported()
    x, wg, wu, wd = (dev(a, "bf16") for a in (w.x, w.w_gate_t, w.w_up_t, w.w_down))
    with pytest.raises(tw.TwellError):
        ffn.capture(x, wg, wu, wd, torch.from_numpy(w.t).cuda())
    assert tw.TwellFFN(tw.make_dims(128, 4096, 1024, 128, 128, 0, 32, 0), tw.BF16).capture_supported()
    assert tw.TwellFFN(tw.make_dims(48, 4096, 1024, 128, 16, 0, 48, 0), tw.BF16).capture_supported()
    assert tw.TwellFFN(tw.make_dims(128, 2048, 1024, 128, 16, 0, 32, 0), tw.BF16).capture_supported()


@pytest.mark.skip(reason="graph capture of the bf16 forward with d_model > 2048 and overflow rows is disabled: one "
                         "process that captured and replayed it (8192 x 4096 x 14336, skewed density) aborted at exit "
                         "in glibc (free(): invalid pointer) with no GPU fault; cause not found, so the case stays "
                         "off the GPU")
def test_forward_graph_replay_skewed_density_full_size():
    """The 8192 x 4096 x 14336 skewed-density forward (overflow rows present)
    recorded into a HIP graph and replayed: each replay equals the eager
    forward bit for bit, and the process exits cleanly."""
    require_gpu()
    w = make_inputs("c4")
    dims = tw.make_dims(w.N, w.D, w.F, w.tile_n, w.slots, 0, max(64, w.N // 8), 0)
    ffn = tw.TwellFFN(dims, tw.BF16)
    x, wg, wu, wd = (dev(a, "bf16") for a in (w.x, w.w_gate_t, w.w_up_t, w.w_down))
    t = torch.from_numpy(w.t).cuda()
    graph = ffn.capture(x, wg, wu, wd, t)
    eager = tw.TwellFFN(dims, tw.BF16)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        y_graph = ffn.y.clone()
        y_eager = eager.forward(x, wg, wu, wd, t).clone()
        torch.cuda.synchronize()
        assert int(eager.pack.n_ovf.item()) > 0
        assert torch.equal(y_graph.view(torch.int32), y_eager.view(torch.int32)), rep
