"""twell_ffn_forward_noalloc (the library's static scratch as the forward's
workspaces, for callers that cannot allocate) against twell_ffn_forward with
caller workspaces, through the C ABI: bit for bit on every output, on two calls
in a row whose second input is smaller, for a layer with overflow rows and for
small batches (the split-GEMV gate, its g in the scratch as well); shapes too
large for the scratch are refused before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from activation_sparse_ffn_03_amd import twell as tw
from synth import make_inputs

from gpu_util import dev, require_gpu, u16

pytestmark = pytest.mark.gpu


def _outputs_equal(dims, pa, pb, ya, yb, sa=None, sb=None):
    N = dims.n_tokens
    assert torch.equal(pa.counts, pb.counts)
    S = dims.slots
    cnt = u16(pa.counts)
    valid = np.arange(S)[None, :, None] < np.minimum(cnt, S)[:, None, :]
    assert np.array_equal(u16(pa.cols)[valid], u16(pb.cols)[valid])
    va = pa.vals.view(torch.int16).cpu().numpy()[valid]
    vb = pb.vals.view(torch.int16).cpu().numpy()[valid]
    assert np.array_equal(va, vb)
    assert torch.equal(pa.ovf_flag, pb.ovf_flag)
    n = int(pa.n_ovf.item())
    assert n == int(pb.n_ovf.item())
    assert int(pa.status.item()) == int(pb.status.item())
    k = min(n, dims.ovf_cap)
    assert torch.equal(pa.ovf_rows[:k], pb.ovf_rows[:k])
    assert torch.equal(pa.ovf_h[:k].view(torch.int16), pb.ovf_h[:k].view(torch.int16))
    assert torch.equal(ya[:N].view(torch.int32), yb[:N].view(torch.int32))
    if sa is not None:
        assert torch.equal(sa.view(torch.int32), sb.view(torch.int32))
    return n


def _run_pair(cfg, N, D, F, T, S, cap, seed, train=False):
    w = make_inputs(cfg, seed=seed, N=N, D=D, F=F, tile_n=T, slots=S)
    dims = tw.make_dims(N, D, F, T, S, 0, cap, 0)
    z = tw.query_sizes(dims, tw.BF16)
    x, wg, wu, wd = (dev(a, "bf16") for a in (w.x, w.w_gate_t, w.w_up_t, w.w_down))
    t = torch.from_numpy(w.t).cuda()
    # reference: the forward with caller workspaces
    pa = tw.alloc_pack(dims, tw.BF16)
    ya = torch.empty((N, D), dtype=torch.float32, device="cuda")
    sa = torch.empty(z["a_save"] // 4, dtype=torch.float32, device="cuda") if train else None
    ws = tw.alloc_workspace(z["ws_fwd"])
    gws = tw.alloc_workspace(z["ws_gate"]) if z["ws_gate"] else None
    tw.ffn_forward(dims, tw.BF16, x, wg, t, pa, wu, wd, ya, a_save=sa, ws=ws, gate_ws=gws)
    # the same on the static scratch
    pb = tw.alloc_pack(dims, tw.BF16)
    yb = torch.full((N, D), float("nan"), dtype=torch.float32, device="cuda")
    sb = torch.full((z["a_save"] // 4,), float("nan"), dtype=torch.float32, device="cuda") if train else None
    tw.ffn_forward_noalloc(dims, tw.BF16, x, wg, t, pb, wu, wd, yb, a_save=sb)
    torch.cuda.synchronize()
    if train:  # a_save is written at the slots of the packed entries of non-overflow rows only
        cnt = np.minimum(u16(pa.counts), S)
        valid = np.arange(S)[None, :, None] < cnt[:, None, :]
        valid &= ~pa.ovf_flag.cpu().numpy().astype(bool)[None, None, :]
        sa_v = sa.view(-1, S, N).cpu().numpy()[valid]
        sb_v = sb.view(-1, S, N).cpu().numpy()[valid]
        assert np.array_equal(sa_v.view(np.int32), sb_v.view(np.int32))
    return _outputs_equal(dims, pa, pb, ya, yb)


@pytest.mark.parametrize("seq", [
    # (cfg, N, D, F, T_n, S, ovf_cap): a layer with overflow rows (the dense-row
    # chunks, their partials in the scratch), then a smaller one
    [("c4", 600, 1024, 3000, 128, 4, 600), ("c4", 130, 1024, 3000, 128, 4, 130)],
    # d_model above 2048: the overflow gate rows' GEMM and several up passes
    [("c4", 384, 4096, 5120, 128, 8, 384), ("c4", 97, 4096, 5120, 128, 8, 97)],
    # small batches: split-GEMV gate with g in the scratch after the forward workspace
    [("c2", 64, 2048, 5632, 128, 128, 64), ("c2", 5, 2048, 5632, 128, 128, 64)],
    [("c3", 33, 4096, 11008, 128, 16, 33), ("c3", 1, 4096, 11008, 128, 16, 8)],
])
def test_noalloc_matches_forward_with_workspaces(seq):
    require_gpu()
    n_ovf = []
    for k, (cfg, N, D, F, T, S, cap) in enumerate(seq):
        print(f"[noalloc] call {k}: {cfg} N={N} D={D} F={F} T={T} S={S} cap={cap}", flush=True)
        n_ovf.append(_run_pair(cfg, N, D, F, T, S, cap, seed=21 + k, train=(k == 0)))
    if seq[0][5] < 16:
        assert n_ovf[0] > 0  # the overflow branch really ran


def test_noalloc_refuses_shapes_beyond_the_scratch():
    require_gpu()
    dims = tw.make_dims(16384, 4096, 11008, 128, 16, 0, 2048, 0)
    z = tw.query_sizes(dims, tw.BF16)
    assert z["ws_fwd"] > tw.NOALLOC_SCRATCH_BYTES
    pk = tw.alloc_pack(tw.make_dims(16384, 4096, 11008, 128, 16, 0, 8, 0), tw.BF16)
    dims8 = tw.make_dims(16384, 4096, 11008, 128, 16, 0, 8, 0)
    # even with a small overflow capacity the forward workspace of 16384 tokens is above 128 MiB
    assert tw.query_sizes(dims8, tw.BF16)["ws_fwd"] > tw.NOALLOC_SCRATCH_BYTES
    y = torch.full((16384, 4096), 7.0, dtype=torch.float32, device="cuda")
    x = torch.zeros((16384, 4096), dtype=torch.bfloat16, device="cuda")
    wgt = torch.zeros((11008, 4096), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(16384, dtype=torch.float32, device="cuda")
    with pytest.raises(tw.TwellError) as e:
        tw.ffn_forward_noalloc(dims8, tw.BF16, x, wgt, t, pk, wgt, wgt, y)
    assert e.value.status == 3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing was enqueued
