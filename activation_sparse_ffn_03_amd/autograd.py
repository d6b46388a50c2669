"""PyTorch autograd wrapper of the libtwell hot path.

`TwellFFNFunction` runs the whole path through libtwell.so: the gate GEMM
with the TwELL pack, the fused up/down projection (forward), and the hybrid
routing with the sparse backward. It computes

    g = x · w_gate_tᵀ,  h = max(g - t_i, 0),  y = (h ⊙ (x · w_up_tᵀ)) · w_down

for x [N, D] and weights [F, D] ("Sakana AI and NVIDIA present TwELL", second
paragraph: the gate projection emits the sparse activation, one pass consumes
it for the up and down projections, and training goes through a hybrid
sparse / dense-backup format). Its backward returns the gradients of
sum(dy ⊙ y) + l1_lambda · sum(h), i.e. the L1 penalty on the gate activation
that makes it sparse is added by the op itself, so callers need not
materialise h. t carries one threshold per token (zeros: plain ReLU).

Every call allocates its own sparse state (TwELL pack, saved activations)
through torch's allocator, so several forward calls may precede their
backward calls. Capacities for overflow rows (a tile count above S) and
dense-backup rows (more than row_cap entries) are fractions of N; by
default a call that exceeds one raises TwellError after a host sync of the
status word (check=False skips the sync and leaves such rows uncomputed).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import twell as tw

_ERR_CAPACITY = 4  # TWELL_ERR_CAPACITY


@dataclass(frozen=True)
class TwellConfig:
    tile_n: int = 128
    slots: int = 16
    row_cap: int = 512
    ovf_frac: float = 0.125
    dense_frac: float = 0.125
    check: bool = True

    def caps(self, n: int, train: bool):
        ovf = max(8, math.ceil(n * self.ovf_frac))
        dense = max(8, math.ceil(n * self.dense_frac)) if train else 0
        return ovf, dense


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return tw.BF16
    if t.dtype == torch.float32:
        return tw.F32
    raise TypeError(f"libtwell computes on bf16 or fp32 inputs, got {t.dtype}")


class TwellFFNFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w_gate_t, w_up_t, w_down, t, l1_lambda: float, cfg: TwellConfig):
        if x.dim() != 2:
            raise ValueError("x must be [N, D]")
        N, D = x.shape
        F = w_gate_t.shape[0]
        dt = _dtype_code(x)
        for w in (w_gate_t, w_up_t, w_down):
            if w.dtype != x.dtype or tuple(w.shape) != (F, D):
                raise ValueError("weights must be [d_ff, d_model] in the dtype of x")
        x, w_gate_t, w_up_t, w_down = (v.contiguous() for v in (x, w_gate_t, w_up_t, w_down))
        t = t.to(torch.float32).contiguous()
        train = any(ctx.needs_input_grad[:4])
        ovf_cap, dense_cap = cfg.caps(N, train)
        dims = tw.make_dims(N, D, F, cfg.tile_n, cfg.slots, min(cfg.row_cap, F) if train else 0, ovf_cap, dense_cap)
        sizes = tw.query_sizes(dims, dt)
        dev = x.device
        pack = tw.alloc_pack(dims, dt, dev)
        y = torch.empty((N, D), dtype=torch.float32, device=dev)
        a_save = torch.empty(sizes["a_save"] // 4, dtype=torch.float32, device=dev) if train else None
        ws = tw.alloc_workspace(sizes["ws_fwd"], dev)
        # small batches (bf16, up to TWELL_SMALL_BATCH_MAX tokens): the split-GEMV gate
        ws_gate = tw.alloc_workspace(sizes["ws_gate"], dev) if sizes["ws_gate"] else None
        tw.gate_pack(dims, dt, x, w_gate_t, t, pack, ws=ws_gate)
        tw.ffn_fwd(dims, dt, pack, x, w_up_t, w_down, y, a_save=a_save, ws=ws)
        if cfg.check and int(pack.status.item()) != 0:
            raise tw.TwellError(_ERR_CAPACITY, "TwellFFNFunction",
                                f"{int(pack.n_ovf.item())} overflow rows exceed the capacity {ovf_cap}")
        ctx.save_for_backward(x, w_gate_t, w_up_t, w_down)
        ctx.state = (dims, dt, sizes, pack, a_save, float(l1_lambda), cfg)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_gate_t, w_up_t, w_down = ctx.saved_tensors
        dims, dt, sizes, pack, a_save, lam, cfg = ctx.state
        if a_save is None:
            return None, None, None, None, None, None, None
        dev = x.device
        N, D = x.shape
        F = w_gate_t.shape[0]
        hyb = tw.alloc_hybrid(dims, dt, dev)
        ws = tw.alloc_workspace(sizes["ws_bwd"], dev)
        dx = torch.empty((N, D), dtype=torch.float32, device=dev)
        dwg = torch.empty((F, D), dtype=torch.float32, device=dev)
        dwu = torch.empty((F, D), dtype=torch.float32, device=dev)
        dwd = torch.empty((F, D), dtype=torch.float32, device=dev)
        dy = dy.to(x.dtype).contiguous()
        tw.route_hybrid(dims, dt, pack, a_save, hyb)
        tw.ffn_bwd(dims, dt, hyb, x, dy, w_gate_t, w_up_t, w_down, lam, dx, dwg, dwu, dwd, ws)
        if cfg.check and int(hyb.status.item()) != 0:
            raise tw.TwellError(_ERR_CAPACITY, "TwellFFNFunction.backward",
                                f"{int(hyb.n_dense.item())} dense-backup rows exceed the capacity {dims.dense_cap}")
        need = ctx.needs_input_grad
        return (dx.to(x.dtype) if need[0] else None, dwg.to(w_gate_t.dtype) if need[1] else None,
                dwu.to(w_up_t.dtype) if need[2] else None, dwd.to(w_down.dtype) if need[3] else None,
                None, None, None)


def twell_ffn(x, w_gate_t, w_up_t, w_down, t=None, l1_lambda: float = 0.0, cfg: TwellConfig = TwellConfig()):
    """Functional form; t defaults to zeros (plain ReLU gate)."""
    if t is None:
        t = torch.zeros(x.shape[0], dtype=torch.float32, device=x.device)
    return TwellFFNFunction.apply(x, w_gate_t, w_up_t, w_down, t, l1_lambda, cfg)


class TwellGatedFFN(torch.nn.Module):
    """Activation-sparse gated FFN block on libtwell: parameters [d_ff, d_model]
    each, initialised N(0, 1/fan_in) (fan_in = d_model for gate and up, d_ff
    for down). forward(x, t=None) takes x [..., d_model] and returns fp32
    [..., d_model]."""

    def __init__(self, d_model: int, d_ff: int, l1_lambda: float = 0.0, cfg: TwellConfig = TwellConfig(),
                 dtype=torch.bfloat16, device="cuda"):
        super().__init__()
        self.l1_lambda, self.cfg = float(l1_lambda), cfg

        def init(fan_in):
            w = torch.randn(d_ff, d_model, device=device) / math.sqrt(fan_in)
            return torch.nn.Parameter(w.to(dtype))

        self.w_gate_t = init(d_model)
        self.w_up_t = init(d_model)
        self.w_down = init(d_ff)

    def forward(self, x, t=None):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1])
        if t is not None:
            t = t.reshape(-1)
        y = twell_ffn(x2, self.w_gate_t, self.w_up_t, self.w_down, t, self.l1_lambda, self.cfg)
        return y.reshape(*lead, y.shape[-1])
