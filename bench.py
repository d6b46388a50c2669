#!/usr/bin/env python3
"""Benchmark of the libtwell hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input.
The default workload is the 7B-class forward (16384 tokens, d_model 4096, d_ff
11008, uniform gate density 1%), the largest single-GPU configuration: gate
GEMM with the TwELL pack epilogue, overflow rows, and the fused up/down
projection. The other workloads are picked with --workload: the 1B-class
forward, the 7B-class forward at 5% and 0.5%, the skewed-density forward, the
training step (forward saving a, hybrid routing and the sparse backward), and
the 1B / 7B forwards with the gate projection on FP8 E4M3 operands (x
quantised per step, W_gate once).

Prints ONE JSON line: throughput in tokens/s, the dense bf16 FFN on the same
GPU and inputs as reference, the roofline of the dominant kernel (device time
from HIP events recorded around each kernel on its own stream through the
library's trace ABI), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFS = 5000.0   # MI355X dense fp8 MFMA, published
VALU_FP32_PEAK_TFS = 157.3   # MI355X fp32 vector, published
METRIC = "sparse FFN tokens/s and speedup vs dense bf16 FFN; HBM GB/s / MFMA % of peak"

WORKLOADS = {
    # name: (config, density override, train, FP8 gate, overrides of the config)
    "c5": ("c5", None, True, False, {}),
    "c2": ("c2", None, False, False, {}),
    "c3_5": ("c3", 0.05, False, False, {}),
    "c3_1": ("c3", 0.01, False, False, {}),
    "c3_05": ("c3", 0.005, False, False, {}),
    "c4": ("c4", None, False, False, {}),
    "c2_fp8": ("c2", None, False, True, {}),
    "c3_1_fp8": ("c3", 0.01, False, True, {}),
    # decode / small batch: the same layers on 1-64 tokens. The TwELL arrays
    # are then tiny, so each tile gets as many slots as it has columns
    # (S = T_n): no row can overflow and the overflow steps are skipped.
    "c2_dec1": ("c2", None, False, False, dict(N=1, slots=128)),
    "c2_dec16": ("c2", None, False, False, dict(N=16, slots=128)),
    "c2_dec64": ("c2", None, False, False, dict(N=64, slots=128)),
    "c3_dec1": ("c3", 0.01, False, False, dict(N=1, slots=128)),
    "c3_dec64": ("c3", 0.01, False, False, dict(N=64, slots=128)),
    "c2_dec1_fp8": ("c2", None, False, True, dict(N=1, slots=128)),
    "c3_dec1_fp8": ("c3", 0.01, False, True, dict(N=1, slots=128)),
    "c3_dec64_fp8": ("c3", 0.01, False, True, dict(N=64, slots=128)),
}


def workload_inputs(name):
    """(inputs, train, fp8) of a named workload."""
    from synth import make_inputs
    cfg, dens, train, fp8, over = WORKLOADS[name]
    return make_inputs(cfg, density=dens, **over), train, fp8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="c3_1", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="skip the graph-replay timings")
    p.add_argument("--cpu-sample", type=int, default=512, help="tokens per window of the CPU oracle sample")
    p.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of CPU oracle work")
    p.add_argument("--copy-calib", action="store_true", help="only run the copy kernel used to scale HBM counters")
    p.add_argument("--traffic-pass", choices=("sparse", "dense"),
                   help="only run warmup + steps of one path, untimed (for the HBM counter runs)")
    return p.parse_args()


def capacities(w, train):
    """Overflow / dense-backup capacities the benchmark launches with (rows)."""
    return max(64, w.N // 8), (max(64, w.N // 8) if train else 0)


def describe(w, train, fp8=False):
    dens = w.density
    d = f"uniform {dens[1] * 100:g}%" if dens[0] == "uniform" else \
        f"lognormal mean {dens[1] * 100:g}% sigma {dens[2]:g} clip [{dens[3] * 100:g}%, {dens[4] * 100:g}%]"
    kind = "training step (fwd + route + bwd)" if train else ("forward, FP8 E4M3 gate" if fp8 else "forward")
    return f"{kind}: {w.N} tokens x d_model {w.D} x d_ff {w.F}, T_n {w.tile_n}, S {w.slots}, density {d}"


def kernel_work(name, w, st, train):
    """Algorithmic bytes and flops of one launch of a main kernel (what the method must move / compute)."""
    N, D, F, e = w.N, w.D, w.F, 2
    nnz, nnz_ell, n_t = st["nnz"], st["nnz_ell"], w.n_tiles
    if name == "gate_mfma_bf16":
        twell = n_t * w.slots * N * (e + 2) + n_t * N * 2
        return {"flops": 2.0 * N * D * F, "bytes": N * D * e + F * D * e + twell, "bound": "mfma", "peak": "bf16"}
    if name == "gate_mfma_fp8":   # one-byte operands and their row scales; TwELL written in bf16
        twell = n_t * w.slots * N * (e + 2) + n_t * N * 2
        return {"flops": 2.0 * N * D * F, "bytes": N * D + F * D + 4 * (N + F) + twell, "bound": "mfma",
                "peak": "fp8"}
    if name == "quantize_e4m3":   # x read (bf16), codes and scales written
        return {"flops": 0.0, "bytes": N * D * e + N * D + 4 * N, "bound": "hbm"}
    if name == "gate_gemv_small":  # small batches: W_gate streamed once, x read, g (fp32) written
        return {"flops": 2.0 * N * D * F, "bytes": F * D * e + N * D * e + N * F * 4, "bound": "hbm"}
    if name == "pack_from_g":      # g read, TwELL written
        twell = n_t * w.slots * N * (e + 2) + n_t * N * 2
        return {"flops": 0.0, "bytes": N * F * 4 + twell, "bound": "hbm"}
    if name in ("ffn_up_kernel", "ffn_up_blocked"):  # x, W_up once; TwELL read; z (and a when training) written
        byt = N * D * e + F * D * e + nnz * (e + 2) + n_t * N * 2 + nnz * 4 + (nnz * 4 if train else 0)
        return {"flops": 2.0 * D * nnz, "bytes": byt, "bound": "hbm", "gathered": nnz * D * e}
    if name == "ffn_down_kernel":  # W_down once; cols + z read; y written (fp32)
        byt = F * D * e + nnz * (2 + 4) + n_t * N * 2 + N * D * 4
        return {"flops": 2.0 * D * nnz, "bytes": byt, "bound": "hbm", "gathered": nnz * D * e}
    if name in ("bwd_dz_ell", "bwd_dz_blocked"):   # dy, W_down once; row-ELL read; (col, z, da, dg) records written
        byt = N * D * e + F * D * e + nnz_ell * (e + 8) + nnz_ell * 20
        return {"flops": 2.0 * D * nnz_ell, "bytes": byt, "bound": "hbm", "gathered": nnz_ell * D * e}
    if name == "bwd_dx":       # W_up once; records read; dx written (fp32)
        byt = F * D * e + nnz * 8 + N * D * 4
        return {"flops": 2.0 * D * nnz, "bytes": byt, "bound": "hbm", "gathered": nnz * D * e}
    if name == "bwd_dx_gate":  # W_gate once; records read; dx read and written (fp32)
        byt = F * D * e + nnz * 8 + 2 * N * D * 4
        return {"flops": 2.0 * D * nnz, "bytes": byt, "bound": "hbm", "gathered": nnz * D * e}
    if name == "bwd_dw_down":  # dy once; records via the column transpose; dW_down written (fp32)
        byt = N * D * e + nnz * 12 + F * D * 4
        return {"flops": 2.0 * D * nnz, "bytes": byt, "bound": "hbm", "gathered": nnz * D * e}
    if name == "bwd_dw":       # x once; records via the column transpose; dW_up, dW_gate written (fp32)
        byt = N * D * e + nnz * 16 + 2 * F * D * 4
        return {"flops": 4.0 * D * nnz, "bytes": byt, "bound": "hbm", "gathered": nnz * D * e}
    return None


def step_work(w, st, train, kernel_names):
    """Algorithmic FLOPs and bytes of one step, for libtwell and for the dense
    bf16 FFN of the same shape. libtwell: the sum of kernel_work over the
    step's main kernels, plus the gate rows of the overflow rows, which are
    recomputed (2 D F FLOP each). Dense: 6 N D F FLOP (18 N D F for a training
    step); bytes are x, the three weights and the [N x F] hidden state written
    and read once in bf16, plus y in bf16 (for a training step also dy, the
    weights and the hidden state again, dx and the three weight gradients in
    fp32)."""
    N, D, F, e = w.N, w.D, w.F, 2
    fl = 2.0 * st["n_ovf"] * D * F
    by = 0.0
    for k in kernel_names:
        wk = kernel_work(k, w, st, train)
        if wk:
            fl += wk["flops"]
            by += wk["bytes"]
    dfl = 6.0 * N * D * F
    dby = N * D * e + 3 * F * D * e + 2 * N * F * e + N * D * e
    if train:
        dfl = 18.0 * N * D * F
        dby += N * D * e + 3 * F * D * e + 2 * N * F * e + N * D * 4 + 3 * F * D * 4
    return {"flops": fl, "bytes": by, "dense_flops": dfl, "dense_bytes": dby}


def measured_step_traffic(workload):
    """HBM bytes per step of libtwell and of the dense baseline from the
    committed counter summary (every kernel of one step, FETCH_SIZE +
    WRITE_SIZE scaled by the copy-kernel calibration), or None if there is
    none or a kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"step_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#") and not line.startswith("|"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != all_sources_hash():
        return None
    return {"sparse": float(kv["sparse_hbm_bytes_per_step"]), "dense": float(kv["dense_hbm_bytes_per_step"])}


def all_sources_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "activation_sparse_ffn_03_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(w, train, sample, budget_s=10.0, fp8=False):
    """The oracle, as it stands, on successive windows of `sample` tokens of the
    same workload (full d_model / d_ff), repeated until about `budget_s` seconds
    of CPU work have been done; returns the oracle's tokens/s."""
    import numpy as np
    from oracle import twell_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    n = max(1, min(sample, w.N))
    if fp8:
        wq, wsc = orc.quantize_rows_e4m3(w.w_gate_t)   # once, as on the GPU
    done, windows = 0, 0
    t0 = time.perf_counter()
    while True:
        lo = (windows * n) % w.N
        rows = np.arange(lo, min(lo + n, w.N))
        x, t = w.x[rows], w.t[rows]
        if fp8:
            xq, xsc = orc.quantize_rows_e4m3(x)
            g = orc.gate_preact_fp8(xq, xsc, wq, wsc)
            pk = orc.pack(g, t, w.tile_n, w.slots, store=w.dtype, arith="f32")
            hq = orc.dense_activation(g, t, store=w.dtype, arith="f32")
            orc.sparse_forward(pk, x, w.w_up_t, w.w_down, ovf_h=hq[pk["ovf_rows"]])
        else:
            fw = orc.ffn_forward(x, w.w_gate_t, w.w_up_t, w.w_down, t, store=w.dtype)
            pk = orc.pack(fw["g"], t, w.tile_n, w.slots, store=w.dtype, arith="f32")
        if train:
            orc.route(pk, w.row_cap, a=fw["a"], ovf_h=fw["hq"][pk["ovf_rows"]])
            orc.ffn_backward(x, w.dy[rows], w.w_gate_t, w.w_up_t, w.w_down, fw["mask"], fw["hq"], w.lam)
        done += rows.size
        windows += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": blas_threads or cores, "kind": "oracle",
            "sample": f"{windows} windows of {n} tokens ({done} tokens) of the same workload, full d_model/d_ff, "
                      f"fp64 NumPy, {'forward + pack + route + backward' if train else 'forward + pack'}"
                      f"{' with FP8 quantisation of x and the FP8 gate' if fp8 else ''}; "
                      f"{dt:.1f} s wall; BLAS threads {blas_threads}, host affinity {cores} cores"}


# Source files whose code makes up each timed kernel: the committed counter
# summary of a kernel is only used while these files are unchanged.
KERNEL_SOURCES = {
    "gate_mfma_bf16": ["gate_pack.hip", "twell_device.h"],
    "gate_mfma_fp8": ["gate_pack.hip", "twell_device.h"],
    "gate_gemv_small": ["gate_pack.hip", "twell_device.h"],
    "pack_from_g": ["gate_pack.hip", "twell_device.h"],
    "quantize_e4m3": ["quant.hip", "twell_device.h"],
    "ffn_up_kernel": ["fused_fwd.hip", "row_ops.h", "twell_device.h"],
    "ffn_up_blocked": ["up_blocked.hip", "blocked_sddmm.h", "row_ops.h", "twell_device.h"],
    "ffn_down_kernel": ["fused_fwd.hip", "block_order.h", "row_ops.h", "twell_device.h"],
    "bwd_dz_ell": ["bwd.hip", "row_ops.h", "twell_device.h"],
    "bwd_dz_blocked": ["bwd_blocked.hip", "blocked_sddmm.h", "twell_device.h"],
    "bwd_dx": ["bwd.hip", "row_ops.h", "twell_device.h"],
    "bwd_dx_gate": ["bwd.hip", "row_ops.h", "twell_device.h"],
    "bwd_dw_down": ["bwd.hip", "row_ops.h", "twell_device.h"],
    "bwd_dw": ["bwd.hip", "row_ops.h", "twell_device.h"],
}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "activation_sparse_ffn_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration),
    or None if there is none or the kernel's source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return float(kv["hbm_bytes_per_launch"])


def copy_calibration():
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters: 1 GiB read and 1 GiB written per launch."""
    import torch
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(multi-GPU sharding is design-only).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from activation_sparse_ffn_03_amd import twell as tw

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calib:
        copy_calibration()
        return
    tw.lib()
    w, train, fp8 = workload_inputs(args.workload)
    print(f"[bench] workload {args.workload}: {describe(w, train, fp8)}", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16)

    x, wg, wu, wd = up(w.x), up(w.w_gate_t), up(w.w_up_t), up(w.w_down)
    t = torch.from_numpy(w.t).to(dev)
    dy = up(w.dy) if train else None
    ovf_cap, dense_cap = capacities(w, train)
    dims = tw.make_dims(w.N, w.D, w.F, w.tile_n, w.slots, w.row_cap if train else 0, ovf_cap, dense_cap)
    ffn = tw.TwellFFN(dims, tw.BF16, train=train, fp8_gate=fp8)
    wgate = tw.quantize_e4m3(wg) if fp8 else wg   # the weight's codes and scales: once, outside the step

    def step():
        ffn.forward(x, wgate, wu, wd, t)
        if train:
            ffn.backward(x, dy, wg, wu, wd, w.lam)

    lam = w.lam

    # dense bf16 FFN on the same GPU and inputs (torch / hipBLASLt), same step definition
    def dense_step():
        g = torch.nn.functional.linear(x, wg)
        a = torch.nn.functional.linear(x, wu)
        m = g > t[:, None]
        h = torch.where(m, g - t[:, None].to(g.dtype), torch.zeros((), dtype=g.dtype, device=dev))
        z = h * a
        y = torch.mm(z, wd)
        if train:
            dz = torch.nn.functional.linear(dy, wd)
            dwd = torch.mm(z.t(), dy)
            da = dz * h
            dg = torch.where(m, dz * a + lam, torch.zeros((), dtype=g.dtype, device=dev))
            dx = torch.mm(da, wu) + torch.mm(dg, wg)
            dwu = torch.mm(da.t(), x)
            dwg = torch.mm(dg.t(), x)
            return y, dx, dwd, dwu, dwg
        return y

    # the dense baseline's matrix products alone (hipBLASLt through torch),
    # without its elementwise work: the bar a fused dense kernel would face
    h_dense = torch.randn((w.N, w.F), device=dev, dtype=torch.bfloat16) if not args.no_dense else None

    def dense_gemms():
        torch.nn.functional.linear(x, wg)
        torch.nn.functional.linear(x, wu)
        torch.mm(h_dense, wd)
        if train:
            torch.nn.functional.linear(dy, wd)
            torch.mm(h_dense.t(), dy)
            torch.mm(h_dense, wu)
            torch.mm(h_dense, wg)
            torch.mm(h_dense.t(), x)
            torch.mm(h_dense.t(), x)

    if args.traffic_pass:
        # counter runs: warmup + steps of one path only, nothing timed
        fn = step if args.traffic_pass == "sparse" else dense_step
        for _ in range(args.warmup + args.steps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"traffic_pass": args.traffic_pass, "workload": args.workload,
                          "steps_run": args.warmup + args.steps}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps
    assert int(ffn.pack.status.item()) == 0, "overflow capacity exceeded"
    if train:
        assert int(ffn.hyb.status.item()) == 0, "dense-backup capacity exceeded"

    # the forward replayed from a HIP graph (the serving-loop form: no host
    # launch cost per kernel); same inputs, same K steps
    graph_ms = None
    # graph replays are timed for the forwards whose capture is supported
    # (TwellFFN.capture_supported); the others are timed eagerly only
    replay = not train and not args.no_graph and ffn.capture_supported()
    if replay:
        graph = ffn.capture(x, wgate, wu, wd, t)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph

    # per-kernel device times: HIP events around every kernel on the stream it runs on
    tw.trace_start(capacity=64 * args.steps + 64)
    for _ in range(args.steps):
        step()
    recs = tw.trace_stop()
    per = {}
    for name, kms in recs:
        per.setdefault(name, []).append(kms)
    kernels = {k: {"launches_per_step": len(v) / args.steps, "avg_ms": sum(v) / len(v),
                   "ms_per_step": sum(v) / args.steps} for k, v in per.items()}

    cnt = ffn.pack.counts.to(torch.int32) & 0xFFFF   # uint16 counts stored in int16
    nnz = int(cnt.to(torch.int64).sum().item())
    stats = {"nnz": nnz, "nnz_ell": nnz, "n_ovf": int(ffn.pack.n_ovf.item())}
    if train:
        isd = ffn.hyb.is_dense.bool()
        rn = ffn.hyb.row_nnz.to(torch.int64)
        stats["nnz_ell"] = int(rn[~isd].sum().item())
        stats["n_dense"] = int(ffn.hyb.n_dense.item())

    main_k = [k for k in kernels if kernel_work(k, w, stats, train)]
    dom = max(main_k, key=lambda k: kernels[k]["ms_per_step"])
    wk = kernel_work(dom, w, stats, train)
    sec = kernels[dom]["avg_ms"] / 1e3
    if wk["bound"] == "mfma":
        ach = wk["flops"] / sec / 1e12
        peak = MFMA_FP8_PEAK_TFS if wk["peak"] == "fp8" else MFMA_BF16_PEAK_TFS
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "traffic": measured_traffic(dom, args.workload), "kernel": dom}
    else:
        ach = wk["bytes"] / sec / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(dom, args.workload), "kernel": dom}
    for k in main_k:
        wk_k = kernel_work(k, w, stats, train)
        s_k = kernels[k]["avg_ms"] / 1e3
        kernels[k]["GBps_algorithmic"] = wk_k["bytes"] / s_k / 1e9
        kernels[k]["TFLOPs"] = wk_k["flops"] / s_k / 1e12
        # the kernel's floor at spec peaks: MFMA (its dtype), or the larger of
        # HBM (algorithmic bytes at 8 TB/s) and VALU (flops at 157.3 TFLOP/s);
        # frac_of_floor = floor / measured time
        if wk_k["bound"] == "mfma":
            peak = MFMA_FP8_PEAK_TFS if wk_k.get("peak") == "fp8" else MFMA_BF16_PEAK_TFS
            floor_s = wk_k["flops"] / (peak * 1e12)
        else:
            floor_s = max(wk_k["bytes"] / (HBM_PEAK_GBS * 1e9), wk_k["flops"] / (VALU_FP32_PEAK_TFS * 1e12))
        kernels[k]["floor_ms"] = floor_s * 1e3
        kernels[k]["frac_of_floor"] = floor_s / s_k
        if "gathered" in wk_k:   # weight (or token) rows delivered per active entry, mostly from L2
            kernels[k]["gather_TBps"] = wk_k["gathered"] / s_k / 1e12

    dense = dense_graph_ms = None
    if not args.no_dense:
        for _ in range(args.warmup):
            dense_step()
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.steps):
            dense_step()
        d1.record(stream)
        torch.cuda.synchronize()
        dense = d0.elapsed_time(d1) / args.steps
        if replay:   # the dense forward replayed from a graph as well
            dgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(dgraph):
                dense_step()
            for _ in range(args.warmup):
                dgraph.replay()
            torch.cuda.synchronize()
            d0.record(stream)
            for _ in range(args.steps):
                dgraph.replay()
            d1.record(stream)
            torch.cuda.synchronize()
            dense_graph_ms = d0.elapsed_time(d1) / args.steps
            del dgraph

    dense_gemm_ms = None
    if not args.no_dense:
        for _ in range(args.warmup):
            dense_gemms()
        torch.cuda.synchronize()
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        for _ in range(args.steps):
            dense_gemms()
        m1.record(stream)
        torch.cuda.synchronize()
        dense_gemm_ms = m0.elapsed_time(m1) / args.steps

    # per-step times (each step bracketed by its own events): warm caches, and
    # cold ones (a 512 MB write between steps evicts the 4 MB L2s and the 256 MB
    # Infinity Cache), median and minimum over `steps` steps each
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def per_step(fn, cold):
        times = []
        for _ in range(args.steps):
            if cold:
                flush_buf.fill_(1)
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            fn()
            a1.record(stream)
            torch.cuda.synchronize()
            times.append(a0.elapsed_time(a1))
        times.sort()
        return {"median": times[len(times) // 2], "min": times[0]}

    step_ms = {"warm": per_step(step, False), "cold": per_step(step, True)}
    dense_step_ms = None
    if dense is not None:
        dense_step_ms = {"warm": per_step(dense_step, False), "cold": per_step(dense_step, True)}
    del flush_buf

    flops_dense = 6.0 * w.N * w.D * w.F * (3 if train else 1)
    # work and HBM bytes of one step against the dense FFN of the same shape
    sw = step_work(w, stats, train, list(kernels))
    meas = measured_step_traffic(args.workload)
    vs_dense = {
        "flops": {"twell": sw["flops"], "dense": sw["dense_flops"], "saved_frac": 1 - sw["flops"] / sw["dense_flops"]},
        "bytes_algorithmic": {"twell": sw["bytes"], "dense": sw["dense_bytes"],
                              "saved_frac": 1 - sw["bytes"] / sw["dense_bytes"]},
        "hbm_bytes_measured": None if meas is None else
        {"twell": meas["sparse"], "dense": meas["dense"], "saved_frac": 1 - meas["sparse"] / meas["dense"],
         "twell_GBps": meas["sparse"] / (ms / 1e3) / 1e9,
         "dense_GBps": (meas["dense"] / (dense / 1e3) / 1e9) if dense else None},
    }
    out = {
        "metric": METRIC,
        "value": w.N / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 gate, bf16" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {describe(w, train, fp8)}", "n_tokens": w.N, "d_model": w.D,
                   "d_ff": w.F, "tile_n": w.tile_n, "slots": w.slots, "row_cap": w.row_cap if train else 0,
                   "parallelism": "none (1 GPU)"},
        "graph_ms_per_step": graph_ms,
        "dense_graph_ms_per_step": dense_graph_ms,
        "speedup_vs_dense": (dense / ms) if dense else None,
        "dense_gemm_only_ms_per_step": dense_gemm_ms,
        "speedup_vs_dense_gemm_only": (dense_gemm_ms / ms) if dense_gemm_ms else None,
        "dense_bf16_ms_per_step": dense,
        "step_ms": step_ms,
        "dense_step_ms": dense_step_ms,
        "dense_equivalent_tflops": flops_dense / (ms / 1e3) / 1e12,
        "roofline": roof,
        "vs_dense": vs_dense,
        "kernels": kernels,
        "workload_stats": {**stats, "density": nnz / (w.N * w.F)},
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, train, args.cpu_sample, args.cpu_budget, fp8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
