"""Host-side bookkeeping of bench.py: the algorithmic work of a step against
the dense FFN of the same shape, and the committed per-step HBM summaries."""
import os

import pytest

import bench
from synth.inputs import CONFIGS


class _W:
    def __init__(self, name):
        c = CONFIGS[name]
        self.N, self.D, self.F, self.slots = c["N"], c["D"], c["F"], c["slots"]
        self.n_tiles = -(-self.F // c["tile_n"])


def test_forward_step_work_counts_gate_overflow_rows_and_active_units():
    w = _W("c2")
    st = {"nnz": 1000, "nnz_ell": 1000, "n_ovf": 3}
    r = bench.step_work(w, st, False, ["gate_mfma_bf16", "ffn_up_kernel", "ffn_down_kernel", "ovf_flags"])
    N, D, F = w.N, w.D, w.F
    # gate over every unit, the 3 overflow rows' gate rows again, 2 D FLOP per active unit in up and in down
    assert r["flops"] == 2.0 * N * D * F + 2.0 * 3 * D * F + 4.0 * D * 1000
    assert r["dense_flops"] == 6.0 * N * D * F
    # kernels without a work model (ovf_flags) add nothing; the three main kernels add theirs
    parts = sum(bench.kernel_work(k, w, st, False)["bytes"]
                for k in ("gate_mfma_bf16", "ffn_up_kernel", "ffn_down_kernel"))
    assert r["bytes"] == parts
    # dense: x, three weights, the hidden state written and read once, y (all bf16)
    assert r["dense_bytes"] == 2 * (N * D + 3 * F * D + 2 * N * F + N * D)


def test_training_step_work_is_three_dense_passes():
    w = _W("c5")
    st = {"nnz": 500, "nnz_ell": 400, "n_ovf": 0, "n_dense": 2}
    r = bench.step_work(w, st, True, ["gate_mfma_bf16", "ffn_up_kernel", "ffn_down_kernel", "bwd_dz_ell", "bwd_dx",
                                      "bwd_dx_gate", "bwd_dw_down", "bwd_dw"])
    N, D, F = w.N, w.D, w.F
    assert r["dense_flops"] == 18.0 * N * D * F
    # forward 4 D per active unit plus the gate, backward 12 D per active ELL / all entries
    assert r["flops"] == 2.0 * N * D * F + 4.0 * D * 500 + 2.0 * D * 400 + 10.0 * D * 500


@pytest.mark.parametrize("wl", ["c2", "c3_1", "c5"])
def test_committed_step_traffic_summaries_parse(wl):
    path = os.path.join(bench.ROOT, "profiles", f"step_traffic_{wl}.txt")
    assert os.path.exists(path)
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert kv["workload"] == wl
    assert float(kv["sparse_hbm_bytes_per_step"]) > 0 and float(kv["dense_hbm_bytes_per_step"]) > 0
    # bench reports them only while every kernel source is unchanged since the counters were taken
    m = bench.measured_step_traffic(wl)
    if kv["source_sha256_16"] == bench.all_sources_hash():
        assert m == {"sparse": float(kv["sparse_hbm_bytes_per_step"]),
                     "dense": float(kv["dense_hbm_bytes_per_step"])}
    else:
        assert m is None


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def _traffic_files():
    d = os.path.join(bench.ROOT, "profiles")
    return sorted(f for f in os.listdir(d) if f.endswith("_traffic.txt") and not f.startswith("step_traffic_"))


@pytest.mark.parametrize("fname", _traffic_files())
def test_committed_kernel_traffic_summaries_parse(fname):
    kv = {}
    for line in open(os.path.join(bench.ROOT, "profiles", fname)):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    kernel, workload = kv["kernel"], kv["workload"]
    assert fname == f"{kernel}_{workload}_traffic.txt"
    assert kernel in bench.KERNEL_SOURCES
    b = float(kv["hbm_bytes_per_launch"])
    f, w = float(kv["fetch_kib_per_dispatch"]), float(kv["write_kib_per_dispatch"])
    assert abs(b - (f * float(kv["fetch_scale"]) + w * float(kv["write_scale"])) * 1024) <= 1e-6 * b + 1024
    m = bench.measured_traffic(kernel, workload)
    assert m == (b if kv["source_sha256_16"] == bench.kernel_source_hash(kernel) else None)
