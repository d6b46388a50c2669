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
