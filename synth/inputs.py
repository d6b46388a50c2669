"""Synthetic workloads for the ReLU-gated FFN with TwELL-packed activations.

The pages (all three) describe an L1-trained ReLU-gated FFN whose gate output
is 95-99% zeros. Trained weights are not available here, so activation
sparsity is imposed by a per-token threshold t_i on the gate pre-activation:
with W ~ N(0, 1/D) and x_i fixed, g_ij = x_i . W_gate[j] is exactly normal
with standard deviation sigma_i = ||x_i||_2 / sqrt(D), so
t_i = sigma_i * Phi^-1(1 - p_i) makes each gate unit active with probability
p_i. The threshold is an input of the method, never derived from the GPU.

Recipe (every config): numpy default_rng(seed) (PCG64) draws, in this fixed
order, x, W_gate^T, W_up^T, W_down, then p_i (lognormal configs only), then dy
(training config only). Normals are drawn in float32, scaled by
1/sqrt(fan_in) (fan_in = D for W_gate^T and W_up^T, F for W_down; x and dy are
N(0, 1)), and rounded to the storage dtype (bf16 with round-to-nearest-even, or
left in fp32). All weights are stored [F][D] row-major.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import scipy.special

# Five synthetic workloads: a tiny fp32 case, a 1B-class, a 7B-class (density
# swept), a skewed-density and a training-step FFN.
CONFIGS = {
    "c1": dict(N=64, D=128, F=512, tile_n=64, slots=16, row_cap=0, dtype="f32",
               density=("uniform", 0.05), train=False, lam=0.0),
    "c2": dict(N=4096, D=2048, F=5632, tile_n=128, slots=16, row_cap=0, dtype="bf16",
               density=("uniform", 0.01), train=False, lam=0.0),
    "c3": dict(N=16384, D=4096, F=11008, tile_n=128, slots=16, row_cap=0, dtype="bf16",
               density=("uniform", 0.01), train=False, lam=0.0),
    "c4": dict(N=8192, D=4096, F=14336, tile_n=128, slots=16, row_cap=0, dtype="bf16",
               density=("lognormal", 0.01, 1.0, 0.001, 0.30), train=False, lam=0.0),
    "c5": dict(N=8192, D=2048, F=8192, tile_n=128, slots=16, row_cap=512, dtype="bf16",
               density=("lognormal", 0.01, 1.0, 0.001, 0.20), train=True, lam=1e-4),
}


def _round_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage dtype; returns float32 holding exact values."""
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    import torch  # torch's float32 -> bfloat16 cast rounds to nearest even
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


@dataclasses.dataclass
class Workload:
    name: str
    N: int
    D: int
    F: int
    tile_n: int
    slots: int
    row_cap: int
    dtype: str           # "bf16" or "f32": storage dtype of x, weights, dy
    train: bool
    lam: float
    density: tuple
    x: np.ndarray        # [N, D] float32 (values exact in the storage dtype)
    w_gate_t: np.ndarray  # [F, D]
    w_up_t: np.ndarray   # [F, D]
    w_down: np.ndarray   # [F, D]
    p: np.ndarray        # [N] float64 target density per token
    t: np.ndarray        # [N] float32 threshold per token
    dy: Optional[np.ndarray]  # [N, D] or None

    @property
    def n_tiles(self) -> int:
        return -(-self.F // self.tile_n)


def _densities(rng, N: int, spec: tuple) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":
        return np.full(N, float(spec[1]), dtype=np.float64)
    if kind == "lognormal":
        mean, s, lo, hi = (float(v) for v in spec[1:5])
        # median chosen so the unclipped lognormal has the stated mean
        mu = math.log(mean) - 0.5 * s * s
        z = rng.standard_normal(N)
        return np.clip(np.exp(mu + s * z), lo, hi)
    raise ValueError(f"unknown density spec {spec!r}")


def _grid(rng, shape, half: int, scale: float) -> np.ndarray:
    """Integers uniform in [-half, half] times a power-of-two scale (exact in bf16)."""
    return (rng.integers(-half, half + 1, size=shape).astype(np.float32) * np.float32(scale))


def make_inputs(name: str, seed: int = 0, *, density=None, N=None, D=None, F=None,
                tile_n=None, slots=None, row_cap=None, grid: bool = False) -> Workload:
    """Draw one workload. Keyword overrides shrink a config for quick tests.

    grid=True draws x as multiples of 1/8 in [-2, 2] and the weights as
    multiples of 1/64 in [-1/8, 1/8] instead of normals: every product is then a
    multiple of 2^-9 and every dot product over d_model <= 8192 stays below
    2^21 * 2^-9, so it is exact in fp32 whatever the summation order. Used to
    make rounding decisions on the gate pre-activation identical on every
    implementation."""
    cfg = dict(CONFIGS[name])
    for k, v in dict(N=N, D=D, F=F, tile_n=tile_n, slots=slots, row_cap=row_cap).items():
        if v is not None:
            cfg[k] = v
    if density is not None:
        cfg["density"] = density if isinstance(density, tuple) else ("uniform", float(density))
    n, d, f = int(cfg["N"]), int(cfg["D"]), int(cfg["F"])
    dt = cfg["dtype"]
    rng = np.random.default_rng(seed)
    if grid:
        x = _grid(rng, (n, d), 16, 1.0 / 8)
        wg = _grid(rng, (f, d), 8, 1.0 / 64)
        wu = _grid(rng, (f, d), 8, 1.0 / 64)
        wd = _grid(rng, (f, d), 8, 1.0 / 64)
        w_std = math.sqrt(sum(k * k for k in range(-8, 9)) / 17.0) / 64.0
    else:
        x = _round_storage(rng.standard_normal((n, d), dtype=np.float32), dt)
        wg = _round_storage(rng.standard_normal((f, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d)), dt)
        wu = _round_storage(rng.standard_normal((f, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d)), dt)
        wd = _round_storage(rng.standard_normal((f, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(f)), dt)
        w_std = 1.0 / math.sqrt(d)
    p = _densities(rng, n, cfg["density"])
    # std of g_ij given x_i when the gate weights have standard deviation w_std
    sigma = np.sqrt(np.einsum("ij,ij->i", x.astype(np.float64), x.astype(np.float64))) * w_std
    t = (sigma * scipy.special.ndtri(1.0 - p)).astype(np.float32)
    dy = None
    if cfg["train"]:
        dy = _grid(rng, (n, d), 16, 1.0 / 8) if grid else _round_storage(rng.standard_normal((n, d), dtype=np.float32), dt)
    return Workload(name=name, N=n, D=d, F=f, tile_n=int(cfg["tile_n"]), slots=int(cfg["slots"]),
                    row_cap=int(cfg["row_cap"]), dtype=dt, train=bool(cfg["train"]),
                    lam=float(cfg["lam"]), density=tuple(cfg["density"]),
                    x=x, w_gate_t=wg, w_up_t=wu, w_down=wd, p=p, t=t, dy=dy)


def config_summary(name: str) -> dict:
    c = CONFIGS[name]
    return {"workload": name, "n_tokens": c["N"], "d_model": c["D"], "d_ff": c["F"],
            "tile_n": c["tile_n"], "slots": c["slots"], "row_cap": c["row_cap"],
            "dtype": c["dtype"], "density": list(c["density"]), "train": c["train"],
            "l1_lambda": c["lam"]}
