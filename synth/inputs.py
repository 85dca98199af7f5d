"""Seeded synthetic FFN-layer inputs shaped like the pages' 0.5B-2B models.

The pages measure trained models on fineweb; neither the weights nor the data
exist here, so these inputs stand in for them. They reproduce the shapes and the
activation statistics the pages report: roughly 29 of 8192 gate units active
per token at the recommended L1 setting (pulsen.vercel.app article, paragraph
on the sparsification recipe: 911 -> 29 non-zeros per layer), about 30% of gate
columns permanently dead (same article, dead-neuron paragraph), tokens whose
active counts range from a handful to hundreds (Tencent Cloud article, section
3, hybrid format), and denser first positions of a sequence (same article,
section 5).

Recipe (all draws from numpy's PCG64, streams spawned from one SeedSequence in
the fixed order x, Wg, Wu, Wd, token-scale, tail, dead-set, zipf-permutation):

* x ~ N(0, 1) with column 0 fixed to 1 so that Wg[:, 0] acts as a gate bias;
  per-token scale a_r multiplies x[r, 1:] (a_r = 1 for uniform workloads).
* Wg[j, 1:], WuT ~ N(0, 1/d); Wd ~ N(0, 1/F); all rounded fp32 -> bf16 (RNE).
* Wg[j, 0] = -theta_j * s_j with s_j = ||Wg[j, 1:]|| (of the bf16 values), so
  a gate pre-activation is -theta_j s_j + a_r N(0, s_j^2) and unit j is active
  with probability Phi_bar(theta_j / a_r).
* Dead columns get a threshold 10 sigma above the largest token scale; always-on
  (saturated) columns get the mirror image.

The module only draws random numbers and picks thresholds from normal
quantiles; it never forms a product of x with a weight matrix.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np
from scipy import special

# Stream order of SeedSequence(seed).spawn(8).
_X, _WG, _WU, _WD, _SCALE, _TAIL, _DEAD, _PERM = range(8)


@dataclass(frozen=True)
class Workload:
    """One synthetic FFN layer: shapes, TwELL tile/capacity and density structure."""

    name: str
    M: int  # tokens
    d: int  # model width
    F: int  # FFN hidden width
    T: int  # TwELL tile width (columns of the gate output per tile)
    C: int  # TwELL slots per (row, tile)
    structure: str  # "uniform" | "heavy_tail" | "zipf"
    mean_nnz: float  # target mean active gate units per token
    seed: int
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def density(self) -> float:
        return self.mean_nnz / self.F

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "M": self.M,
            "d": self.d,
            "F": self.F,
            "T": self.T,
            "C": self.C,
            "structure": self.structure,
            "mean_nnz_target": round(self.mean_nnz, 4),
            "density_target": round(self.density, 6),
            "seed": self.seed,
        }


def _uniform(name, M, d, F, T, C, p, seed):
    return Workload(name, M, d, F, T, C, "uniform", p * F, seed)


SWEEP_DENSITIES = (0.001, 0.0035, 0.01, 0.03, 0.11)


def sweep_workloads() -> list[Workload]:
    """Density sweep at M=8192, d=2048, F=8192 (0.1% ... 11% = dense-ReLU level)."""
    return [
        _uniform(f"sweep_p{100 * p:g}pct", 8192, 2048, 8192, 128, 16, p, 1040 + i)
        for i, p in enumerate(SWEEP_DENSITIES)
    ]


WORKLOADS: dict[str, Workload] = {
    # Tiny layer that the oracle finishes in well under a second.
    "tiny": _uniform("tiny", 64, 256, 1024, 64, 8, 0.05, 1000),
    # 1.5B-like layer at the recommended sparsity: 29 active of 8192 per token.
    "ffn1p5b": _uniform("ffn1p5b", 4096, 2048, 8192, 128, 16, 29 / 8192, 1001),
    # Same shape, heavy-tailed per-token counts, 30% dead columns.
    "ffn1p5b_heavytail": Workload(
        "ffn1p5b_heavytail", 4096, 2048, 8192, 128, 16, "heavy_tail", 29.0, 1002,
        extra={"dead_frac": 0.30, "tail_frac": 0.02, "tail_lo": 501, "tail_hi": 2000,
               "seq_len": 1024, "dense_positions": 8, "dense_factor": 10.0, "sigma": 1.0},
    ),
    # 2B-like layer: lognormal per-token counts, Zipf(1.1) column rates.
    "ffn2b_zipf": Workload(
        "ffn2b_zipf", 16384, 2560, 10240, 128, 16, "zipf", 20.0, 1003,
        extra={"zipf_s": 1.1, "sigma": 1.0},
    ),
}
for _w in sweep_workloads():
    WORKLOADS[_w.name] = _w

DECODE_BATCHES = (1, 16, 64, 256)


def decode_workloads() -> list[Workload]:
    """The 1.5B-like layer at small batches (decode / batched decode)."""
    return [
        _uniform(f"decode_m{m}", m, 2048, 8192, 128, 16, 29 / 8192, 1050 + i)
        for i, m in enumerate(DECODE_BATCHES)
    ]


for _w in decode_workloads():
    WORKLOADS[_w.name] = _w


def scaled(w: Workload, **changes) -> Workload:
    """Same density structure at other sizes (for oracle-sized parity cases).

    The active fraction is kept: mean_nnz scales with F unless given.
    """
    name = changes.pop("name", None)
    if "F" in changes and "mean_nnz" not in changes:
        changes["mean_nnz"] = w.mean_nnz * changes["F"] / w.F
    out = dataclasses.replace(w, **changes)
    if name is None:
        name = f"{w.name}[M={out.M},d={out.d},F={out.F},T={out.T},C={out.C}]"
    return dataclasses.replace(out, name=name)


@dataclass
class Inputs:
    """bf16 bit patterns (uint16), row-major. All weights are [F, d], row j = unit j."""

    workload: Workload
    x: np.ndarray  # [M, d]
    Wg: np.ndarray  # [F, d]  gate_proj.weight
    WuT: np.ndarray  # [F, d] up_proj.weight
    Wd: np.ndarray  # [F, d]  down_proj.weight transposed
    info: dict


# --------------------------------------------------------------------------- bf16
def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, as raw bits (finite inputs only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------- helpers
def _phi_bar(t):
    """Upper normal tail P(N(0,1) > t)."""
    return special.ndtr(-np.asarray(t, dtype=np.float64))


def _upper_quantile(p):
    """t with P(N(0,1) > t) = p."""
    return -special.ndtri(np.asarray(p, dtype=np.float64))


def _lognormal_counts(rng, n, mean, sigma):
    mu = np.log(mean) - 0.5 * sigma * sigma
    return rng.lognormal(mu, sigma, size=n)


def _zipf_rates(F, total, s, perm):
    """q_j = min(1, c * rank_j^-s) with sum_j q_j = total; rank from a permutation."""
    rank = np.empty(F, dtype=np.float64)
    rank[perm] = np.arange(1, F + 1, dtype=np.float64)
    lo, hi = 1e-6, float(F)
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * rank ** -s).sum() > total:
            hi = c
        else:
            lo = c
    c = 0.5 * (lo + hi)
    return np.minimum(1.0, c * rank ** -s), c


def _monotone_inverse(grid, values, targets):
    """Invert a (numerically) increasing tabulated function by interpolation."""
    v = np.maximum.accumulate(values)
    return np.interp(targets, v, grid)


def _fit_zipf(theta0, saturated, n_target, iters=4):
    """Alternate per-token scales a_r and per-column quantiles theta_j so that
    token counts match n_target and column rates match the Zipf rates."""
    live = ~saturated
    q_live = _phi_bar(theta0[live])
    theta = theta0.copy()
    a_grid = np.geomspace(0.05, 40.0, 1200)
    t_grid = np.linspace(-6.0, 9.0, 3000)
    a = np.ones_like(n_target)
    n_sat = float(saturated.sum())
    for _ in range(iters):
        # token counts as a function of the token scale
        f = n_sat + _phi_bar(theta[live][None, :] / a_grid[:, None]).sum(axis=1)
        n_clip = np.clip(n_target, f.min(), f.max())
        a = _monotone_inverse(a_grid, f, n_clip)
        # column rates as a function of the column quantile, over the token mix
        a_q = np.quantile(a, np.linspace(0.0005, 0.9995, 512))
        g = _phi_bar(t_grid[:, None] / a_q[None, :]).mean(axis=1)  # decreasing in t
        theta_live = _monotone_inverse(-t_grid[::-1], g[::-1], q_live)
        theta[live] = -theta_live
    return theta, a


# ----------------------------------------------------------------------- main
def make_inputs(w: Workload, seed: int | None = None) -> Inputs:
    seed = w.seed if seed is None else seed
    rngs = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(8)]
    M, d, F = w.M, w.d, w.F
    info: dict = {"seed": seed}

    # Weights first: thresholds depend on the bf16 gate rows.
    wg32 = rngs[_WG].standard_normal((F, d), dtype=np.float32)
    wg32 *= np.float32(1.0 / np.sqrt(d))
    Wg = _to_bf16_bits(wg32)
    del wg32
    s = np.sqrt(np.square(_bf16_bits_to_f32(Wg[:, 1:]).astype(np.float64)).sum(axis=1))

    theta = np.zeros(F)
    a = np.ones(M)
    dead = np.zeros(F, dtype=bool)
    saturated = np.zeros(F, dtype=bool)
    n_target = np.full(M, w.mean_nnz)

    if w.structure == "uniform":
        theta[:] = _upper_quantile(w.mean_nnz / F)
    elif w.structure == "heavy_tail":
        e = w.extra
        n_dead = int(round(e["dead_frac"] * F))
        dead[rngs[_DEAD].permutation(F)[:n_dead]] = True
        L = F - n_dead
        theta[~dead] = _upper_quantile(w.mean_nnz / L)
        n_target = _lognormal_counts(rngs[_SCALE], M, w.mean_nnz, e["sigma"])
        tail = rngs[_TAIL].random(M) < e["tail_frac"]
        n_target[tail] = rngs[_TAIL].integers(e["tail_lo"], e["tail_hi"] + 1, size=int(tail.sum()))
        early = (np.arange(M) % e["seq_len"]) < e["dense_positions"]
        n_target[early] *= e["dense_factor"]
        # P(active) = Phi_bar(theta / a) < 1/2 for every a, so cap below L/2.
        n_target = np.clip(n_target, 0.05, 0.45 * L)
        a = theta[~dead][0] / _upper_quantile(n_target / L)
        info.update(dead_columns=int(n_dead), tail_tokens=int(tail.sum()),
                    early_tokens=int(early.sum()))
    elif w.structure == "zipf":
        e = w.extra
        q, c = _zipf_rates(F, w.mean_nnz, e["zipf_s"], rngs[_PERM].permutation(F))
        saturated = q >= 1.0
        theta0 = np.where(saturated, -np.inf, _upper_quantile(np.clip(q, 1e-12, 1 - 1e-12)))
        n_target = _lognormal_counts(rngs[_SCALE], M, w.mean_nnz, e["sigma"])
        theta, a = _fit_zipf(theta0, saturated, n_target)
        info.update(zipf_c=float(c), saturated_columns=int(saturated.sum()),
                    column_rate=q)
    else:
        raise ValueError(f"unknown structure {w.structure!r}")

    big = 10.0 * float(a.max())
    bias = np.where(dead, -big, np.where(saturated, big, -theta)) * s
    Wg[:, 0] = _to_bf16_bits(bias.astype(np.float32))

    x32 = rngs[_X].standard_normal((M, d), dtype=np.float32)
    if w.structure != "uniform":
        x32[:, 1:] *= a.astype(np.float32)[:, None]
    x32[:, 0] = 1.0
    x = _to_bf16_bits(x32)
    del x32

    wu32 = rngs[_WU].standard_normal((F, d), dtype=np.float32)
    wu32 *= np.float32(1.0 / np.sqrt(d))
    WuT = _to_bf16_bits(wu32)
    del wu32
    wd32 = rngs[_WD].standard_normal((F, d), dtype=np.float32)
    wd32 *= np.float32(1.0 / np.sqrt(F))
    Wd = _to_bf16_bits(wd32)
    del wd32

    # n_target is the model-side expected active count of each token; the
    # realised counts come from the data and are measured by the consumers.
    info.update(token_scale=a, n_target=n_target, dead=dead, saturated=saturated, theta=theta)
    return Inputs(w, x, Wg, WuT, Wd, info)


# --------------------------------------------------------- training side
_DY = 8  # a ninth stream of the same SeedSequence: the first eight are unchanged


def make_upstream_grad(w: Workload, seed: int | None = None) -> np.ndarray:
    """Upstream gradient dy for the backward: bf16 bits [M, d], N(0, 1/d)
    (the scale of a loss gradient spread over d outputs), RNE-rounded."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(_DY + 1)[_DY])
    dy = rng.standard_normal((w.M, w.d), dtype=np.float32) * np.float32(1.0 / np.sqrt(w.d))
    return _to_bf16_bits(dy)
