"""Seeded synthetic workloads for the owner-side Muon step.

This module only draws inputs: shapes, seeds, value distributions and the
hyperparameters each workload runs with.  It holds none of the step's
arithmetic, so both the GPU path and the CPU oracle can be fed from it.

The pages evaluate on production models (Qwen2.5-7B, VLA models, models up to
32B; DMuon summary §4, MatrixFSDP summary "Resultados").  Only the weight
shapes matter for the cost of the optimizer step, so seeded Gaussian
gradients at the shapes of a 4096-hidden / 11008-MLP decoder layer stand in
for them.

Recipe (per workload): ``numpy.random.Generator(PCG64(seed))``; for each
matrix in list order draw G, then M0, then (timing runs only) W0, each as
float32 standard normals times the workload's standard deviation, then cast
to the storage dtype with round-to-nearest-even.  A packed AdamW tail, when
present, draws p then g from its own stream ``PCG64([seed, 1])``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

BF16 = "bf16"
F32 = "f32"
TORCH_DTYPE = {BF16: torch.bfloat16, F32: torch.float32}

#: Coefficients published with Muon (Jordan et al., 2024); not on the pages.
QUINTIC = (3.4445, -4.7750, 2.0315)


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int
    cols: int
    dtype: str = BF16


@dataclass(frozen=True)
class AdamWConfig:
    numel: int
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    step: int = 1
    param_std: float = 0.02
    grad_std: float = 1e-3


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    seed: int
    matrices: tuple
    grad_std: float
    mom_std: float
    weight_std: float = 0.02
    lr: float = 0.02
    beta: float = 0.95
    coeffs: tuple = QUINTIC
    steps: int = 5
    eps: float = 1e-7
    tail: AdamWConfig | None = None
    extra: dict = field(default_factory=dict)

    @property
    def count(self) -> int:
        return len(self.matrices)


# --- shapes ------------------------------------------------------------------------------

HIDDEN, MLP = 4096, 11008


def layer_shapes(prefix: str = "") -> list[MatrixSpec]:
    """One decoder layer: Q, K, V, O square; gate and up wide; down tall."""
    return [
        MatrixSpec(prefix + "q", HIDDEN, HIDDEN),
        MatrixSpec(prefix + "k", HIDDEN, HIDDEN),
        MatrixSpec(prefix + "v", HIDDEN, HIDDEN),
        MatrixSpec(prefix + "o", HIDDEN, HIDDEN),
        MatrixSpec(prefix + "gate", HIDDEN, MLP),
        MatrixSpec(prefix + "up", HIDDEN, MLP),
        MatrixSpec(prefix + "down", MLP, HIDDEN),
    ]


def _cost(spec: MatrixSpec) -> float:
    """Flop-model cost used only to pick an owner's share (3 m^2 n + 17 m^3)."""
    m, n = min(spec.rows, spec.cols), max(spec.rows, spec.cols)
    return 3.0 * m * m * n + 17.0 * m ** 3


def owner_share(layers: int = 32, ranks: int = 8, rank: int = 0) -> list[MatrixSpec]:
    """Greedy longest-processing-time owner assignment; return one rank's matrices.

    Matrices are sorted by cost, descending and stable in layer order; each goes
    to the least-loaded rank, the lowest rank index on ties.  The returned list
    keeps layer order.
    """
    allm = []
    for layer in range(layers):
        allm.extend(layer_shapes(f"L{layer}."))
    order = sorted(range(len(allm)), key=lambda i: -_cost(allm[i]))
    load = [0.0] * ranks
    owner = [0] * len(allm)
    for i in order:
        r = min(range(ranks), key=lambda j: (load[j], j))
        owner[i] = r
        load[r] += _cost(allm[i])
    return [allm[i] for i in range(len(allm)) if owner[i] == rank]


SMALL_SHAPES = [(256, 256), (512, 2048), (768, 768), (768, 3072), (1024, 1024)]


def many_small(count: int = 512, seed: int = 5) -> list[MatrixSpec]:
    idx = np.random.Generator(np.random.PCG64([seed, 2])).integers(0, len(SMALL_SHAPES), count)
    return [MatrixSpec(f"s{i}", *SMALL_SHAPES[k]) for i, k in enumerate(idx)]


# --- the workloads -------------------------------------------------------------------------

WORKLOADS = {
    "single_f32_256x1024": Workload(
        name="single_f32_256x1024",
        description="one fp32 256x1024 matrix, G and M0 ~ N(0,1)",
        seed=1, matrices=(MatrixSpec("w", 256, 1024, F32),), grad_std=1.0, mom_std=1.0),
    "batch16_bf16_1024x4096": Workload(
        name="batch16_bf16_1024x4096",
        description="16 bf16 1024x4096 matrices, G and M0 ~ N(0, 1e-3^2)",
        seed=2, matrices=tuple(MatrixSpec(f"w{i}", 1024, 4096) for i in range(16)),
        grad_std=1e-3, mom_std=1e-3),
    "layer4096_bf16": Workload(
        name="layer4096_bf16",
        description="one 4096-hidden decoder layer: Q,K,V,O 4096x4096, gate/up 4096x11008, "
                    "down 11008x4096, bf16, G and M0 ~ N(0, 1e-3^2)",
        seed=3, matrices=tuple(layer_shapes()), grad_std=1e-3, mom_std=1e-3),
    "owner_share_32x4096_bf16": Workload(
        name="owner_share_32x4096_bf16",
        description="one owner's 28 matrices of a 32-layer 4096/11008 decoder split over 8 owners "
                    "by greedy makespan, bf16, plus a 2M-value fp32 AdamW tail",
        seed=4, matrices=tuple(owner_share()), grad_std=1e-3, mom_std=1e-3,
        tail=AdamWConfig(numel=2 * 1024 * 1024)),
    "many_small_512_bf16": Workload(
        name="many_small_512_bf16",
        description="512 bf16 matrices with shapes drawn from 256^2, 512x2048, 768^2, 768x3072, 1024^2",
        seed=5, matrices=tuple(many_small()), grad_std=1e-3, mom_std=1e-3),
}


def custom(name: str, shapes, dtype: str = BF16, seed: int = 0, grad_std: float = 1e-3,
           mom_std: float = 1e-3, **kw) -> Workload:
    """A workload of arbitrary shapes (used by tests for ragged and edge cases)."""
    mats = tuple(MatrixSpec(f"{name}{i}", int(r), int(c), dtype) for i, (r, c) in enumerate(shapes))
    return Workload(name=name, description=f"custom {name}", seed=seed, matrices=mats,
                    grad_std=grad_std, mom_std=mom_std, **kw)


# --- drawing -----------------------------------------------------------------------------

def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(TORCH_DTYPE[dtype])


def generate(wl: Workload, *, weights: str = "zeros", device=None):
    """Yield (spec, W, G, M0) per matrix, as CPU tensors or moved to ``device``.

    ``weights="zeros"`` gives W0 = 0 (parity runs: then W' = -step * O, so the
    comparison is not drowned by one rounding of a large W); ``"random"`` draws
    W0 ~ N(0, weight_std^2) after G and M0 (timing runs).
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    for spec in wl.matrices:
        shape = (spec.rows, spec.cols)
        G = _draw(rng, shape, wl.grad_std, spec.dtype)
        M = _draw(rng, shape, wl.mom_std, spec.dtype)
        if weights == "random":
            W = _draw(rng, shape, wl.weight_std, spec.dtype)
        else:
            W = torch.zeros(shape, dtype=TORCH_DTYPE[spec.dtype])
        if device is not None:
            G, M, W = G.to(device), M.to(device), W.to(device)
        yield spec, W, G, M


def generate_tail(wl: Workload, device=None):
    """Draw the AdamW tail (p, g, m=0, v=0) from its own stream, PCG64([seed, 1])."""
    if wl.tail is None:
        return None
    rng = np.random.Generator(np.random.PCG64([wl.seed, 1]))
    t = wl.tail
    p = _draw(rng, (t.numel,), t.param_std, F32)
    g = _draw(rng, (t.numel,), t.grad_std, F32)
    m = torch.zeros(t.numel, dtype=torch.float32)
    v = torch.zeros(t.numel, dtype=torch.float32)
    if device is not None:
        p, g, m, v = p.to(device), g.to(device), m.to(device), v.to(device)
    return p, g, m, v


# --- Shampoo inputs ----------------------------------------------------------------------

def _spd(rng: np.random.Generator, n: int, scale: float, cond: float, reflections: int = 8) -> np.ndarray:
    """Q diag(lam) Q^T in float64 with lam log-uniform over [scale / cond, scale] and Q the
    product of `reflections` Householder reflections I - 2 v v^T (v Gaussian, normalised).

    H S H = S - v w^T - w v^T with u = S v, w = 2 u - 2 (v^T u) v: one symmetric matrix-vector
    product and one symmetric rank-2 update per reflection, on the upper triangle (BLAS
    dsymv and dsyr2), so large statistics cost O(n^2)."""
    from scipy.linalg import blas

    lam = scale * np.exp(rng.uniform(-np.log(cond), 0.0, n))
    S = np.asfortranarray(np.diag(lam))
    for _ in range(reflections):
        v = rng.standard_normal(n)
        v /= np.linalg.norm(v)
        u = blas.dsymv(1.0, S, v, lower=0)
        w = 2.0 * u - 2.0 * float(v @ u) * v
        S = blas.dsyr2(-1.0, v, w, a=S, lower=0, overwrite_a=1)
    U = np.triu(S)
    return U + np.triu(U, 1).T


def shampoo_inputs(shapes, seed: int, *, grad_std: float = 1e-2, weight_std: float = 0.02,
                   stats: str = "warm", cond: float = 1e3):
    """Yield (W, G, L0, R0) per (rows, cols) shape as float32 CPU tensors.

    Recipe: ``numpy.random.Generator(PCG64(seed))``; per matrix in list order draw W0 and G
    as float32 normals times weight_std and grad_std, then (``stats="warm"``) the left and
    the right statistic as symmetric positive definite matrices Q diag(lam) Q^T with lam
    log-uniform over [s / cond, s], s = grad_std^2 max(rows, cols) (the size of the
    eigenvalues of one G G^T) and Q a product of 8 Householder reflections, rounded to
    float32 and made exactly symmetric; or zero
    statistics (``stats="zero"``, a first step).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    for r, c in shapes:
        W = _draw(rng, (r, c), weight_std, F32)
        G = _draw(rng, (r, c), grad_std, F32)
        if stats == "warm":
            s = grad_std ** 2 * max(r, c)
            Lm = _spd(rng, r, s, cond).astype(np.float32)
            Rm = _spd(rng, c, s, cond).astype(np.float32)
            L0 = torch.from_numpy(np.triu(Lm) + np.triu(Lm, 1).T)
            R0 = torch.from_numpy(np.triu(Rm) + np.triu(Rm, 1).T)
        elif stats == "zero":
            L0 = torch.zeros((r, r), dtype=torch.float32)
            R0 = torch.zeros((c, c), dtype=torch.float32)
        else:
            raise ValueError(f"stats must be 'warm' or 'zero', not {stats!r}")
        yield W, G, L0, R0


@dataclass(frozen=True)
class ShampooWorkload:
    """Inputs of a Shampoo step: shapes, seed and distributions (see shampoo_inputs) and the
    hyperparameters it runs with."""
    name: str
    description: str
    seed: int
    shapes: tuple
    grad_std: float = 1e-3
    weight_std: float = 0.02
    stats: str = "warm"
    cond: float = 1e3
    lr: float = 1e-3
    beta2: float = 0.9
    eps: float = 1e-6
    root_iters: int = 12

    @property
    def count(self) -> int:
        return len(self.shapes)

    def generate(self, device=None):
        for W, G, L0, R0 in shampoo_inputs(self.shapes, self.seed, grad_std=self.grad_std,
                                           weight_std=self.weight_std, stats=self.stats, cond=self.cond):
            if device is not None:
                W, G, L0, R0 = W.to(device), G.to(device), L0.to(device), R0.to(device)
            yield W, G, L0, R0


SHAMPOO_WORKLOADS = {
    "shampoo_layer4096_f32": ShampooWorkload(
        name="shampoo_layer4096_f32",
        description="one 4096-hidden decoder layer (Q,K,V,O 4096x4096, gate/up 4096x11008, down "
                    "11008x4096) in fp32, G ~ N(0, 1e-3^2), warm statistics (condition 1e3), "
                    "12 coupled Newton steps per root",
        seed=7, shapes=tuple((s.rows, s.cols) for s in layer_shapes())),
    "shampoo_attn4096_f32": ShampooWorkload(
        name="shampoo_attn4096_f32",
        description="the four 4096x4096 attention matrices of one 4096-hidden layer in fp32, "
                    "G ~ N(0, 1e-3^2), warm statistics (condition 1e3), 12 coupled Newton steps per root",
        seed=8, shapes=((4096, 4096),) * 4),
}
