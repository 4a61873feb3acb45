"""The largest sizes the C ABI accepts, on the GPU.

Muon: one side of 2^20 (the limit) against the full oracle.  Shampoo: a 1 x 65536 matrix (the
limit) from zero statistics.  Its right statistic R' = g^T g is 65536 x 65536 (17 GB, five
workspace slots of that size) and of rank one, so every Newton iterate is a polynomial in R':
X_R g^T = f(sigma^2 + eps) g^T and X_L = f(sigma^2 + eps), with sigma = ||g|| and f the
K-step root polynomial at nu = sigma^2 + eps.  The exact update is then W' - W = -lr f^2 g,
where f is the oracle's inverse_root_newton on diag(sigma^2 + eps, eps); this holds at any size.
These operands exceed 2 GB, so the launches take the 64-bit pointer path."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from oracle import inverse_root_newton
from tests.gpu_helpers import DEV, check_matrix, log, relf, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,dtype", [((1, 1 << 20), W.BF16), ((1 << 20, 1), W.BF16),
                                         ((3, 1 << 20), W.F32)], ids=str)
def test_muon_longest_side(shape, dtype):
    log(f"max size muon {shape} {dtype}")
    std = 1.0 if dtype == W.F32 else 1e-3
    wl = W.custom("max", [shape], dtype=dtype, seed=5, grad_std=std, mom_std=std)
    res = run_gpu(wl)
    check_matrix(res, 0, wl)


@pytest.mark.parametrize("shape,iters", [((1, 65536), 2), ((65536, 1), 1)], ids=str)
def test_shampoo_largest_statistic(shape, iters):
    r, c = shape
    n = max(r, c)
    log(f"max size shampoo {shape} iters={iters}")
    rng = np.random.default_rng(17)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    lr, eps = 0.05, 1e-6
    G = torch.from_numpy(g).reshape(r, c).to(DEV)
    Wt = torch.from_numpy(w0).reshape(r, c).to(DEV)
    Ls = torch.zeros((r, r), dtype=torch.float32, device=DEV)
    Rs = torch.zeros((c, c), dtype=torch.float32, device=DEV)
    step = nm.ShampooStep([Wt], [G], [Ls], [Rs], lr=lr, beta2=1.0, eps=eps, root_iters=iters)
    log(f"  workspace {step.ws_bytes / 2**30:.1f} GiB")
    step()
    torch.cuda.synchronize()
    big = Rs if c > r else Ls
    # the big statistic: g g^T at sampled entries
    idx = torch.from_numpy(rng.integers(0, n, size=(2, 4096))).to(DEV)
    got = big[idx[0], idx[1]].double().cpu().numpy()
    g64 = g.astype(np.float64)
    want = g64[idx[0].cpu().numpy()] * g64[idx[1].cpu().numpy()]
    assert relf(got, want) <= 1e-5  # products of two values: one rounding each
    # The 1 x 1 statistic is one fp32 sum of 65536 squares: its rounding grows like
    # sqrt(n) u = 256 x 6e-8 = 1.5e-5, so it is held to the fp32 bar of the step's outputs.
    small = (Ls if c > r else Rs).double().cpu().numpy()
    s2 = float(g64 @ g64)
    assert abs(small[0, 0] - s2) <= 1e-4 * s2
    # the update
    sig2 = float(np.float32(np.sum(g64 * g64)))
    f = inverse_root_newton(np.diag([sig2 + eps, eps]), sig2 + eps, iters)[0, 0]
    d_want = -lr * f * f * g64
    d_got = Wt.reshape(-1).double().cpu().numpy() - w0.astype(np.float64)
    err = relf(d_got, d_want)
    log(f"  update error {err:.3e}")
    assert err <= 1e-4
    del step, big
    torch.cuda.empty_cache()
