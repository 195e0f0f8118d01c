"""Coefficients of the GELU used by the GPU kernels' forward epilogues.

GELU(z) = z * Phi(z) (the exact, erf form of the activation the expert FFNs
apply; survey notes sec. 1.1.2.1).  Written as

    GELU(z) = max(z, 0) - |z| * Q(|z|),   Q(x) = Phi(-x)  (the normal tail),

which holds for either sign of z.  The kernels evaluate
Q(x) = 2^g(u), u = min(x, 6) / 3 - 1, with g a degree-9 polynomial in u fitted
here to log2 Q on [0, 6]: one exp2 per element and no reciprocal (the
Abramowitz-Stegun 7.1.26 form of erf needs both).  Past x = 6 the clamp keeps
Q at Q(6) ~ 1e-9, so |z| Q(|z|) stays below 1e-9 |z|.

The fit is a Chebyshev least-squares fit whose weights are reweighted toward
the minimax (Lawson) solution, then converted to monomials in u; the kernel
evaluates it in fp32 by Horner's rule.  Max |GELU error| of that fp32
evaluation: about 3e-7 (tests/test_gelu_cpu.py checks the coefficients in
csrc/common.h against this fit and the error bound).

    python -m mixture_experts_layer_24_amd.gelu_fit     prints the coefficients
"""
from __future__ import annotations

import math

import numpy as np

DEGREE = 9
XMAX = 6.0


def fit(degree: int = DEGREE, xmax: float = XMAX, nodes: int = 6000, sweeps: int = 30):
    """Monomial coefficients (u^0 first, fp32) of g(u) ~ log2 Q(xmax/2 (u + 1))."""
    from scipy.special import log_ndtr
    u = np.cos(np.pi * (np.arange(nodes) + 0.5) / nodes)
    g = log_ndtr(-xmax / 2 * (u + 1)) / math.log(2.0)
    V = np.polynomial.chebyshev.chebvander(u, degree)
    w = np.ones(nodes)
    for _ in range(sweeps):
        c, *_ = np.linalg.lstsq(V * w[:, None], g * w, rcond=None)
        r = np.abs(V @ c - g)
        w = w * np.sqrt(r + 1e-30)
        w /= w.max()
    return np.polynomial.chebyshev.cheb2poly(c).astype(np.float32)


def gelu_fp32(z, coeffs):
    """The kernels' evaluation order in fp32 (numpy), for checking."""
    f = np.float32
    z = np.asarray(z, dtype=f)
    x = np.minimum(np.abs(z), f(XMAX))
    u = (x * f(1.0 / 3.0) + f(-1.0)).astype(f)
    g = f(coeffs[-1])
    for c in coeffs[-2::-1]:
        g = (g * u + f(c)).astype(f)
    return (np.maximum(z, f(0)) - np.abs(z) * np.exp2(g).astype(f)).astype(f)


if __name__ == "__main__":
    for i, c in enumerate(fit()):
        print(f"u^{i}: {c:.9e}f")
