"""Gaussian Lloyd-Max scalar codebook (oracle side).

ai-accelerate.xyz TurboQuant article, section "TurboQuantの仕組み", step 1: after
the rotation each coordinate is close to Gaussian and is quantized on its own
with the optimal scalar (Lloyd-Max) quantizer. Reading: the quantizer is the
Lloyd-Max quantizer of the standard normal N(0, 1) with 2**bits cells (Lloyd
1982; Max 1960); a rotated unit vector has coordinates of variance 1/d, so the
unit-domain levels are centroid / sqrt(d).

Lloyd's iteration, in the order the method states it:
  start  c_i = Phi^-1((i + 1/2) / L)
  repeat t_i = (c_i + c_{i+1}) / 2
         c_i = E[X | t_{i-1} <= X < t_i] = (phi(t_{i-1}) - phi(t_i)) / (Phi(t_i) - Phi(t_{i-1}))
  until the largest change is below 1e-14; then symmetrise (c_i = -c_{L-1-i}).

Canonical stored form (reading; the pages fix no precision): centroids rounded
to float16, round to nearest even; thresholds are the exact midpoints of
neighbouring rounded centroids, the middle one being +0.0. Codes ascend with the
centroid value.
"""
from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(x: float) -> float:
    return 0.0 if math.isinf(x) else _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _upper_tail(x: float) -> float:
    """1 - Phi(x), accurate in the upper tail."""
    return 0.5 * math.erfc(x / _SQRT2)


def _cell_prob(a: float, b: float) -> float:
    return _upper_tail(a) - _upper_tail(b)


def lloyd_max_gaussian(bits: int, tol: float = 1e-14, max_iter: int = 200000):
    """Unrounded Lloyd-Max centroids of N(0,1) with 2**bits levels.

    Returns (centroids float64 [L], iterations, final max change)."""
    L = 1 << bits
    nd = NormalDist()
    c = [nd.inv_cdf((i + 0.5) / L) for i in range(L)]
    delta = math.inf
    it = 0
    while delta >= tol and it < max_iter:
        t = [-math.inf] + [(c[i] + c[i + 1]) / 2.0 for i in range(L - 1)] + [math.inf]
        new = [(_phi(t[i]) - _phi(t[i + 1])) / _cell_prob(t[i], t[i + 1]) for i in range(L)]
        delta = max(abs(a - b) for a, b in zip(new, c))
        c = new
        it += 1
    c = np.array(c)
    c = (c - c[::-1]) / 2.0
    return c, it, delta


def lloyd_residual(c: np.ndarray) -> float:
    """max |c_i - E[X | cell_i]| for the cells the midpoints of c define."""
    L = len(c)
    t = [-math.inf] + [(c[i] + c[i + 1]) / 2.0 for i in range(L - 1)] + [math.inf]
    cm = [(_phi(t[i]) - _phi(t[i + 1])) / _cell_prob(t[i], t[i + 1]) for i in range(L)]
    return float(np.max(np.abs(np.array(cm) - c)))


def expected_sq_error(c: np.ndarray, t: np.ndarray) -> float:
    """E[(X - c(X))^2] for X ~ N(0,1), cells bounded by thresholds t (len L-1).

    Uses int_a^b (x - c)^2 phi(x) dx
        = (1 + c^2) P[a,b] - (b phi(b) - a phi(a)) + 2 c (phi(b) - phi(a))."""
    edges = [-math.inf] + [float(v) for v in t] + [math.inf]
    tot = 0.0
    for i, ci in enumerate(c):
        a, b = edges[i], edges[i + 1]
        p = _cell_prob(a, b)
        aphi = 0.0 if math.isinf(a) else a * _phi(a)
        bphi = 0.0 if math.isinf(b) else b * _phi(b)
        tot += (1.0 + ci * ci) * p - (bphi - aphi) + 2.0 * ci * (_phi(b) - _phi(a))
    return tot


def mse_fixed_point(c: np.ndarray) -> float:
    """MSE of a Lloyd fixed point: 1 - sum c_i^2 P_i (centroids are conditional means)."""
    L = len(c)
    t = [-math.inf] + [(c[i] + c[i + 1]) / 2.0 for i in range(L - 1)] + [math.inf]
    return 1.0 - sum(c[i] ** 2 * _cell_prob(t[i], t[i + 1]) for i in range(L))


def canonical(bits: int):
    """Stored codebook: (centroids, thresholds) as float64 holding fp16-exact centroids
    and their exact midpoints; the middle threshold is +0.0."""
    c, _, _ = lloyd_max_gaussian(bits)
    c16 = c.astype(np.float16).astype(np.float64)
    t = (c16[:-1] + c16[1:]) / 2.0
    t[len(t) // 2] = 0.0
    return c16, t


# ---------------------------------------------------------------------------
# Sphere-exact codebook (format variant).
#
# The article's step 1 says the rotated coordinates are close to Gaussian; the
# exact law of one coordinate u of a uniformly random unit vector in d
# dimensions has density proportional to (1 - u^2)^((d - 3)/2) on [-1, 1]
# (equivalently (1 + u)/2 ~ Beta((d-1)/2, (d-1)/2)). This variant runs the same
# Lloyd iteration on that law, in the same standard units z = u sqrt(d) (so
# E[z^2] = 1), with the same canonical stored form (float16 centroids, exact
# midpoints, middle threshold +0.0).
#   P(a <= u < b)          = I_{(1+b)/2}(al, al) - I_{(1+a)/2}(al, al),  al = (d-1)/2
#   int_a^b u f(u) du      = ((1 - a^2)^(k+1) - (1 - b^2)^(k+1)) / (2 (k+1) B(1/2, k+1)),  k = (d-3)/2
# (the second from d/du (1 - u^2)^(k+1) = -2 (k+1) u (1 - u^2)^k, and
# int_{-1}^{1} (1 - u^2)^k du = B(1/2, k+1)).

def _sphere_cdf(u: float, d: int) -> float:
    from scipy.special import betainc
    al = (d - 1) / 2.0
    x = min(max((1.0 + u) / 2.0, 0.0), 1.0)
    return float(betainc(al, al, x))


def _sphere_partial_mean(a: float, b: float, d: int) -> float:
    """int_a^b u f(u) du for the sphere-coordinate density f (u in [-1, 1])."""
    from scipy.special import betaln
    k = (d - 3) / 2.0
    lb = betaln(0.5, k + 1.0)
    def g(u):
        v = 1.0 - u * u
        return 0.0 if v <= 0.0 else math.exp((k + 1.0) * math.log(v) - lb)
    return (g(a) - g(b)) / (2.0 * (k + 1.0))


def lloyd_max_sphere(bits: int, d: int, tol: float = 1e-14, max_iter: int = 200000):
    """Unrounded Lloyd-Max centroids (standard units) of one coordinate of a
    uniform unit vector in d >= 3 dimensions. Returns (centroids, iterations, last change)."""
    from scipy.special import betaincinv
    L = 1 << bits
    sd = math.sqrt(d)
    al = (d - 1) / 2.0
    # start at the quantiles (i + 1/2) / L of the law, as the Gaussian iteration does
    c = [sd * (2.0 * float(betaincinv(al, al, (i + 0.5) / L)) - 1.0) for i in range(L)]
    delta = math.inf
    it = 0
    while delta >= tol and it < max_iter:
        t = [-1.0] + [min(max((c[i] + c[i + 1]) / 2.0 / sd, -1.0), 1.0) for i in range(L - 1)] + [1.0]
        new = []
        for i in range(L):
            p = _sphere_cdf(t[i + 1], d) - _sphere_cdf(t[i], d)
            new.append(sd * _sphere_partial_mean(t[i], t[i + 1], d) / p)
        delta = max(abs(a - b) for a, b in zip(new, c))
        c = new
        it += 1
    c = np.array(c)
    c = (c - c[::-1]) / 2.0
    return c, it, delta


def sphere_cell_probs(c: np.ndarray, d: int) -> np.ndarray:
    """P(cell i) under the sphere law for the cells the midpoints of c (standard units) define."""
    sd = math.sqrt(d)
    L = len(c)
    t = [-1.0] + [min(max((c[i] + c[i + 1]) / 2.0 / sd, -1.0), 1.0) for i in range(L - 1)] + [1.0]
    return np.array([_sphere_cdf(t[i + 1], d) - _sphere_cdf(t[i], d) for i in range(L)])


def mse_fixed_point_sphere(c: np.ndarray, d: int) -> float:
    """MSE (standard units) of a Lloyd fixed point of the sphere law: 1 - sum c_i^2 P_i."""
    return 1.0 - float(np.sum(np.asarray(c) ** 2 * sphere_cell_probs(c, d)))


def canonical_sphere(bits: int, d: int = 128):
    """Stored sphere codebook: fp16-exact centroids and exact midpoints (middle +0.0)."""
    c, _, _ = lloyd_max_sphere(bits, d)
    c16 = c.astype(np.float16).astype(np.float64)
    t = (c16[:-1] + c16[1:]) / 2.0
    t[len(t) // 2] = 0.0
    return c16, t
