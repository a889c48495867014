"""Seeded random matrices (oracle side).

ai-accelerate.xyz TurboQuant article, section "TurboQuantの仕組み", step 1: each
KV vector is multiplied by a random orthogonal matrix. Reading: the matrix is
Haar-distributed, built as Q diag(sign(diag R)) from the QR factorisation of a
d x d matrix of i.i.d. standard normals (Mezzadri, "How to generate random
matrices from the classical compact groups", Notices AMS 2007), with sign(0)
taken as +1. The Gaussian matrix is filled row-major from the seeded normal
stream. The result is rounded to float32, the precision the library stores, and
used in float64 from there on. y = Pi x.

Step 2 of the same section (QJL) uses a Johnson-Lindenstrauss projection;
reading: S is the d x d Gaussian matrix of its own seed, not orthogonalised,
rounded to float32.
"""
from __future__ import annotations

import numpy as np

from . import rng


def gaussian_matrix(seed: int, d: int) -> np.ndarray:
    """d x d matrix of standard normals, row-major from the seed's stream (float64)."""
    return rng.normals(seed, d * d).reshape(d, d)


def haar_rotation_f64(seed: int, d: int) -> np.ndarray:
    """Haar orthogonal matrix before rounding (float64)."""
    g = gaussian_matrix(seed, d)
    q, r = np.linalg.qr(g)          # Householder QR (LAPACK geqrf/orgqr)
    s = np.where(np.diag(r) >= 0.0, 1.0, -1.0)
    return q * s[None, :]


def haar_rotation(seed: int, d: int) -> np.ndarray:
    """Pi as stored: float32-rounded, returned as float64 values."""
    return haar_rotation_f64(seed, d).astype(np.float32).astype(np.float64)


def qjl_projection(seed: int, d: int) -> np.ndarray:
    """S as stored: float32-rounded Gaussian matrix, returned as float64 values."""
    return gaussian_matrix(seed, d).astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Randomized Hadamard rotation (format variant).
#
# A cheaper orthogonal rotation than the dense Haar matrix: Pi = H D / sqrt(d),
# with H the d x d Sylvester-Hadamard matrix (H[i][j] = (-1)^popcount(i & j),
# d a power of two) and D = diag(s) of seeded random signs; applied with the
# fast Walsh-Hadamard transform it costs O(d log d). Reading: s_j = +1 when the
# top bit of SplitMix64 output j+1 of the seed is 0, else -1. Stored as a
# dense float32 matrix like Pi, so every kernel takes it unchanged.

def sylvester_hadamard(d: int) -> np.ndarray:
    """H_d from the doubling recursion H_2n = [[H, H], [H, -H]] (float64)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_signs(seed: int, d: int) -> np.ndarray:
    z = rng.splitmix64(seed, d)
    return np.where((z >> np.uint64(63)) == 0, 1.0, -1.0)


def hadamard_rotation(seed: int, d: int) -> np.ndarray:
    """Pi = H D / sqrt(d), float32-rounded, returned as float64 values."""
    pi = sylvester_hadamard(d) * hadamard_signs(seed, d)[None, :] / np.sqrt(d)
    return pi.astype(np.float32).astype(np.float64)
