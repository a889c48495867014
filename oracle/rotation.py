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
