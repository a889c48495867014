"""SplitMix64 and Box-Muller normals (oracle side).

The pages only say the rotation is random (ai-accelerate.xyz TurboQuant article,
section "TurboQuantの仕組み", step 1). Reading: the random stream is SplitMix64
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014; the finalizer constants are Vigna's published splitmix64 variant),
a counter-based generator: output k (k = 1, 2, ...) is the 64-bit finalizer
applied to seed + k * 0x9E3779B97F4A7C15 (mod 2**64).

Uniforms take the top 53 bits plus one half: u = ((z >> 11) + 0.5) * 2**-53,
evaluated in IEEE double (the sum rounds to nearest even once z >> 11 >= 2**52),
so u lies in (0, 1] and ln(u) is always finite. Normals come in pairs from consecutive uniforms
(u1, u2) by the Box-Muller transform (Box and Muller, 1958):
r = sqrt(-2 ln u1), first = r cos(2 pi u2), second = r sin(2 pi u2).
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """First n outputs of SplitMix64 started at `seed` (uint64 array)."""
    with np.errstate(over="ignore"):
        k = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniforms(seed: int, n: int) -> np.ndarray:
    """n doubles in (0, 1] from the top 53 bits of each output."""
    z = splitmix64(seed, n)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0**-53


def normals(seed: int, n: int) -> np.ndarray:
    """n standard normals; pair k uses uniforms 2k and 2k+1 (cos first, then sin)."""
    m = (n + 1) // 2
    u = uniforms(seed, 2 * m)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * m)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:n]
