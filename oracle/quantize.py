"""Quantize K/V vectors into the packed cache (oracle side).

Method (ai-accelerate.xyz TurboQuant article, section "TurboQuantの仕組み"):
step 1 rotates each vector with the random orthogonal matrix and quantizes each
rotated coordinate with the Gaussian Lloyd-Max codebook, keeping no per-block
scale; step 2 (QJL, optional, keys) keeps one sign bit per coordinate of a
Gaussian projection of the quantization error.

Readings where the pages are silent:
* Only the vector's Euclidean norm n = |x| is kept (float32). The quantizer acts
  on u = Pi x / n, a unit vector whose coordinates have variance 1/d, so the
  unit-domain levels are centroid / sqrt(d). n = 0 gives u = 0.
* Code rule: code_j = #{ i : u_j >= t_i / sqrt(d) }, i.e. codes ascend with the
  centroid and a value on a threshold goes to the upper cell (u = 0 lands on
  code 2**(bits-1)).
* QJL (keys): r = u - c[code] / sqrt(d), gamma = |r| (float32),
  sign bit_i = [ (S r)_i >= 0 ].
* Bit layouts (all little-endian uint32 words, LSB-first bit streams: stream bit
  k is bit k mod 32 of word k div 32):
    key layout    one record of d*bits/32 words per token; coordinate j's code
                  sits at stream bits [bits*j, bits*j + bits).
    value layout  tokens grouped in blocks of 8 (8*t0 .. 8*t0+7); one block
                  record of 8*d*bits/32 words; the code of token 8*t0 + i at
                  coordinate j sits at stream bits [bits*(8j + i), ... + bits).
    QJL signs     d/32 words per token, bit i = sign bit of coordinate i.
  Both code layouts use d*bits/8 bytes per token.
"""
from __future__ import annotations

import math

import numpy as np

VALUE_BLOCK = 8


def norms(X: np.ndarray) -> np.ndarray:
    """Euclidean norm of each row, float64."""
    X = np.asarray(X, dtype=np.float64)
    return np.sqrt(np.sum(X * X, axis=1))


def unit_rotated(X: np.ndarray, Pi: np.ndarray):
    """(u, n): u = Pi x / n for every row x of X (u = 0 where n = 0)."""
    X = np.asarray(X, dtype=np.float64)
    n = norms(X)
    Y = X @ Pi.T
    safe = np.where(n > 0, n, 1.0)
    U = np.where(n[:, None] > 0, Y / safe[:, None], 0.0)
    return U, n


def codes_from_unit(U: np.ndarray, thresholds: np.ndarray, d: int) -> np.ndarray:
    """code_j = number of thresholds t_i with u_j >= t_i / sqrt(d)."""
    tu = np.asarray(thresholds, dtype=np.float64) / math.sqrt(d)
    codes = np.zeros(U.shape, dtype=np.int64)
    for t in tu:
        codes += (U >= t)
    return codes


def boundary_distance(U: np.ndarray, thresholds: np.ndarray, d: int) -> np.ndarray:
    """Distance of each unit-domain coordinate to its nearest decision threshold."""
    tu = np.asarray(thresholds, dtype=np.float64) / math.sqrt(d)
    return np.min(np.abs(U[..., None] - tu), axis=-1)


def qjl(U: np.ndarray, codes: np.ndarray, centroids: np.ndarray, S: np.ndarray, d: int):
    """(sign bits int [N, d], gamma float64 [N], z = S r) for the quantization residual."""
    R = U - centroids[codes] / math.sqrt(d)
    gamma = np.sqrt(np.sum(R * R, axis=1))
    Z = R @ S.T
    return (Z >= 0.0).astype(np.int64), gamma, Z


def pack_bitstream(seq: np.ndarray, bits: int) -> np.ndarray:
    """Pack rows of small integers LSB-first into uint32 words: element k of a row
    occupies stream bits [bits*k, bits*k + bits)."""
    seq = np.asarray(seq, dtype=np.uint64)
    N, m = seq.shape
    assert (m * bits) % 32 == 0
    words = np.zeros((N, m * bits // 32), dtype=np.uint64)
    for k in range(m):
        pos = bits * k
        w, o = divmod(pos, 32)
        v = seq[:, k] << np.uint64(o)
        words[:, w] |= v & np.uint64(0xFFFFFFFF)
        if o + bits > 32:
            words[:, w + 1] |= v >> np.uint64(32)
    return words.astype(np.uint32)


def unpack_bitstream(words: np.ndarray, bits: int, m: int) -> np.ndarray:
    """Inverse of pack_bitstream: rows of m integers."""
    words = np.asarray(words, dtype=np.uint64)
    N = words.shape[0]
    out = np.zeros((N, m), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for k in range(m):
        pos = bits * k
        w, o = divmod(pos, 32)
        v = words[:, w] >> np.uint64(o)
        if o + bits > 32:
            v |= words[:, w + 1] << np.uint64(32 - o)
        out[:, k] = (v & mask).astype(np.int64)
    return out


def pack_keys(codes: np.ndarray, bits: int) -> np.ndarray:
    """Key layout: [N, d] codes -> [N, d*bits/32] words."""
    return pack_bitstream(codes, bits)


def unpack_keys(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    return unpack_bitstream(words, bits, d)


def pack_values(codes: np.ndarray, bits: int) -> np.ndarray:
    """Value layout for one head: [T, d] codes (T a multiple of 8) -> [T/8, 8*d*bits/32]
    words; within a block the stream runs over coordinates, and over the block's 8
    tokens inside each coordinate."""
    T, d = codes.shape
    assert T % VALUE_BLOCK == 0
    seq = codes.reshape(T // VALUE_BLOCK, VALUE_BLOCK, d).transpose(0, 2, 1).reshape(-1, VALUE_BLOCK * d)
    return pack_bitstream(seq, bits)


def unpack_values(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    nblk = words.shape[0]
    seq = unpack_bitstream(words, bits, VALUE_BLOCK * d)
    return seq.reshape(nblk, d, VALUE_BLOCK).transpose(0, 2, 1).reshape(nblk * VALUE_BLOCK, d)


def pack_signs(signs: np.ndarray) -> np.ndarray:
    return pack_bitstream(signs, 1)


def unpack_signs(words: np.ndarray, d: int) -> np.ndarray:
    return unpack_bitstream(words, 1, d)


def quantize_head(X, Pi, centroids, thresholds, S=None):
    """Quantize the vectors of one head, [T, d] -> dict with codes, norm (float32
    as stored), unit-domain u, and for QJL the sign bits, gamma (float32) and z."""
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[1]
    U, n = unit_rotated(X, Pi)
    codes = codes_from_unit(U, thresholds, d)
    out = {"codes": codes, "norm": n.astype(np.float32), "u": U}
    if S is not None:
        signs, gamma, Z = qjl(U, codes, centroids, S, d)
        out.update(signs=signs, gamma=gamma.astype(np.float32), z=Z)
    return out
