"""Dequantization and decode attention over the packed cache (oracle side).

Decode attention of one new query per head over the cached keys and values,
computed two ways:

* textbook: dequantize every key and value, s_t = scale * q . k_t,
  p = softmax(s), o = sum_t p_t v_t;
* rotated domain: because Pi is orthogonal, q . (Pi^T c) = (Pi q) . c and
  sum_t p_t Pi^T c_t = Pi^T sum_t p_t c_t, so the query is rotated once,
  scores come from codebook levels times key norms, values are summed in the
  rotated domain and one inverse rotation is applied at the end.

The QJL key estimate (ai-accelerate.xyz TurboQuant article, section
"TurboQuantの仕組み", step 2) adds n * gamma * sqrt(pi/2) / d * (S Pi q) . sigma
to the key inner product, sigma_i = 2 bit_i - 1: for a Gaussian row s,
E[sign(s . r) (s . y)] = sqrt(2/pi) (y . r) / |r|, which makes the estimate of
y . r unbiased.

Readings where the pages are silent: scale = 1/sqrt(d); query head h reads KV
head floor(h / G); only tokens t < ctx_len take part; ctx_len = 0 gives a zero
output.
"""
from __future__ import annotations

import math

import numpy as np


def dequantize_head(codes, norm, Pi, centroids, d, signs=None, gamma=None, S=None):
    """x_hat_t = n_t Pi^T (c[code_t] / sqrt(d) [+ gamma_t sqrt(pi/2)/d S^T sigma_t])."""
    W = centroids[np.asarray(codes)] / math.sqrt(d)
    if signs is not None:
        sigma = 2.0 * np.asarray(signs, dtype=np.float64) - 1.0
        W = W + (np.asarray(gamma, dtype=np.float64) * math.sqrt(math.pi / 2.0) / d)[:, None] * (sigma @ S)
    return np.asarray(norm, dtype=np.float64)[:, None] * (W @ Pi)


def softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_textbook(q, K, V, scale, ctx_len=None):
    """o[h] = sum_t softmax_t(scale q[h] . K[t]) V[t] for q [G, d] against one KV head."""
    q = np.asarray(q, dtype=np.float64)
    T = K.shape[0] if ctx_len is None else int(ctx_len)
    if T == 0:
        return np.zeros_like(q)
    s = scale * (q @ np.asarray(K[:T], dtype=np.float64).T)
    return softmax(s) @ np.asarray(V[:T], dtype=np.float64)


def rotated_scores(q, k_codes, k_norm, PiK, cK, d, scale, k_signs=None, k_gamma=None, S=None):
    """Scores of q [G, d] against one packed key head, in the rotated domain."""
    qr = np.asarray(q, dtype=np.float64) @ PiK.T                 # q' = Pi q
    s = (qr @ (cK[np.asarray(k_codes)] / math.sqrt(d)).T)        # q' . c / sqrt(d)
    if k_signs is not None:
        q2 = qr @ S.T                                             # q'' = S q'
        sigma = 2.0 * np.asarray(k_signs, dtype=np.float64) - 1.0
        s = s + (q2 @ sigma.T) * (np.asarray(k_gamma, dtype=np.float64) * math.sqrt(math.pi / 2.0) / d)[None, :]
    return scale * s * np.asarray(k_norm, dtype=np.float64)[None, :]


def attend_rotated(q, k, v, PiK, PiV, cK, cV, d, scale, ctx_len=None, S=None):
    """Rotated-domain decode of q [G, d] over one KV head.

    k, v: dicts with 'codes' [T, d], 'norm' [T] (and for QJL keys 'signs', 'gamma')."""
    T = k["codes"].shape[0] if ctx_len is None else int(ctx_len)
    G = q.shape[0]
    if T == 0:
        return np.zeros((G, d))
    s = rotated_scores(q, k["codes"][:T], k["norm"][:T], PiK, cK, d, scale,
                       k.get("signs")[:T] if "signs" in k else None,
                       k.get("gamma")[:T] if "gamma" in k else None, S)
    p = softmax(s)
    vr = np.asarray(v["norm"][:T], dtype=np.float64)[:, None] * cV[np.asarray(v["codes"][:T])] / math.sqrt(d)
    o_rot = p @ vr                                                # sum_t p_t v'_t
    return o_rot @ PiV                                            # Pi^T o'


def attend_chunk_causal(q, k, v, PiK, PiV, cK, cV, d, scale, ctx_len, S=None):
    """Chunked prefill / multi-query attention over one KV head: q [M, G, d]
    holds the M newest tokens of a context of ctx_len tokens (their keys and
    values already in the cache), token i at position ctx_len - M + i; each
    attends causally to cache tokens 0 .. ctx_len - M + i. Query i is therefore
    the decode of its G heads over the first ctx_len - M + i + 1 tokens (the
    plain definition, one query at a time)."""
    M = q.shape[0]
    out = np.zeros((M, q.shape[1], d))
    for i in range(M):
        n = max(int(ctx_len) - M + i + 1, 0)
        out[i] = attend_rotated(q[i], k, v, PiK, PiV, cK, cV, d, scale, ctx_len=n, S=S)
    return out


def split_partials(s: np.ndarray, vr: np.ndarray, bounds):
    """Per-chunk (m, l, acc) of flash-decoding for scores s [G, T], rotated values vr [T, d]."""
    parts = []
    for a, b in bounds:
        if b <= a:
            parts.append((np.full(s.shape[0], -np.inf), np.zeros(s.shape[0]), np.zeros((s.shape[0], vr.shape[1]))))
            continue
        m = np.max(s[:, a:b], axis=1)
        e = np.exp(s[:, a:b] - m[:, None])
        parts.append((m, e.sum(axis=1), e @ vr[a:b]))
    return parts


def merge_partials(parts):
    """o' = sum_c e^{m_c - M} acc_c / sum_c e^{m_c - M} l_c with M = max_c m_c."""
    M = np.max(np.stack([p[0] for p in parts]), axis=0)
    num = 0.0
    den = 0.0
    for m, l, acc in parts:
        w = np.where(np.isfinite(m), np.exp(m - M), 0.0)
        num = num + w[:, None] * acc
        den = den + w * l
    return num / den[:, None]


def cosine(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Row-wise cosine similarity."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.sum(a * b, axis=1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))
