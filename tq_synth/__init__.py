"""Seeded synthetic workloads for the TurboQuant KV-cache path.

This module only draws random inputs (keys, values, queries) with the shapes and
value distributions of the five workloads below. It holds none of the method's
arithmetic: no rotation, no codebook, no quantization. Both the CPU oracle and
the HIP path receive the same bytes from here.

Workloads (shapes and distributions restate the workload descriptions that come
with the method's KV-cache claims; the Qwen-like norm ranges are the key/value
norm figures quoted for Qwen models on the ai-accelerate.xyz page, section on
what TurboQuant means for local LLM users):

  tiny       B=1,  H_q=16, H_kv=1, T=1024,   fp32, N(0,1) x 10**U(0,1) per token
  llama8b    B=1,  H_q=32, H_kv=8, T=32768,  bf16, N(0,1), 4 outlier channels x20
  qwen       B=4,  H_q=28, H_kv=4, T=131072, bf16, sphere directions,
                   |k| ~ U[172,778], |v| ~ U[2,4]
  qjl        B=16, H_q=32, H_kv=8, T=8192,   bf16, N(0,1)
  stress70b  B=32, H_q=64, H_kv=8, T=32768,  bf16, N(0,1), 1% of tokens x10

Every (tensor, batch row, head) slice has its own PCG64 stream derived from
(data seed, tensor id, b, h), so any slice can be regenerated on its own.
Values of bf16 workloads are rounded to bf16 (round to nearest even) and
returned as float32 arrays holding those exact values.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

D = 128

# tensor ids for stream derivation
_K, _V, _Q, _OUTLIER_CH, _TOKEN_POS, _NORMS = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    T: int
    dtype: str            # "f32" or "bf16": dtype of K, V and q
    kind: str             # distribution recipe
    seed: int
    k_bits: int = 3
    v_bits: int = 3
    k_qjl: int = 0
    d: int = D

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    def scaled(self, **kw) -> "Workload":
        """Same recipe with some sizes replaced (for fast test cases)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 1, 1024, "f32", "lognorm", 1001),
    "llama8b": Workload("llama8b", 1, 32, 8, 32768, "bf16", "outlier_channels", 1002),
    "qwen": Workload("qwen", 4, 28, 4, 131072, "bf16", "sphere_norms", 1003, k_bits=4, v_bits=2),
    "qjl": Workload("qjl", 16, 32, 8, 8192, "bf16", "normal", 1004, k_bits=2, v_bits=3, k_qjl=1),
    "stress70b": Workload("stress70b", 32, 64, 8, 32768, "bf16", "token_outliers", 1005),
}

# Rotation / projection seeds used by all workloads.
ROT_SEED = 42
QJL_SEED = 4242


def _rng(seed: int, *path: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *path])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return (u & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def _finish(w: Workload, x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    return round_bf16(x) if w.dtype == "bf16" else x


def outlier_channels(w: Workload, which: str, h: int) -> np.ndarray:
    """The 4 distinct outlier channels of KV head h (drawn separately for K and V)."""
    tid = _K if which == "k" else _V
    return np.sort(_rng(w.seed, _OUTLIER_CH, tid, h).choice(w.d, size=4, replace=False))


def outlier_tokens(w: Workload, b: int) -> np.ndarray:
    """1% of token positions of batch row b (shared by all heads and by K and V)."""
    n = int(round(0.01 * w.T))
    return np.sort(_rng(w.seed, _TOKEN_POS, b).choice(w.T, size=n, replace=False))


def kv_head(w: Workload, which: str, b: int, h: int) -> np.ndarray:
    """K or V vectors of (batch row b, KV head h): float32 [T, d]."""
    assert which in ("k", "v")
    tid = _K if which == "k" else _V
    g = _rng(w.seed, tid, b, h)
    x = g.standard_normal((w.T, w.d), dtype=np.float32)
    if w.kind == "lognorm":
        x *= (10.0 ** g.random(w.T, dtype=np.float64)).astype(np.float32)[:, None]
    elif w.kind == "outlier_channels":
        x[:, outlier_channels(w, which, h)] *= 20.0
    elif w.kind == "sphere_norms":
        lo, hi = (172.0, 778.0) if which == "k" else (2.0, 4.0)
        nrm = g.uniform(lo, hi, size=w.T)
        x64 = x.astype(np.float64)
        x64 /= np.linalg.norm(x64, axis=1, keepdims=True)
        x = (x64 * nrm[:, None]).astype(np.float32)
    elif w.kind == "token_outliers":
        x[outlier_tokens(w, b)] *= 10.0
    elif w.kind == "normal":
        pass
    else:
        raise ValueError(w.kind)
    return _finish(w, x)


def queries(w: Workload, b: int) -> np.ndarray:
    """Decode queries of batch row b: float32 [H_q, d], N(0,1)."""
    g = _rng(w.seed, _Q, b)
    return _finish(w, g.standard_normal((w.H_q, w.d), dtype=np.float32))


def kv_full(w: Workload, which: str) -> np.ndarray:
    """All K or V vectors in the [B][T][H_kv][d] input layout (small workloads only)."""
    out = np.empty((w.B, w.T, w.H_kv, w.d), dtype=np.float32)
    for b in range(w.B):
        for h in range(w.H_kv):
            out[b, :, h, :] = kv_head(w, which, b, h)
    return out


def queries_full(w: Workload) -> np.ndarray:
    return np.stack([queries(w, b) for b in range(w.B)])


def random_unit_vectors(n: int, d: int, seed: int) -> np.ndarray:
    """Directions uniform on the sphere S^{d-1}, float64 [n, d]."""
    g = _rng(seed, 99)
    x = g.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def torch_kv(w: Workload, which: str, device, seed_offset: int = 0):
    """The same recipe drawn with torch's generator on `device`, in the [B][T][H_kv][d]
    layout and the workload's dtype. Used where only the distribution matters (timing):
    the values differ from kv_head's."""
    import torch

    tid = _K if which == "k" else _V
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed * 1000 + tid * 10 + seed_offset)
    x = torch.randn((w.B, w.T, w.H_kv, w.d), generator=gen, device=device, dtype=torch.float32)
    if w.kind == "lognorm":
        s = 10.0 ** torch.rand((w.B, w.T, 1, 1), generator=gen, device=device)
        x *= s
    elif w.kind == "outlier_channels":
        for h in range(w.H_kv):
            ch = torch.as_tensor(outlier_channels(w, which, h), device=device)
            x[:, :, h, ch] *= 20.0
    elif w.kind == "sphere_norms":
        lo, hi = (172.0, 778.0) if which == "k" else (2.0, 4.0)
        x /= x.norm(dim=-1, keepdim=True)
        x *= lo + (hi - lo) * torch.rand((w.B, w.T, w.H_kv, 1), generator=gen, device=device)
    elif w.kind == "token_outliers":
        for b in range(w.B):
            pos = torch.as_tensor(outlier_tokens(w, b), device=device)
            x[b, pos] *= 10.0
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return x.to(dt)


def torch_queries(w: Workload, device, seed_offset: int = 0):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed * 1000 + _Q * 10 + seed_offset)
    q = torch.randn((w.B, w.H_q, w.d), generator=gen, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16 if w.dtype == "bf16" else torch.float32)
