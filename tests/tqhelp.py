"""Test glue between the seeded workloads, the CPU oracle and the GPU library."""
from __future__ import annotations

import math

import numpy as np

import tq_synth
from oracle import attention as oa
from oracle import codebook as ocb
from oracle import quantize as oq
from oracle import rotation as orot

D = 128
BOUNDARY = 1e-6      # decision-boundary band (unit domain) inside which codes may differ
TOL_ATTN = 2e-3      # relative L2 tolerance of decode outputs
# Two GPU results of one attention that differ only in how the work is cut
# (context chunks, query tiles, when the running maximum moves) round each
# softmax weight to float16 on their own (unit roundoff 2^-11): on random data
# they differ by about 2^-11 * sqrt(2/3) = 4e-4 relative L2, while a wrong
# merge or rescale factor moves the result by O(1).
TOL_RECUT = 1e-3
U_F16 = 2.0 ** -11   # float16 unit roundoff (one rounding of a weight)


def log(msg: str):
    print(f"[case] {msg}", flush=True)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def shifted_codebook(bits: int):
    """A codebook that does not mirror around 0: the canonical levels moved up by
    3/16 and rounded to float16 (still ascending and float16-exact), with the
    exact midpoints as thresholds. It takes the kernels' general code search."""
    c, _ = ocb.canonical(bits)
    c = np.asarray(c, dtype=np.float64) + 0.1875
    c = c.astype(np.float16).astype(np.float64)
    assert np.all(np.diff(c) > 0)
    return c, (c[:-1] + c[1:]) / 2


class OracleModel:
    """Oracle rotation, projection and codebooks of a workload."""

    def __init__(self, w: tq_synth.Workload, codebook: str = "gaussian", rotation: str = "haar"):
        self.w = w
        d = w.d
        self.Pi = (orot.hadamard_rotation if rotation == "hadamard" else orot.haar_rotation)(tq_synth.ROT_SEED, d)
        self.S = orot.qjl_projection(tq_synth.QJL_SEED, d) if w.k_qjl else None
        if codebook == "sphere":
            make = lambda bits: ocb.canonical_sphere(bits, d)
        elif codebook == "shifted":
            make = shifted_codebook
        else:
            make = ocb.canonical
        self.cK, self.tK = make(w.k_bits)
        self.cV, self.tV = make(w.v_bits)

    def quantize(self, which: str, X: np.ndarray) -> dict:
        if which == "k":
            return oq.quantize_head(X, self.Pi, self.cK, self.tK, S=self.S)
        return oq.quantize_head(X, self.Pi, self.cV, self.tV)

    def heads(self, which: str, bs=None, hs=None) -> dict:
        w = self.w
        out = {}
        for b in (range(w.B) if bs is None else bs):
            for h in (range(w.H_kv) if hs is None else hs):
                out[(b, h)] = self.quantize(which, tq_synth.kv_head(w, which, b, h))
        return out

    def decode(self, kh: dict, vh: dict, q: np.ndarray, b: int, kv: int, ctx=None) -> np.ndarray:
        w = self.w
        G = w.G
        qs = np.asarray(q[b, kv * G:(kv + 1) * G], dtype=np.float64)
        return oa.attend_rotated(qs, kh[(b, kv)], vh[(b, kv)], self.Pi, self.Pi, self.cK, self.cV, w.d,
                                 1.0 / math.sqrt(w.d), ctx_len=ctx, S=self.S)


def pack_head(role: str, codes: np.ndarray, bits: int, T_cap: int) -> np.ndarray:
    """Oracle-packed words of one head padded to T_cap tokens (uint32)."""
    full = np.zeros((T_cap, codes.shape[1]), dtype=np.int64)
    full[:codes.shape[0]] = codes
    if role == "k":
        return oq.pack_keys(full, bits).reshape(-1)
    return oq.pack_values(full, bits).reshape(-1)


def unpack_head(role: str, words: np.ndarray, bits: int, T: int, d: int = D) -> np.ndarray:
    words = np.asarray(words).view(np.uint32)
    W = d * bits // 32
    if role == "k":
        return oq.unpack_keys(words.reshape(-1, W), bits, d)[:T]
    return oq.unpack_values(words.reshape(-1, 8 * W), bits, d)[:T]


def code_mismatch(role, gpu_words, ref: dict, bits: int, thresholds, T: int):
    """(mismatches, mismatches outside the boundary band, coordinates compared)."""
    d = ref["codes"].shape[1]
    got = unpack_head(role, gpu_words, bits, T, d)
    want = ref["codes"][:T]
    bad = got != want
    exempt = oq.boundary_distance(ref["u"][:T], thresholds, d) < BOUNDARY
    return int(bad.sum()), int((bad & ~exempt).sum()), bad.size


def upload_oracle_cache(tq, model: OracleModel, which: str, heads: dict, T_cap: int, device="cuda"):
    """A device Cache holding the oracle's packed cache (oracle rotation and codebook)."""
    import torch

    w = model.w
    role = tq.KEYS if which == "k" else tq.VALUES
    bits = w.k_bits if which == "k" else w.v_bits
    qjl = which == "k" and w.k_qjl
    cache = tq.Cache(role, bits, w.B, w.H_kv, T_cap, device=device, rot=model.Pi.astype(np.float32),
                     proj=model.S.astype(np.float32) if qjl else None, qjl=qjl,
                     centroids=(model.cK if which == "k" else model.cV).astype(np.float32), d=w.d)
    codes = np.zeros((w.B, w.H_kv, T_cap * w.d * bits // 32), dtype=np.uint32)
    norms = np.zeros((w.B, w.H_kv, T_cap), dtype=np.float32)
    signs = np.zeros((w.B, w.H_kv, T_cap, 4), dtype=np.uint32) if qjl else None
    gamma = np.zeros((w.B, w.H_kv, T_cap), dtype=np.float32) if qjl else None
    for (b, h), r in heads.items():
        T = r["codes"].shape[0]
        codes[b, h] = pack_head(which, r["codes"], bits, T_cap)
        norms[b, h, :T] = r["norm"]
        if qjl:
            signs[b, h, :T] = oq.pack_signs(r["signs"])
            gamma[b, h, :T] = r["gamma"]
    cache.codes.copy_(torch.from_numpy(codes.view(np.int32)))
    cache.norms.copy_(torch.from_numpy(norms))
    if qjl:
        cache.signs.copy_(torch.from_numpy(signs.view(np.int32)))
        cache.gamma.copy_(torch.from_numpy(gamma))
    return cache


def device_inputs(w: tq_synth.Workload, which: str, device="cuda"):
    """Workload K or V as a device tensor [B, T, H_kv, d] in the workload dtype."""
    import torch

    x = torch.from_numpy(tq_synth.kv_full(w, which))
    x = x.to(torch.bfloat16) if w.dtype == "bf16" else x
    return x.to(device)


def device_queries(w: tq_synth.Workload, device="cuda"):
    import torch

    q = torch.from_numpy(tq_synth.queries_full(w))
    q = q.to(torch.bfloat16) if w.dtype == "bf16" else q
    return q.to(device).contiguous()


def gpu_heads(cache, w: tq_synth.Workload, which: str, T: int) -> dict:
    """The GPU cache's own codes, norms (and QJL sign bits and gamma) per
    (row, KV head), in the oracle's per-head form, so that the oracle can decode
    exactly the bytes the kernels read (kernel parity)."""
    bits = w.k_bits if which == "k" else w.v_bits
    codes = cache.codes.cpu().numpy()
    norms = cache.norms.cpu().numpy()
    qjl = which == "k" and w.k_qjl
    if qjl:
        signs = cache.signs.cpu().numpy().view(np.uint32)
        gamma = cache.gamma.cpu().numpy()
    out = {}
    for b in range(w.B):
        for h in range(w.H_kv):
            d = {"codes": unpack_head(which, codes[b, h], bits, T, w.d), "norm": norms[b, h, :T].astype(np.float64)}
            if qjl:
                d["signs"] = oq.unpack_signs(signs[b, h, :T], w.d)
                d["gamma"] = gamma[b, h, :T].astype(np.float64)
            out[(b, h)] = d
    return out


def head_errors(out, ref) -> np.ndarray:
    """Relative L2 error of every output vector (last axis), NaN where the
    reference vector is zero (an empty context)."""
    a = np.asarray(out, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(a - b, axis=-1)
    den = np.linalg.norm(b, axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(den > 0, num / den, np.nan)


def assert_heads(out, ref, tol: float, what: str) -> float:
    """Every output vector (per row, head; per row, token, head for chunked
    attention) within `tol` relative L2 of the reference; where the reference is
    zero the output must be zero too. Returns the worst error."""
    e = head_errors(out, ref)
    zero = np.isnan(e)
    assert np.all(np.asarray(out)[zero] == 0), f"{what}: nonzero output where the reference is zero"
    worst = float(np.nanmax(e)) if np.any(~zero) else 0.0
    idx = np.unravel_index(int(np.nanargmax(np.where(zero, -1.0, e))), e.shape) if np.any(~zero) else None
    assert worst <= tol, f"{what}: worst vector {idx} rel L2 {worst:.3e} > {tol:g}"
    return worst


def band_report(w: tq_synth.Workload, model: "OracleModel", oracle_heads: dict, gpu: dict, b: int, kv: int,
                which: str) -> str:
    """Why one (row, KV head) differs end to end: how many of its codes lie in the
    1e-6 decision-boundary band, how many codes differ from the oracle's, and for
    QJL keys how many tokens carry sign bits that differ."""
    thr = model.tK if which == "k" else model.tV
    ref = oracle_heads[(b, kv)]
    T = ref["codes"].shape[0]
    band = oq.boundary_distance(ref["u"][:T], thr, w.d) < BOUNDARY
    diff = gpu[(b, kv)]["codes"] != ref["codes"][:T]
    msg = f"{which}: {int(band.sum())} band codes, {int(diff.sum())} codes differ"
    if which == "k" and w.k_qjl:
        flipped = np.any(gpu[(b, kv)]["signs"] != ref["signs"][:T], axis=1)
        msg += f", {int(flipped.sum())} tokens with differing sign bits"
    return msg
