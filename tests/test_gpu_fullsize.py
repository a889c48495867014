"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic context split), on sampled (row, KV head) slices
that the CPU oracle computes one by one.

Inputs come from the seeded on-device generator the benchmark uses
(tq_synth.torch_kv / torch_queries); the sampled input slices are copied to the
host and given to the oracle unchanged. For each sampled slice:
  * codes (bit-exact outside the decision-boundary band), norms (and QJL signs
    and gammas) of every token against the oracle's quantization of the slice;
  * decode outputs of its G query heads against the oracle's decode of the
    GPU's own packed codes (kernel parity) and of the oracle's codes (end to
    end), relative L2 within 2e-3;
and for the whole output, properties that hold at any size (finite values,
identical results on repeat, agreement between context splits).
"""
import math

import numpy as np
import pytest

import tq_synth
from tqhelp import BOUNDARY, TOL_ATTN, TOL_RECUT, OracleModel, code_mismatch, log, rel_l2, unpack_head

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = tq_synth.WORKLOADS


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_tq_amd as lib
    return lib


def _sample(w, n, seed):
    rng = np.random.default_rng(seed)
    pairs = [(int(b), int(h)) for b in range(w.B) for h in range(w.H_kv)]
    if len(pairs) <= n:
        return pairs
    idx = rng.choice(len(pairs), size=n, replace=False)
    return sorted(pairs[i] for i in idx)


def _gpu_head(tq, w, which, cache, b, h, T):
    """The GPU's packed slice (b, h) as the oracle's code dictionary."""
    bits = w.k_bits if which == "k" else w.v_bits
    words = cache.codes[b, h].cpu().numpy()
    r = {"codes": unpack_head(which, words, bits, T),
         "norm": cache.norms[b, h, :T].cpu().numpy().astype(np.float64)}
    if which == "k" and w.k_qjl:
        from oracle import quantize as oq
        r["signs"] = oq.unpack_signs(cache.signs[b, h, :T].cpu().numpy().view(np.uint32), 128)
        r["gamma"] = cache.gamma[b, h, :T].cpu().numpy().astype(np.float64)
    return r


def _check_codes(model, which, ref, got, w, b, h):
    from oracle import quantize as oq
    bits = w.k_bits if which == "k" else w.v_bits
    thr = model.tK if which == "k" else model.tV
    bad = got["codes"] != ref["codes"]
    exempt = oq.boundary_distance(ref["u"], thr, 128) < BOUNDARY
    outside = int((bad & ~exempt).sum())
    nr, want = got["norm"], ref["norm"].astype(np.float64)
    assert np.all(np.abs(nr - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)
    if which == "k" and w.k_qjl:
        flip_vec = np.any(exempt, axis=1)
        sb = (got["signs"] != ref["signs"]) & ~(np.abs(ref["z"]) < BOUNDARY) & ~flip_vec[:, None]
        outside += int(sb.sum())
        ok = np.abs(got["gamma"] - ref["gamma"]) <= 1e-5 * ref["gamma"] + 1e-7
        assert np.all(ok | flip_vec), (b, h)
    return int(bad.sum()), outside, bad.size


def _full_case(tq, name, n_sample, ctx_lens=None, seed=7):
    w = W[name]
    dev = torch.device("cuda")
    T = w.T
    T_cap = (T + 7) // 8 * 8
    log(f"full size {name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} T={T} K{w.k_bits}{'+qjl' if w.k_qjl else ''}"
        f"/V{w.v_bits}, {n_sample} sampled (row, KV head) slices")
    model = OracleModel(w)
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, device=dev, qjl=bool(w.k_qjl))
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, device=dev)
    xk = tq_synth.torch_kv(w, "k", dev)
    xv = tq_synth.torch_kv(w, "v", dev)
    tq.quantize_kv(xk, kc)
    tq.quantize_kv(xv, vc)
    q = tq_synth.torch_queries(w, dev)
    n_split = tq.decode_splits(w.B, w.H_kv, T)
    ws = tq.Workspace(tq.decode_workspace_bytes(w.B, w.H_q, w.H_kv, T, 0, w.k_qjl), dev)
    cl = None if ctx_lens is None else torch.tensor(ctx_lens, dtype=torch.int32, device=dev)
    out = tq.decode_attention(kc, vc, q, ctx_lens=cl, T=T, workspace=ws)
    again = tq.decode_attention(kc, vc, q, ctx_lens=cl, T=T, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "decode is not deterministic"
    assert bool(torch.isfinite(out).all())
    log(f"  automatic split: {n_split} context chunk(s) per (row, KV head)")
    qn = q.float().cpu().numpy()
    outn = out.cpu().numpy()
    G = w.G
    stats = {"k": [0, 0, 0], "v": [0, 0, 0]}
    kern_err, e2e_err = [], []
    for (b, h) in _sample(w, n_sample, seed):
        ctx = None if ctx_lens is None else int(ctx_lens[b])
        heads = {}
        for which, x, cache in (("k", xk, kc), ("v", xv, vc)):
            X = x[b, :, h].float().cpu().numpy()
            ref = model.quantize(which, X)
            got = _gpu_head(tq, w, which, cache, b, h, T)
            m, o, n = _check_codes(model, which, ref, got, w, b, h)
            stats[which] = [stats[which][0] + m, stats[which][1] + o, stats[which][2] + n]
            heads[which] = (ref, got)
        kh = {(b, h): heads["k"][1]}
        vh = {(b, h): heads["v"][1]}
        want = model.decode(kh, vh, qn, b, h, ctx)
        got_o = outn[b, h * G:(h + 1) * G]
        kern_err.append(rel_l2(got_o, want) if np.linalg.norm(want) > 0 else float(np.abs(got_o).max()))
        kh = {(b, h): heads["k"][0]}
        vh = {(b, h): heads["v"][0]}
        want = model.decode(kh, vh, qn, b, h, ctx)
        e2e_err.append(rel_l2(got_o, want) if np.linalg.norm(want) > 0 else float(np.abs(got_o).max()))
    for which in ("k", "v"):
        m, o, n = stats[which]
        log(f"  {which} codes: {m}/{n} differ ({m / n:.2e}); outside the {BOUNDARY:g} band: {o}")
        assert o == 0
    log(f"  decode rel L2, kernel parity: worst {max(kern_err):.3e}; end to end: worst {max(e2e_err):.3e}")
    assert max(kern_err) <= TOL_ATTN
    assert max(e2e_err) <= TOL_ATTN
    return tq, w, kc, vc, q, out, cl, ws


def test_fullsize_stress70b(tq):
    """The benchmarked workload: B=32, H_q=64, H_kv=8, T=32768, 3-bit K and V,
    decoded in one launch (one context chunk per (row, KV head))."""
    _, w, kc, vc, q, out, cl, ws = _full_case(tq, "stress70b", n_sample=8)
    assert tq.decode_splits(w.B, w.H_kv, w.T) == 1
    # the same heads through the split path: 4 context chunks and the combine
    ws4 = tq.Workspace(tq.decode_workspace_bytes(w.B, w.H_q, w.H_kv, w.T, 4, 0), torch.device("cuda"))
    out4 = tq.decode_attention(kc, vc, q, T=w.T, n_split=4, workspace=ws4)
    err = rel_l2(out4.cpu().numpy(), out.cpu().numpy())
    log(f"  4 chunks vs 1 chunk: rel L2 {err:.3e}")
    assert err <= TOL_RECUT


def test_fullsize_stress70b_ragged(tq):
    """Same workload with ragged context lengths (empty, single token, partial
    steps, partial value blocks, full)."""
    w = W["stress70b"]
    rng = np.random.default_rng(11)
    ctx = rng.integers(0, w.T + 1, size=w.B)
    ctx[:6] = [0, 1, 7, 33, w.T - 1, w.T]
    _full_case(tq, "stress70b", n_sample=8, ctx_lens=[int(c) for c in ctx], seed=3)


def test_fullsize_llama8b(tq):
    """B=1, H_q=32, H_kv=8, T=32768 with outlier channels: every KV head, 32 chunks."""
    _full_case(tq, "llama8b", n_sample=8)


def test_fullsize_qwen(tq):
    """B=4, H_q=28, H_kv=4 (G=7), T=131072, K4/V2 with Qwen-like norms."""
    _full_case(tq, "qwen", n_sample=4)


def test_fullsize_qjl(tq):
    """B=16, H_q=32, H_kv=8, T=8192, 2-bit keys with the QJL sketch, 3-bit values."""
    _full_case(tq, "qjl", n_sample=6)
