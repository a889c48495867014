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
    r = {"codes": unpack_head(which, words, bits, T, w.d),
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
    exempt = oq.boundary_distance(ref["u"], thr, w.d) < BOUNDARY
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


def _full_case(tq, name, n_sample, ctx_lens=None, seed=7, w=None, rotation="haar"):
    w = W[name] if w is None else w
    dev = torch.device("cuda")
    T = w.T
    T_cap = (T + 7) // 8 * 8
    log(f"full size {name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} d={w.d} T={T} K{w.k_bits}{'+qjl' if w.k_qjl else ''}"
        f"/V{w.v_bits}, {n_sample} sampled (row, KV head) slices")
    model = OracleModel(w, rotation=rotation)
    rot = tq.make_rotation(tq_synth.ROT_SEED, tq.HADAMARD, w.d) if rotation == "hadamard" else None
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, device=dev, qjl=bool(w.k_qjl), d=w.d, rot=rot)
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, device=dev, d=w.d, rot=rot)
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
    # the same heads through the split path: 4 context chunks and the merge
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


@pytest.mark.parametrize("d", [64, 256])
def test_fullsize_stress70b_head_dims(tq, d):
    """The benchmark's head-dimension legs: the 70B-like shape (B=32, H_q=64,
    H_kv=8, T=32768, K3/V3) at d = 64 and 256, quantized on MFMA and decoded
    in one launch on the scan tiles."""
    _full_case(tq, f"stress70b_d{d}", n_sample=6, w=W["stress70b"].scaled(d=d))


def test_fullsize_stress70b_hadamard(tq):
    """The benchmark's second prefill: the 70B-like layer quantized with the
    randomized Hadamard rotation (the bulk kernel's one-pass sign-matrix path),
    codes against the oracle built with the same rotation, then decoded."""
    _full_case(tq, "stress70b_hadamard", n_sample=6, w=W["stress70b"], rotation="hadamard")


def test_fullsize_llama8b(tq):
    """B=1, H_q=32, H_kv=8, T=32768 with outlier channels: every KV head, 32 chunks."""
    _full_case(tq, "llama8b", n_sample=8)


def test_fullsize_qwen(tq):
    """B=4, H_q=28, H_kv=4 (G=7), T=131072, K4/V2 with Qwen-like norms."""
    _full_case(tq, "qwen", n_sample=4)


def test_fullsize_qjl(tq):
    """B=16, H_q=32, H_kv=8, T=8192, 2-bit keys with the QJL sketch, 3-bit values."""
    _full_case(tq, "qjl", n_sample=6)


def test_fullsize_stress70b_prefill(tq):
    """Chunked causal attention on the full 70B-like caches in the launch
    configuration the benchmark times (M = 2: the decode's column tiles; M = 16
    and 128: the dense kernel, automatic context split, queries drawn as the
    benchmark draws them). Sampled (row, KV head) slices and query tokens: the
    oracle decodes query token i over the first ctx - M + i + 1 tokens of the
    GPU's own packed codes (the causal definition, one query at a time), per
    (row, token, head) within 2e-3; for the whole output, finite values,
    identical results on repeat, a forced context split within the recut bound,
    and the last token equal to a decode over the whole context."""
    from oracle import attention as oa
    w = W["stress70b"]
    dev = torch.device("cuda")
    T = w.T
    model = OracleModel(w)
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T, device=dev)
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T, device=dev)
    tq.quantize_kv(tq_synth.torch_kv(w, "k", dev), kc)
    tq.quantize_kv(tq_synth.torch_kv(w, "v", dev), vc)
    torch.cuda.synchronize()
    slices = _sample(w, 3, seed=11)
    heads = {(b, h): (_gpu_head(tq, w, "k", kc, b, h, T), _gpu_head(tq, w, "v", vc, b, h, T)) for b, h in slices}
    sc = 1 / math.sqrt(128)
    for M, toks in ((2, (0, 1)), (16, (0, 7, 15)), (128, (0, 64, 127))):
        q = torch.randn((w.B, M, w.H_q, w.d), generator=torch.Generator(device=dev).manual_seed(M), device=dev)
        q = q.to(torch.bfloat16)
        ws = tq.Workspace(tq.prefill_workspace_bytes(w.B, w.H_q, w.H_kv, M, T, 0, 0), dev)
        out = tq.prefill_attention(kc, vc, q, T=T, workspace=ws)
        again = tq.prefill_attention(kc, vc, q, T=T, workspace=ws)
        split4 = tq.prefill_attention(kc, vc, q, T=T, n_split=4)
        last = tq.decode_attention(kc, vc, q[:, -1].contiguous(), T=T)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all()), M
        assert torch.equal(out, again), M
        outn = out.cpu().numpy()
        assert rel_l2(split4.cpu().numpy(), outn) <= TOL_RECUT, M
        assert rel_l2(outn[:, -1], last.cpu().numpy()) <= TOL_RECUT, M
        qn = q.float().cpu().numpy().astype(np.float64)
        worst = 0.0
        for (b, h), (gk, gv) in heads.items():
            for i in toks:
                n = T - M + i + 1
                want = oa.attend_rotated(qn[b, i, h * w.G:(h + 1) * w.G], gk, gv, model.Pi, model.Pi, model.cK,
                                         model.cV, 128, sc, ctx_len=n)
                got = outn[b, i, h * w.G:(h + 1) * w.G]
                for g in range(w.G):
                    e = rel_l2(got[g], want[g])
                    worst = max(worst, e)
                    assert e <= TOL_ATTN, (M, b, h, i, g, e)
        log(f"  prefill M={M} at full size: kernel parity worst (row, token, head) {worst:.2e} over "
            f"{len(heads)} slices x {len(toks)} tokens")


def test_fullsize_stress70b_one_call_step(tq):
    """The step the benchmark times, at full size: one call that appends a new
    key and value per (row, KV head) at token T - 1 and decodes (one launch)
    equals the separate append (tq_append_kv) followed by the decode, bit for
    bit in the outputs and in every byte of both caches. The fresh token (not
    the one the prefill quantized there) rewrites token T - 1's codes and moves
    the output (not in every row: where a few outlier tokens dominate a row's
    scores, the new token's weight is below float32's range)."""
    w = W["stress70b"]
    dev = torch.device("cuda")
    T = w.T
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T, device=dev)
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T, device=dev)
    tq.quantize_kv(tq_synth.torch_kv(w, "k", dev), kc)
    tq.quantize_kv(tq_synth.torch_kv(w, "v", dev), vc)
    q = tq_synth.torch_queries(w, dev)
    before = tq.decode_attention(kc, vc, q, T=T)
    old_last = kc.codes.view(w.B, w.H_kv, T, -1)[:, :, T - 1].clone()
    g = torch.Generator(device=dev).manual_seed(5)
    new_k = (4 * torch.randn((w.B, 1, w.H_kv, w.d), generator=g, device=dev)).to(torch.bfloat16)
    new_v = (4 * torch.randn((w.B, 1, w.H_kv, w.d), generator=g, device=dev)).to(torch.bfloat16)
    k2 = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T, device=dev)
    v2 = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T, device=dev)
    for dst, src in ((k2, kc), (v2, vc)):
        dst.codes.copy_(src.codes)
        dst.norms.copy_(src.norms)
    one = tq.decode_attention_append(kc, vc, new_k, new_v, q, T=T)
    tq.append_kv(new_k, new_v, k2, v2, T - 1)
    two = tq.decode_attention(k2, v2, q, T=T)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    for x, y in ((kc, k2), (vc, v2)):
        assert torch.equal(x.codes, y.codes)
        assert torch.equal(x.norms, y.norms)
    moved = (one - before).abs().flatten(1).amax(dim=1)
    log(f"  one-call step at full size: bitwise equal to append + decode; output moved by "
        f"{moved.min().item():.3e} .. {moved.max().item():.3e} per row")
    assert bool((moved > 0).any())
    changed = (kc.codes.view(w.B, w.H_kv, T, -1)[:, :, T - 1] != old_last).any(dim=-1)
    assert bool(changed.all()), "the appended key codes did not replace token T - 1's"


def test_fullsize_stress70b_paged(tq):
    """The benchmark's paged leg at full size: the 70B-like layer quantized into
    caches of 256-token blocks mapped through a seeded permutation of the
    physical blocks equals the contiguous caches byte for byte (read through the
    table), and decode and the one-call step on them equal the contiguous ones
    bit for bit."""
    w = W["stress70b"]
    dev = torch.device("cuda")
    T, bt = w.T, 256
    maxblk = T // bt
    perm = torch.randperm(w.B * maxblk, generator=torch.Generator().manual_seed(5), dtype=torch.int64)
    table = perm.to(torch.int32).reshape(w.B, maxblk).to(dev)
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T, device=dev)
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T, device=dev)
    pk = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T, device=dev, block_table=table, block_tokens=bt,
                  n_blocks=w.B * maxblk)
    pv = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T, device=dev, block_table=table, block_tokens=bt,
                  n_blocks=w.B * maxblk)
    for which, c, p in (("k", kc, pk), ("v", vc, pv)):
        x = tq_synth.torch_kv(w, which, dev)
        tq.quantize_kv(x, c)
        tq.quantize_kv(x, p)
        del x
    torch.cuda.synchronize()
    # physical block table[b, j] holds logical block j of row b, all heads
    tl = table.long()
    for c, p in ((kc, pk), (vc, pv)):
        per_tok = c.codes.shape[-1] // T
        got = p.codes.view(w.B * maxblk, w.H_kv, bt * per_tok)[tl.flatten()]
        got = got.view(w.B, maxblk, w.H_kv, bt * per_tok).permute(0, 2, 1, 3).reshape(c.codes.shape)
        assert torch.equal(got, c.codes)
        gn = p.norms.view(w.B * maxblk, w.H_kv, bt)[tl.flatten()].view(w.B, maxblk, w.H_kv, bt)
        assert torch.equal(gn.permute(0, 2, 1, 3).reshape(c.norms.shape), c.norms)
    q = tq_synth.torch_queries(w, dev)
    assert torch.equal(tq.decode_attention(pk, pv, q, T=T), tq.decode_attention(kc, vc, q, T=T))
    g = torch.Generator(device=dev).manual_seed(6)
    new_k = torch.randn((w.B, 1, w.H_kv, w.d), generator=g, device=dev).to(torch.bfloat16)
    new_v = torch.randn((w.B, 1, w.H_kv, w.d), generator=g, device=dev).to(torch.bfloat16)
    one_p = tq.decode_attention_append(pk, pv, new_k, new_v, q, T=T)
    one_c = tq.decode_attention_append(kc, vc, new_k, new_v, q, T=T)
    torch.cuda.synchronize()
    assert torch.equal(one_p, one_c)
    log("  paged caches at full size (256-token blocks, seeded permutation): bytes, decode and the "
        "one-call step equal the contiguous ones")
