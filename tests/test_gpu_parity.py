"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by
element, on seeded workloads scaled so the oracle finishes in seconds while still
spanning many 32-token steps, several context chunks and ragged tails."""
import math

import numpy as np
import pytest

import tq_synth
from tqhelp import (BOUNDARY, TOL_ATTN, TOL_RECUT, U_F16, OracleModel, assert_heads, band_report, code_mismatch,
                    device_inputs, device_queries, gpu_heads, head_errors, log, rel_l2, upload_oracle_cache)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = tq_synth.WORKLOADS
CASES = {
    "tiny": W["tiny"],                                                  # fp32, G = 16
    "llama8b_T2000": W["llama8b"].scaled(T=2000),                       # ragged T, G = 4
    "qwen_k4v2": W["qwen"].scaled(B=2, T=1500),                         # G = 7, K4/V2
    "qwen_k4v4": W["qwen"].scaled(B=2, T=1024, v_bits=4),
    "qjl_k2v3": W["qjl"].scaled(B=2, T=1024),                           # QJL keys
    "stress70b_B2": W["stress70b"].scaled(B=2, T=4096),                 # G = 8
}


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_tq_amd as lib
    return lib


def tcap(T):
    return (T + 7) // 8 * 8


def _lib_caches(tq, w, T_cap):
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, qjl=bool(w.k_qjl))
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap)
    return kc, vc


@pytest.mark.parametrize("name", list(CASES))
def test_quantize_codes_match_oracle(tq, name):
    w = CASES[name]
    T_cap = tcap(w.T)
    log(f"quantize {name}: B={w.B} H_kv={w.H_kv} T={w.T} bits K{w.k_bits}{'+qjl' if w.k_qjl else ''}/V{w.v_bits}")
    model = OracleModel(w)
    kc, vc = _lib_caches(tq, w, T_cap)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    torch.cuda.synchronize()
    for which, cache, bits, thr in (("k", kc, w.k_bits, model.tK), ("v", vc, w.v_bits, model.tV)):
        heads = model.heads(which)
        codes = cache.codes.cpu().numpy()
        norms = cache.norms.cpu().numpy()
        tot = out = n = 0
        for (b, h), ref in heads.items():
            m, mo, c = code_mismatch(which, codes[b, h], ref, bits, thr, w.T)
            tot, out, n = tot + m, out + mo, n + c
            nr = norms[b, h, :w.T].astype(np.float64)
            want = ref["norm"].astype(np.float64)
            assert np.all(np.abs(nr - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)
        log(f"  {which}: {tot}/{n} codes differ ({tot / n:.2e}); outside the {BOUNDARY:g} band: {out}")
        assert out == 0
        if which == "k" and w.k_qjl:
            signs = cache.signs.cpu().numpy().view(np.uint32)
            gamma = cache.gamma.cpu().numpy()
            from oracle import quantize as oq
            bad_total = 0
            for (b, h), ref in heads.items():
                got = oq.unpack_signs(signs[b, h, :w.T], 128)
                flip_vec = np.any(oq.boundary_distance(ref["u"], thr, 128) < BOUNDARY, axis=1)
                bad = (got != ref["signs"]) & ~(np.abs(ref["z"]) < BOUNDARY) & ~flip_vec[:, None]
                bad_total += int(bad.sum())
                g = gamma[b, h, :w.T].astype(np.float64)
                gw = ref["gamma"].astype(np.float64)
                ok = np.abs(g - gw) <= 1e-5 * gw + 1e-7
                assert np.all(ok | flip_vec), (b, h)
            log(f"  qjl signs differing outside the band: {bad_total}")
            assert bad_total == 0


@pytest.mark.parametrize("name", list(CASES))
def test_decode_on_oracle_cache_matches_oracle(tq, name):
    """Decode kernel parity: same packed bytes on both sides."""
    w = CASES[name]
    T_cap = tcap(w.T)
    log(f"decode {name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} T={w.T}")
    model = OracleModel(w)
    kh, vh = model.heads("k"), model.heads("v")
    kc = upload_oracle_cache(tq, model, "k", kh, T_cap)
    vc = upload_oracle_cache(tq, model, "v", vh, T_cap)
    q = device_queries(w)
    out = tq.decode_attention(kc, vc, q, T=w.T).cpu().numpy()
    qn = tq_synth.queries_full(w)
    ref = np.zeros_like(out, dtype=np.float64)
    for b in range(w.B):
        for kv in range(w.H_kv):
            ref[b, kv * w.G:(kv + 1) * w.G] = model.decode(kh, vh, qn, b, kv)
    err = rel_l2(out, ref)
    worst = assert_heads(out, ref, TOL_ATTN, f"decode {name} per (row, head)")
    log(f"  rel L2 {err:.3e} (worst head {worst:.3e})")
    assert err <= TOL_ATTN


@pytest.mark.parametrize("name", list(CASES))
def test_end_to_end_matches_oracle(tq, name):
    """GPU quantize + GPU decode (library rotation and codebook) against the oracle
    quantize + oracle decode of the same inputs."""
    w = CASES[name]
    T_cap = tcap(w.T)
    log(f"end-to-end {name}")
    model = OracleModel(w)
    kc, vc = _lib_caches(tq, w, T_cap)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    out = tq.decode_attention(kc, vc, device_queries(w), T=w.T).cpu().numpy()
    kh, vh = model.heads("k"), model.heads("v")
    gk, gv = gpu_heads(kc, w, "k", w.T), gpu_heads(vc, w, "v", w.T)
    qn = tq_synth.queries_full(w)
    ref = np.zeros_like(out, dtype=np.float64)
    kern = np.zeros_like(out, dtype=np.float64)
    for b in range(w.B):
        for kv in range(w.H_kv):
            ref[b, kv * w.G:(kv + 1) * w.G] = model.decode(kh, vh, qn, b, kv)
            kern[b, kv * w.G:(kv + 1) * w.G] = model.decode(gk, gv, qn, b, kv)
    err = rel_l2(out, ref)
    # kernel parity per (row, head): the oracle decoding the GPU's own codes
    worst_k = assert_heads(out, kern, TOL_ATTN, f"end-to-end {name}, kernel parity per (row, head)")
    e = head_errors(out, ref)
    b, h = np.unravel_index(int(np.nanargmax(e)), e.shape)
    kv = h // w.G
    log(f"  rel L2 {err:.3e}; worst head end to end {e[b, h]:.3e} at (row {b}, head {h}): "
        f"{band_report(w, model, kh, gk, b, kv, 'k')}; {band_report(w, model, vh, gv, b, kv, 'v')}; "
        f"on the GPU's codes that head is at {head_errors(out[b, h], kern[b, h]):.3e} (worst {worst_k:.3e})")
    assert err <= TOL_ATTN


@pytest.mark.parametrize("name", ["tiny", "qwen_k4v2", "qjl_k2v3"])
def test_dequantize_matches_oracle(tq, name):
    from oracle import attention as oa
    w = CASES[name]
    T_cap = tcap(w.T)
    log(f"dequantize {name}")
    model = OracleModel(w)
    for which in ("k", "v"):
        heads = model.heads(which)
        cache = upload_oracle_cache(tq, model, which, heads, T_cap)
        got = tq.dequantize(cache, 0, w.T).cpu().numpy()
        cos = []
        for (b, h), r in heads.items():
            c = model.cK if which == "k" else model.cV
            qj = which == "k" and w.k_qjl
            want = oa.dequantize_head(r["codes"], r["norm"], model.Pi, c, 128,
                                      r.get("signs") if qj else None, r.get("gamma") if qj else None,
                                      model.S if qj else None)
            assert rel_l2(got[b, h], want) <= 1e-5
            cos.append(oa.cosine(tq_synth.kv_head(w, which, b, h), got[b, h]).mean())
        log(f"  {which}: mean cosine {np.mean(cos):.4f}")


def test_dequantize_window(tq):
    w = CASES["llama8b_T2000"]
    model = OracleModel(w)
    heads = model.heads("v")
    cache = upload_oracle_cache(tq, model, "v", heads, tcap(w.T))
    full = tq.dequantize(cache, 0, w.T).cpu().numpy()
    part = tq.dequantize(cache, 37, 1501).cpu().numpy()
    assert np.array_equal(full[:, :, 37:1501], part)


def test_split_invariance_and_determinism(tq):
    w = CASES["stress70b_B2"]
    T_cap = tcap(w.T)
    log("split invariance stress70b_B2")
    kc, vc = _lib_caches(tq, w, T_cap)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    q = device_queries(w)
    base = tq.decode_attention(kc, vc, q, T=w.T)
    again = tq.decode_attention(kc, vc, q, T=w.T)
    assert torch.equal(base, again)
    for ns in (1, 3, 7, 64, 128):
        o = tq.decode_attention(kc, vc, q, T=w.T, n_split=ns)
        assert rel_l2(o.cpu().numpy(), base.cpu().numpy()) <= TOL_RECUT, ns


@pytest.mark.parametrize("d", [128, 64, 256])
def test_merge_batches_at_full_context(tq, d):
    """Context splits that reach every batch size of the chunk merge (one chunk
    per lane up to 4 chunks, 2 up to 8, 4 up to 16, 8 up to 32, and more than
    one batch above 32) on the Llama-8B-like layer at its full 32k context, at
    each head dimension: each within the recut bound of one chunk, repeated bit
    for bit, and the oracle decoding the GPU's own codes per (row, head)."""
    w = W["llama8b"].scaled(d=d)
    T_cap = tcap(w.T)
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, d=d)
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, d=d)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    q = device_queries(w)
    one = tq.decode_attention(kc, vc, q, T=w.T, n_split=1).cpu().numpy()
    gk, gv = gpu_heads(kc, w, "k", w.T), gpu_heads(vc, w, "v", w.T)
    model = OracleModel(w)
    qn = tq_synth.queries_full(w)
    kern = np.zeros_like(one, dtype=np.float64)
    for kv in range(w.H_kv):
        kern[0, kv * w.G:(kv + 1) * w.G] = model.decode(gk, gv, qn, 0, kv)
    assert_heads(one, kern, TOL_ATTN, f"llama8b d={d} one chunk, kernel parity per (row, head)")
    seen = set()
    for ns in (2, 5, 11, 22, 64):
        got = tq.decode_splits(w.B, w.H_kv, w.T, ns)
        assert got == ns, (ns, got)
        o = tq.decode_attention(kc, vc, q, T=w.T, n_split=ns)
        again = tq.decode_attention(kc, vc, q, T=w.T, n_split=ns)
        assert torch.equal(o, again), ns
        o = o.cpu().numpy()
        log(f"llama8b d={d} n_split={ns}: vs one chunk {rel_l2(o, one):.2e}")
        assert rel_l2(o, one) <= TOL_RECUT, ns
        assert_heads(o, kern, TOL_ATTN, f"llama8b d={d} n_split={ns}, kernel parity per (row, head)")
        seen.add(1 if ns <= 4 else 2 if ns <= 8 else 4 if ns <= 16 else 8 if ns <= 32 else 0)
    assert seen == {0, 1, 2, 4, 8}


@pytest.mark.parametrize("bits,cos_lo,cos_hi", [(2, 0.9395, 0.9420), (3, 0.9822, 0.9840), (4, 0.9948, 0.9960)])
def test_value_cosine_per_bit_width(tq, bits, cos_lo, cos_hi):
    """The GPU's quantize then dequantize of 65,536 random unit value vectors
    (float32 input): mean reconstruction cosine inside the same bounds the
    oracle is pinned to (Haar rotation, Gaussian Lloyd-Max codebook, d = 128),
    and at 2 bits the pages' 0.94 within 0.005."""
    B, H, T = 1, 8, 8192
    g = torch.Generator(device="cuda").manual_seed(100 + bits)
    x = torch.randn((B, T, H, 128), generator=g, device="cuda", dtype=torch.float32)
    x = x / x.norm(dim=-1, keepdim=True)
    vc = tq.Cache(tq.VALUES, bits, B, H, T)
    tq.quantize_kv(x, vc)
    xh = tq.dequantize(vc, 0, T)   # [B, H_kv, T, d]
    a = x.permute(0, 2, 1, 3).double()
    cos = ((a * xh.double()).sum(-1) / (a.norm(dim=-1) * xh.double().norm(dim=-1))).mean().item()
    log(f"  value cosine at {bits} bits on the GPU: {cos:.4f}")
    assert cos_lo < cos < cos_hi
    if bits == 2:
        assert abs(cos - 0.94) < 0.005


@pytest.mark.parametrize("bits,qjl,slope,tol", [(2, True, 1.0, 0.02), (2, False, 1 - 0.1175, 0.01),
                                                 (3, False, 1 - 0.03455, 0.006)])
def test_key_score_slope(tq, bits, qjl, slope, tol):
    """Inner products with the GPU's dequantized keys (65,536 random Gaussian
    keys, float32 input, 8 random queries per KV head) regressed on the exact
    ones: with the QJL sign sketch the slope is 1 (the estimate is unbiased);
    MSE-only Lloyd-Max keys shrink it to 1 - MSE of the codebook (the centroid
    condition E[c(z) z] = E[c(z)^2] = 1 - MSE)."""
    B, H, T = 1, 8, 8192
    g = torch.Generator(device="cuda").manual_seed(200 + bits + 10 * qjl)
    k = torch.randn((B, T, H, 128), generator=g, device="cuda", dtype=torch.float32)
    q = torch.randn((H, 8, 128), generator=g, device="cuda", dtype=torch.float64)
    kc = tq.Cache(tq.KEYS, bits, B, H, T, qjl=qjl)
    tq.quantize_kv(k, kc)
    kh = tq.dequantize(kc, 0, T)[0].double()           # [H, T, d]
    kt = k[0].permute(1, 0, 2).double()                 # [H, T, d]
    s = torch.bmm(q, kt.transpose(1, 2).contiguous()).flatten()
    sh = torch.bmm(q, kh.transpose(1, 2).contiguous()).flatten()
    sc = s - s.mean()
    b = ((sh - sh.mean()) * sc).sum().item() / (sc * sc).sum().item()
    log(f"  keys {bits} bits{' + QJL' if qjl else ''}: score slope {b:.4f} (expected {slope:.4f})")
    assert abs(b - slope) < tol


def test_ragged_context_lengths(tq):
    w = CASES["stress70b_B2"].scaled(B=4)
    T_cap = tcap(w.T)
    ctx = [w.T, 1000, 0, 33]
    log(f"ragged contexts {ctx}")
    model = OracleModel(w)
    kh, vh = model.heads("k"), model.heads("v")
    kc = upload_oracle_cache(tq, model, "k", kh, T_cap)
    vc = upload_oracle_cache(tq, model, "v", vh, T_cap)
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    out = tq.decode_attention(kc, vc, device_queries(w), ctx_lens=cl, T=w.T).cpu().numpy()
    qn = tq_synth.queries_full(w)
    for b in range(w.B):
        ref = np.concatenate([model.decode(kh, vh, qn, b, kv, ctx=ctx[b]) for kv in range(w.H_kv)])
        if ctx[b] == 0:
            assert np.all(out[b] == 0)
        else:
            assert rel_l2(out[b], ref) <= TOL_ATTN, b
            assert_heads(out[b], ref, TOL_ATTN, f"ragged row {b} per head")


def _check_against_oracle(tq, w, model, which, cache, T):
    """Codes (outside the boundary band), norms (and QJL bits) of a cache against
    the oracle's quantization of the workload."""
    bits = w.k_bits if which == "k" else w.v_bits
    thr = model.tK if which == "k" else model.tV
    heads = model.heads(which)
    codes = cache.codes.cpu().numpy()
    norms = cache.norms.cpu().numpy()
    out = n = 0
    for (b, h), ref in heads.items():
        _, mo, c = code_mismatch(which, codes[b, h], ref, bits, thr, T)
        out, n = out + mo, n + c
        nr = norms[b, h, :T].astype(np.float64)
        want = ref["norm"].astype(np.float64)
        assert np.all(np.abs(nr - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)
    assert out == 0, (which, out, n)


def test_append_in_pieces_matches_bulk(tq):
    """Writing tokens in pieces (offsets not multiples of 8, single tokens) gives
    the bulk result: the same bytes for multi-token pieces, and for single
    tokens (a separate latency-oriented kernel with float32 rotation) the same
    codes outside the decision-boundary band and the same norms to 1e-6."""
    w = CASES["qjl_k2v3"].scaled(T=300)
    T_cap = tcap(w.T)
    log("append in pieces")
    model = OracleModel(w)
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    kb, vb = _lib_caches(tq, w, T_cap)
    tq.quantize_kv(xk, kb)
    tq.quantize_kv(xv, vb)
    kp, vp = _lib_caches(tq, w, T_cap)
    cuts = [0, 5, 6, 7, 8, 77, 131, 299, 300]
    for a, b in zip(cuts[:-1], cuts[1:]):
        tq.quantize_kv(xk[:, a:b], kp, t_offset=a)
        tq.quantize_kv(xv[:, a:b], vp, t_offset=a)
    torch.cuda.synchronize()
    # QJL keys take the tiled kernel for every piece: identical bytes
    assert torch.equal(kb.codes, kp.codes) and torch.equal(kb.norms, kp.norms)
    assert torch.equal(kb.signs, kp.signs) and torch.equal(kb.gamma, kp.gamma)
    _check_against_oracle(tq, w, model, "v", vp, w.T)
    # tokens written by multi-token pieces are byte-identical to the bulk call
    single = {5, 6, 7, 299}
    multi = [t for t in range(w.T) if t not in single]
    vbn, vpn = vb.norms.cpu().numpy(), vp.norms.cpu().numpy()
    assert np.array_equal(vbn[:, :, multi], vpn[:, :, multi])


@pytest.mark.parametrize("name", ["stress70b_B2", "llama8b_T2000", "tiny", "qwen_k4v2"])
def test_single_token_appends_match_oracle(tq, name):
    """Token-by-token appends (T = 1 at every offset, the decode-step path) of
    keys and values against the oracle."""
    w = CASES[name].scaled(T=43)
    T_cap = tcap(w.T)
    log(f"single-token appends {name}: B={w.B} H_kv={w.H_kv} K{w.k_bits}/V{w.v_bits} {w.dtype}")
    model = OracleModel(w)
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    kc, vc = _lib_caches(tq, w, T_cap)
    for t in range(w.T):
        tq.quantize_kv(xk[:, t:t + 1], kc, t_offset=t)
        tq.quantize_kv(xv[:, t:t + 1], vc, t_offset=t)
    torch.cuda.synchronize()
    _check_against_oracle(tq, w, model, "k", kc, w.T)
    _check_against_oracle(tq, w, model, "v", vc, w.T)


@pytest.mark.parametrize("name", ["stress70b_B2", "qwen_k4v2", "qjl_k2v3", "tiny"])
def test_append_kv_equals_two_quantize_calls(tq, name):
    """tq_append_kv (key and value of one token in one call) writes the same bytes
    as two single-token tq_quantize_kv calls, at every offset of a few value
    blocks (QJL keys take the two-launch path inside the call)."""
    w = CASES[name].scaled(T=21)
    T_cap = tcap(w.T)
    log(f"append_kv {name}: B={w.B} H_kv={w.H_kv} K{w.k_bits}{'+qjl' if w.k_qjl else ''}/V{w.v_bits} {w.dtype}")
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    kc, vc = _lib_caches(tq, w, T_cap)
    kr, vr = _lib_caches(tq, w, T_cap)
    for cache in (kc, vc, kr, vr):
        for name_ in ("codes", "norms", "signs", "gamma"):
            arr = getattr(cache, name_)
            if arr is not None:
                arr.zero_()
    for t in range(w.T):
        tq.append_kv(xk[:, t], xv[:, t], kc, vc, t)
        tq.quantize_kv(xk[:, t:t + 1], kr, t_offset=t)
        tq.quantize_kv(xv[:, t:t + 1], vr, t_offset=t)
    torch.cuda.synchronize()
    for got, want in ((kc, kr), (vc, vr)):
        for name_ in ("codes", "norms", "signs", "gamma"):
            g, r = getattr(got, name_), getattr(want, name_)
            if g is not None:
                assert torch.equal(g.view(torch.int32) if g.dtype == torch.float32 else g,
                                   r.view(torch.int32) if r.dtype == torch.float32 else r), name_


def test_value_block_partial_write_keeps_neighbours(tq):
    """A partial value block keeps the bits of tokens outside the written range."""
    w = CASES["stress70b_B2"].scaled(T=64)
    x = device_inputs(w, "v")
    vc = tq.Cache(tq.VALUES, 3, w.B, w.H_kv, 64)
    vc.codes.fill_(-1)
    tq.quantize_kv(x[:, 10:13], vc, t_offset=10)
    ref = tq.Cache(tq.VALUES, 3, w.B, w.H_kv, 64)
    tq.quantize_kv(x, ref)
    from tqhelp import unpack_head
    got = unpack_head("v", vc.codes[0, 0].cpu().numpy(), 3, 64)
    want = unpack_head("v", ref.codes[0, 0].cpu().numpy(), 3, 64)
    assert np.array_equal(got[10:13], want[10:13])
    assert np.all(got[:10] == 7) and np.all(got[13:] == 7)


def test_degenerate_inputs(tq):
    """Zero vectors (code 2^(b-1), norm 0), a single token, T = 0."""
    w = CASES["stress70b_B2"].scaled(B=1, H_q=8, H_kv=1, T=8)
    kc, vc = _lib_caches(tq, w, 8)
    z = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    tq.quantize_kv(z, kc)
    tq.quantize_kv(z, vc)
    from tqhelp import unpack_head
    assert np.all(unpack_head("k", kc.codes[0, 0].cpu().numpy(), 3, 8) == 4)
    assert np.all(unpack_head("v", vc.codes[0, 0].cpu().numpy(), 3, 8) == 4)
    assert torch.all(kc.norms == 0)
    q = device_queries(w)
    out = tq.decode_attention(kc, vc, q, T=8)
    assert torch.all(out == 0)
    out0 = tq.decode_attention(kc, vc, q, T=0)
    assert torch.all(out0 == 0)
    # single token: output is that token's reconstruction (its weight, the value
    # norm times a power of two, is rounded once to float16)
    x = device_inputs(w, "v")
    tq.quantize_kv(x[:, :1], vc)
    tq.quantize_kv(device_inputs(w, "k")[:, :1], kc)
    o1 = tq.decode_attention(kc, vc, q, T=1).cpu().numpy()
    v0 = tq.dequantize(vc, 0, 1).cpu().numpy()[0, 0, 0]
    assert np.allclose(o1[0], np.repeat(v0[None], 8, axis=0), rtol=U_F16 + 1e-5, atol=1e-6)


@pytest.mark.parametrize("scale", [1e30, 1e-30])
def test_extreme_magnitudes(tq, scale):
    """Inputs near the ends of the bfloat16 range (the per-vector power-of-two
    scaling keeps the rotation and the norm finite and exact to the bar), in
    bulk and single-token calls, against the oracle on the same bytes."""
    w = CASES["stress70b_B2"].scaled(T=24)
    T_cap = tcap(w.T)
    log(f"extreme magnitudes x{scale:g}")
    base = {}
    for which in ("k", "v"):
        x = torch.from_numpy(tq_synth.kv_full(w, which) * np.float32(scale)).to(torch.bfloat16)
        base[which] = x
    # the oracle sees exactly the bfloat16 values the GPU gets
    model = OracleModel(w)
    for mode in ("bulk", "single"):
        kc, vc = _lib_caches(tq, w, T_cap)
        for which, cache in (("k", kc), ("v", vc)):
            xd = base[which].to("cuda")
            if mode == "bulk":
                tq.quantize_kv(xd, cache)
            else:
                for t in range(w.T):
                    tq.quantize_kv(xd[:, t:t + 1], cache, t_offset=t)
        torch.cuda.synchronize()
        for which, cache in (("k", kc), ("v", vc)):
            bits = w.k_bits if which == "k" else w.v_bits
            thr = model.tK if which == "k" else model.tV
            xf = base[which].float().numpy().astype(np.float64)
            codes = cache.codes.cpu().numpy()
            norms = cache.norms.cpu().numpy()
            for b in range(w.B):
                for h in range(w.H_kv):
                    ref = model.quantize(which, xf[b, :, h])
                    _, mo, _ = code_mismatch(which, codes[b, h], ref, bits, thr, w.T)
                    assert mo == 0, (mode, which, b, h)
                    nr = norms[b, h, :w.T].astype(np.float64)
                    assert np.all(np.abs(nr - ref["norm"]) <= 1e-6 * ref["norm"]), (mode, which, b, h)


@pytest.mark.parametrize("name", ["stress70b_B2", "qjl_k2v3", "tiny"])
def test_value_norm_scale(tq, name):
    """Value norms of any overall scale: the output is linear in the value norms,
    and the kernel scales its float16 weights by a power of two taken from the
    norms themselves, so scaling every value norm by 2^k scales the output by
    2^k (up to the re-rounding of the weights: the exponent offset enters the
    float32 softmax argument, so single float16 roundings may flip) even where
    unscaled weights would fall into float16 subnormals or to zero (2^-40) or
    overflow (2^+24); also a scale that is not a power of two; all against the
    oracle per (row, head)."""
    w = CASES[name].scaled(T=min(CASES[name].T, 1024))
    T_cap = tcap(w.T)
    log(f"value-norm scale {name}")
    model = OracleModel(w)
    kh, vh = model.heads("k"), model.heads("v")
    kc = upload_oracle_cache(tq, model, "k", kh, T_cap)
    vc = upload_oracle_cache(tq, model, "v", vh, T_cap)
    q = device_queries(w)
    base = tq.decode_attention(kc, vc, q, T=w.T)
    qn = tq_synth.queries_full(w)
    ref = np.zeros(tuple(base.shape), dtype=np.float64)
    for b in range(w.B):
        for kv in range(w.H_kv):
            ref[b, kv * w.G:(kv + 1) * w.G] = model.decode(kh, vh, qn, b, kv)
    norms0 = vc.norms.clone()
    for s in (2.0 ** -40, 2.0 ** -20, 2.0 ** 24, 3.7e-9):
        vc.norms.copy_(norms0 * s)
        o = tq.decode_attention(kc, vc, q, T=w.T).cpu().numpy() / s
        err = rel_l2(o, base.cpu().numpy())
        log(f"  value norms x{s:.3g}: rel L2 {err:.2e} against the unscaled output")
        assert err <= TOL_RECUT, s
        assert_heads(o, ref, TOL_ATTN, f"value norms x{s:g}, per (row, head)")
    vc.norms.copy_(norms0)
