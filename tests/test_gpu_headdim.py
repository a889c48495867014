"""Head dimensions 64 and 256 against the CPU oracle, through the C ABI: bulk
and piecewise quantize, single-token appends, the fused append + decode step,
dequantize, decode on the oracle's own packed bytes (kernel parity: the scan
tiles at d = 64 and at d = 256 up to 8 heads per KV head, the generic decode
at d = 256 with 16), context splits, chunked prefill, end to end with ragged
contexts, a paged cache, and the degenerate inputs (zero vectors, empty
contexts)."""
import numpy as np
import pytest

import tq_synth
from tqhelp import (BOUNDARY, TOL_ATTN, OracleModel, assert_heads, code_mismatch, device_inputs, device_queries,
                    log, rel_l2, unpack_head, upload_oracle_cache)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = tq_synth.WORKLOADS
CASES = {
    "d64_llama": W["llama8b"].scaled(T=1500, d=64),              # bf16, G = 4, outlier channels
    "d64_stress": W["stress70b"].scaled(B=2, T=1000, d=64),      # bf16, G = 8, outlier tokens
    "d256_qwen": W["qwen"].scaled(B=2, T=700, d=256),            # bf16, G = 7, K4/V2
    "d256_tiny": W["tiny"].scaled(T=500, d=256),                 # float32, G = 16 (generic decode)
    "d64_tiny": W["tiny"].scaled(T=700, d=64),                   # float32, G = 16 (16-column tile)
    # the randomized Hadamard rotation, with the other bit split at each d
    "d64_qwen_hadamard": W["qwen"].scaled(B=2, T=600, d=64),     # K4/V2
    "d256_stress_hadamard": W["stress70b"].scaled(B=2, T=500, d=256),   # K3/V3
}
# Decode on identical packed bytes. The generic kernel (d = 256, G > 8) works in
# float32 throughout, so it stays within a few float32 roundings per token of
# the float64 oracle; the scan tiles round each softmax weight to float16
# (TOL_ATTN, as at d = 128).
TOL_GENERIC = 1e-4


def kernel_tol(w):
    return TOL_GENERIC if w.d > 128 and w.G > 8 else TOL_ATTN


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_tq_amd as lib
    return lib


def tcap(T):
    return (T + 7) // 8 * 8


def _rotation(name):
    return "hadamard" if name.endswith("_hadamard") else "haar"


def _model(name, w=None):
    return OracleModel(CASES[name] if w is None else w, rotation=_rotation(name))


def _caches(tq, w, T_cap, rotation="haar", **kw):
    rot = tq.make_rotation(tq_synth.ROT_SEED, tq.HADAMARD if rotation == "hadamard" else tq.HAAR, w.d)
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, d=w.d, rot=rot, **kw.get("k", {}))
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, d=w.d, rot=rot, **kw.get("v", {}))
    return kc, vc


def _check_codes(w, model, which, cache, T, heads=None):
    bits = w.k_bits if which == "k" else w.v_bits
    thr = model.tK if which == "k" else model.tV
    heads = model.heads(which) if heads is None else heads
    codes = cache.codes.cpu().numpy()
    norms = cache.norms.cpu().numpy()
    tot = out = n = 0
    for (b, h), ref in heads.items():
        m, mo, c = code_mismatch(which, codes[b, h], ref, bits, thr, T)
        tot, out, n = tot + m, out + mo, n + c
        nr = norms[b, h, :T].astype(np.float64)
        want = ref["norm"][:T].astype(np.float64)
        assert np.all(np.abs(nr - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)
    log(f"  {which}: {tot}/{n} codes differ; outside the {BOUNDARY:g} band: {out}")
    assert out == 0


def _oracle_decode(w, model, kh, vh, ctx=None):
    qn = tq_synth.queries_full(w)
    ref = np.zeros((w.B, w.H_q, w.d))
    for b in range(w.B):
        for kv in range(w.H_kv):
            c = None if ctx is None else ctx[b]
            ref[b, kv * w.G:(kv + 1) * w.G] = model.decode(kh, vh, qn, b, kv, ctx=c)
    return ref


@pytest.mark.parametrize("name", list(CASES))
def test_quantize_matches_oracle(tq, name):
    w = CASES[name]
    log(f"quantize {name}: d={w.d} B={w.B} H_kv={w.H_kv} T={w.T} K{w.k_bits}/V{w.v_bits} {w.dtype}")
    model = _model(name)
    kc, vc = _caches(tq, w, tcap(w.T), _rotation(name))
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    torch.cuda.synchronize()
    _check_codes(w, model, "k", kc, w.T)
    _check_codes(w, model, "v", vc, w.T)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_on_oracle_cache_matches_oracle(tq, name):
    """Kernel parity: the oracle's packed bytes decoded on both sides."""
    w = CASES[name]
    log(f"decode {name}: d={w.d} H_q={w.H_q} H_kv={w.H_kv} T={w.T}")
    model = _model(name)
    kh, vh = model.heads("k"), model.heads("v")
    kc = upload_oracle_cache(tq, model, "k", kh, tcap(w.T))
    vc = upload_oracle_cache(tq, model, "v", vh, tcap(w.T))
    out = tq.decode_attention(kc, vc, device_queries(w), T=w.T).cpu().numpy()
    ref = _oracle_decode(w, model, kh, vh)
    worst = assert_heads(out, ref, kernel_tol(w), f"decode {name} per (row, head)")
    log(f"  rel L2 {rel_l2(out, ref):.3e} (worst head {worst:.3e})")


@pytest.mark.parametrize("name", ["d64_stress", "d256_qwen", "d64_qwen_hadamard", "d256_stress_hadamard"])
def test_end_to_end_ragged(tq, name):
    """GPU quantize + GPU decode with ragged context lengths (full, partial,
    empty, one token) against the oracle's quantize + decode."""
    w = CASES[name].scaled(B=4)
    ctx = [w.T, 333, 0, 1]
    log(f"end-to-end {name}: contexts {ctx}")
    model = _model(name, w)
    kc, vc = _caches(tq, w, tcap(w.T), _rotation(name))
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    out = tq.decode_attention(kc, vc, device_queries(w), ctx_lens=cl, T=w.T).cpu().numpy()
    ref = _oracle_decode(w, model, model.heads("k"), model.heads("v"), ctx=ctx)
    assert np.all(out[2] == 0)
    worst = assert_heads(out, ref, TOL_ATTN, f"end-to-end {name} per (row, head)")
    log(f"  worst head rel L2 {worst:.3e}")


@pytest.mark.parametrize("name", ["d64_llama", "d256_tiny", "d256_stress_hadamard"])
def test_dequantize_matches_oracle(tq, name):
    from oracle import attention as oa
    w = CASES[name]
    log(f"dequantize {name}")
    model = _model(name)
    for which in ("k", "v"):
        heads = model.heads(which)
        cache = upload_oracle_cache(tq, model, which, heads, tcap(w.T))
        got = tq.dequantize(cache, 0, w.T).cpu().numpy()
        part = tq.dequantize(cache, 37, w.T - 5).cpu().numpy()
        assert np.array_equal(got[:, :, 37:w.T - 5], part)
        c = model.cK if which == "k" else model.cV
        for (b, h), r in heads.items():
            want = oa.dequantize_head(r["codes"], r["norm"], model.Pi, c, w.d)
            assert rel_l2(got[b, h], want) <= 1e-5, (which, b, h)


@pytest.mark.parametrize("name", ["d64_stress", "d256_qwen"])
def test_pieces_and_appends_match_bulk(tq, name):
    """Quantizing in pieces (offsets off the 8-token value blocks) gives the
    bulk call's bytes for every token a multi-token piece wrote (each token's
    codes and norm depend on that token alone; partial value blocks keep the
    bits of the tokens outside the piece); single tokens (tq_append_kv, the
    one-token kernel with float32 rotation) hold the oracle's codes outside the
    decision-boundary band and its norms to 1e-6."""
    w = CASES[name].scaled(T=83)
    T_cap = tcap(w.T)
    log(f"pieces {name}: d={w.d}")
    model = _model(name, w)
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    kb, vb = _caches(tq, w, T_cap)
    tq.quantize_kv(xk, kb)
    tq.quantize_kv(xv, vb)
    kp, vp = _caches(tq, w, T_cap)
    vp.codes.fill_(-1)
    cuts = [0, 5, 6, 7, 8, 29, 64, 71, 82, 83]
    single = set()
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b - a == 1:
            tq.append_kv(xk[:, a], xv[:, a], kp, vp, a)
            single.add(a)
        else:
            tq.quantize_kv(xk[:, a:b], kp, t_offset=a)
            tq.quantize_kv(xv[:, a:b], vp, t_offset=a)
    torch.cuda.synchronize()
    multi = [t for t in range(w.T) if t not in single]
    for got_c, want_c, which, bits in ((kp, kb, "k", w.k_bits), (vp, vb, "v", w.v_bits)):
        assert torch.equal(got_c.norms[:, :, multi], want_c.norms[:, :, multi]), which
        for b in range(w.B):
            for h in range(w.H_kv):
                got = unpack_head(which, got_c.codes[b, h].cpu().numpy(), bits, T_cap, w.d)
                want = unpack_head(which, want_c.codes[b, h].cpu().numpy(), bits, T_cap, w.d)
                assert np.array_equal(got[multi], want[multi]), (which, b, h)
                if which == "v":
                    # tokens 83 .. 87 of the last block were never written (bits kept = all ones)
                    assert np.all(got[w.T:] == (1 << bits) - 1)
    _check_codes(w, model, "k", kp, w.T)
    _check_codes(w, model, "v", vp, w.T)


@pytest.mark.parametrize("name", ["d64_llama", "d256_qwen", "d64_qwen_hadamard", "d256_tiny"])
def test_fused_append_decode_step(tq, name):
    """decode_attention_append: the new token of each row goes to
    ctx_len[b] - 1, then decode over tokens 0 .. ctx_len[b] - 1; the caches then
    hold the oracle's codes and the output matches the oracle's decode."""
    w = CASES[name].scaled(B=3, T=300)
    ctx = [300, 129, 1]
    T_cap = tcap(w.T)
    log(f"fused append + decode {name}: contexts {ctx}")
    model = _model(name, w)
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    kc, vc = _caches(tq, w, T_cap, _rotation(name))
    for b, c in enumerate(ctx):   # rows hold their first c - 1 tokens
        if c > 1:
            tq.quantize_kv(xk[b:b + 1, :c - 1].contiguous(), _row(tq, kc, b), t_offset=0)
            tq.quantize_kv(xv[b:b + 1, :c - 1].contiguous(), _row(tq, vc, b), t_offset=0)
    idx = torch.tensor([c - 1 for c in ctx], device="cuda")
    kn = xk[torch.arange(w.B, device="cuda"), idx].contiguous()
    vn = xv[torch.arange(w.B, device="cuda"), idx].contiguous()
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    out = tq.decode_attention_append(kc, vc, kn, vn, device_queries(w), ctx_lens=cl, T=w.T).cpu().numpy()
    kh, vh = model.heads("k"), model.heads("v")
    codes_k, codes_v = kc.codes.cpu().numpy(), vc.codes.cpu().numpy()
    for b, c in enumerate(ctx):
        for h in range(w.H_kv):
            for which, codes, heads, bits, thr in (("k", codes_k, kh, w.k_bits, model.tK),
                                                   ("v", codes_v, vh, w.v_bits, model.tV)):
                _, mo, _ = code_mismatch(which, codes[b, h], heads[(b, h)], bits, thr, c)
                assert mo == 0, (which, b, h)
    ref = _oracle_decode(w, model, kh, vh, ctx=ctx)
    worst = assert_heads(out, ref, TOL_ATTN, f"fused step {name} per (row, head)")
    log(f"  worst head rel L2 {worst:.3e}")


def _row(tq, cache, b):
    """A one-row view of a contiguous cache (row b's arrays, same rotation and codebook)."""
    r = tq.Cache.__new__(tq.Cache)
    r.__dict__.update(cache.__dict__)
    r.B = 1
    r.codes = cache.codes[b:b + 1]
    r.norms = cache.norms[b:b + 1]
    return r


def test_paged_matches_contiguous(tq):
    """A paged d = 64 cache (seeded permutation of physical blocks, spare
    blocks, unmapped logical blocks) holds the contiguous cache's bytes and
    decodes to its output bit for bit."""
    w = CASES["d64_stress"]
    bt, used = 32, -(-w.T // 32)
    maxblk = used + 2
    T_cap = maxblk * bt
    log(f"paged d=64: block_tokens={bt}")
    rng = np.random.default_rng(5)
    tabs = {}
    for which, spare in (("k", 5), ("v", 3)):
        nb = w.B * used + spare
        tab = np.full((w.B, maxblk), -1, dtype=np.int32)
        tab[:, :used] = rng.permutation(nb)[: w.B * used].reshape(w.B, used)
        tabs[which] = (tab, nb)
    kw = {x: dict(block_table=torch.as_tensor(tabs[x][0], device="cuda"), block_tokens=bt, n_blocks=tabs[x][1])
          for x in ("k", "v")}
    kp, vp = _caches(tq, w, T_cap, **kw)
    kc, vc = _caches(tq, w, T_cap)
    for cache_k, cache_v in ((kp, vp), (kc, vc)):
        tq.quantize_kv(device_inputs(w, "k"), cache_k)
        tq.quantize_kv(device_inputs(w, "v"), cache_v)
    for which, pc, cc in (("k", kp, kc), ("v", vp, vc)):
        tab = tabs[which][0]
        g = pc.codes[torch.as_tensor(tab[:, :used].reshape(-1).astype(np.int64), device="cuda")]
        g = g.reshape(w.B, used, w.H_kv, -1).transpose(1, 2).reshape(w.B, w.H_kv, -1)
        assert torch.equal(g, cc.codes[:, :, :g.shape[-1]]), which
    cl = torch.tensor([w.T, 517], dtype=torch.int32, device="cuda")
    q = device_queries(w)
    a = tq.decode_attention(kp, vp, q, ctx_lens=cl, T=w.T)
    b = tq.decode_attention(kc, vc, q, ctx_lens=cl, T=w.T)
    assert torch.equal(a, b)
    assert torch.equal(tq.dequantize(vp, 0, w.T), tq.dequantize(vc, 0, w.T))


@pytest.mark.parametrize("d", [64, 256])
def test_degenerate_inputs(tq, d):
    """Zero vectors: code 2^(bits-1) (the cell just above 0) and norm 0; T = 0
    writes nothing; an empty context decodes to zeros."""
    kc = tq.Cache(tq.KEYS, 4, 1, 2, 16, d=d)
    vc = tq.Cache(tq.VALUES, 2, 1, 2, 16, d=d)
    z = torch.zeros((1, 16, 2, d), dtype=torch.bfloat16, device="cuda")
    tq.quantize_kv(z, kc)
    tq.quantize_kv(z, vc)
    tq.quantize_kv(z[:, :0], kc, t_offset=3)
    assert np.all(unpack_head("k", kc.codes[0, 1].cpu().numpy(), 4, 16, d) == 8)
    assert np.all(unpack_head("v", vc.codes[0, 1].cpu().numpy(), 2, 16, d) == 2)
    assert torch.all(kc.norms == 0) and torch.all(vc.norms == 0)
    q = torch.randn((1, 4, d), device="cuda")
    out = tq.decode_attention(kc, vc, q, ctx_lens=torch.zeros(1, dtype=torch.int32, device="cuda"), T=16)
    assert torch.all(out == 0)
    # zero keys: uniform weights over zero values -> zeros; finite everywhere
    out = tq.decode_attention(kc, vc, q, T=16)
    assert torch.all(torch.isfinite(out)) and torch.all(out == 0)


@pytest.mark.parametrize("name", ["d64_stress", "d256_stress_hadamard", "d64_tiny"])
def test_split_plans_match_one_pass(tq, name):
    """Context splits (chunk partials merged by the merge kernel) give the
    one-chunk result within the float16-weight recut bound, and repeat bit for
    bit; both match the oracle."""
    from tqhelp import TOL_RECUT
    w = CASES[name]
    model = _model(name)
    kh, vh = model.heads("k"), model.heads("v")
    kc = upload_oracle_cache(tq, model, "k", kh, tcap(w.T))
    vc = upload_oracle_cache(tq, model, "v", vh, tcap(w.T))
    q = device_queries(w)
    one = tq.decode_attention(kc, vc, q, T=w.T, n_split=1).cpu().numpy()
    ref = _oracle_decode(w, model, kh, vh)
    assert_heads(one, ref, TOL_ATTN, f"{name} one chunk")
    for ns in (2, 5, 16):
        o = tq.decode_attention(kc, vc, q, T=w.T, n_split=ns)
        again = tq.decode_attention(kc, vc, q, T=w.T, n_split=ns)
        assert torch.equal(o, again)
        log(f"{name} n_split={ns}: vs one chunk {rel_l2(o.cpu().numpy(), one):.2e}")
        assert rel_l2(o.cpu().numpy(), one) <= TOL_RECUT
        assert_heads(o.cpu().numpy(), ref, TOL_ATTN, f"{name} n_split={ns}")


@pytest.mark.parametrize("name,M", [("d64_stress", 5), ("d64_llama", 3), ("d256_qwen", 1), ("d256_stress_hadamard", 1)])
def test_prefill_matches_oracle(tq, name, M):
    """Chunked causal attention of the M newest tokens (the scan tiles with
    (token, head) columns) against the oracle's causal definition; M = 1 equals
    the decode bit for bit."""
    from oracle import attention as oa
    w = CASES[name].scaled(B=2)
    ctx = [w.T, 300]
    model = _model(name, w)
    kh, vh = model.heads("k"), model.heads("v")
    kc = upload_oracle_cache(tq, model, "k", kh, tcap(w.T))
    vc = upload_oracle_cache(tq, model, "v", vh, tcap(w.T))
    g = torch.Generator(device="cuda").manual_seed(M)
    q = torch.randn((w.B, M, w.H_q, w.d), generator=g, device="cuda").to(torch.bfloat16)
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    out = tq.prefill_attention(kc, vc, q, ctx_lens=cl, T=w.T).cpu().numpy()
    qn = q.float().cpu().numpy().astype(np.float64)
    ref = np.zeros_like(out, dtype=np.float64)
    for b in range(w.B):
        for kv in range(w.H_kv):
            qs = qn[b, :, kv * w.G:(kv + 1) * w.G]
            ref[b, :, kv * w.G:(kv + 1) * w.G] = oa.attend_chunk_causal(
                qs, kh[(b, kv)], vh[(b, kv)], model.Pi, model.Pi, model.cK, model.cV, w.d, 1.0 / np.sqrt(w.d), ctx[b])
    worst = assert_heads(out, ref, TOL_ATTN, f"prefill {name} M={M} per (row, token, head)")
    log(f"prefill {name} M={M}: worst {worst:.3e}")
    if M == 1:
        dec = tq.decode_attention(kc, vc, q[:, 0].contiguous(), ctx_lens=cl, T=w.T).cpu().numpy()
        assert np.array_equal(dec, out[:, 0])


@pytest.mark.parametrize("name", ["d64_stress", "d256_qwen", "d256_tiny"])
def test_noalloc_equals_workspace_call(tq, name):
    """tq_decode_attention_noalloc (partials in the library's static scratch)
    gives tq_decode_attention's output bit for bit at d = 64 and 256, with
    context splits and ragged contexts, twice in a row."""
    w = CASES[name]
    model = _model(name)
    kc = upload_oracle_cache(tq, model, "k", model.heads("k"), tcap(w.T))
    vc = upload_oracle_cache(tq, model, "v", model.heads("v"), tcap(w.T))
    q = device_queries(w)
    cl = torch.tensor([max(w.T - 37 * b, 1) for b in range(w.B)], dtype=torch.int32, device="cuda")
    for ns in (0, 3):
        want = tq.decode_attention(kc, vc, q, ctx_lens=cl, T=w.T, n_split=ns)
        for _ in range(2):
            got = tq.decode_attention_noalloc(kc, vc, q, ctx_lens=cl, T=w.T, n_split=ns)
            assert torch.equal(got, want), (name, ns)
