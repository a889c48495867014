"""Chunked causal (prefill) attention over the packed caches against the oracle.

The caches hold every token of the context (the M query tokens already
appended); token i of row b attends to cache tokens 0 .. ctx_b - M + i. For
each case: the whole output tensor within 2e-3 relative L2 of the oracle on the
GPU's own codes (kernel parity) and on the oracle's codes (end to end), with
ragged context lengths (including rows shorter than M, whose first queries see
nothing and give zeros); M = 1 equals decode bit for bit; a forced context
split agrees with the automatic plan.
"""
import numpy as np
import pytest

import tq_synth
from tqhelp import TOL_ATTN, TOL_RECUT, OracleModel, assert_heads, device_inputs, log, rel_l2, unpack_head

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = tq_synth.WORKLOADS
CASES = {
    "stress70b_M2": (W["stress70b"].scaled(B=2, T=2048), 2),      # G = 8: 16 columns (8-wave tile)
    "stress70b_M37": (W["stress70b"].scaled(B=2, T=2048), 37),    # many tiles, ragged last tile
    "llama8b_M3": (W["llama8b"].scaled(T=1500), 3),               # G = 4: 12 columns
    "llama8b_M2": (W["llama8b"].scaled(T=1500), 2),               # G = 4: 8 columns, 16-wave tile
    "qwen_M5": (W["qwen"].scaled(B=2, T=1200), 5),                # G = 7, K4/V2
    "qjl_M9": (W["qjl"].scaled(B=2, T=1024), 9),                  # QJL keys
    "tiny_M3": (W["tiny"], 3),                                    # fp32, G = 16 (dense: 48 columns)
    # the dense kernel (32 (token, head) columns per wavefront, one cache read per chunk)
    "stress70b_M16": (W["stress70b"].scaled(B=2, T=2048), 16),    # 128 columns: one 4-wavefront group
    "llama8b_M16": (W["llama8b"].scaled(B=2, T=1500), 16),        # G = 4: 64 columns, ragged T
    "stress70b_M100": (W["stress70b"].scaled(B=1, T=1200), 100),  # 800 columns: 7 groups, last one partial
    "qwen_M9_k4v2": (W["qwen"].scaled(B=2, T=1000), 9),           # G = 7, K4/V2, large key norms
}


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_tq_amd as lib
    return lib


def _queries(w, M, seed=99):
    q = np.random.default_rng(seed).standard_normal((w.B, M, w.H_q, 128))
    if w.dtype == "bf16":
        t = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16)
        return t.cuda(), t.float().numpy().astype(np.float64)
    t = torch.from_numpy(q.astype(np.float32))
    return t.cuda(), t.numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(tq, name):
    from oracle import attention as oa
    from oracle import quantize as oq
    w, M = CASES[name]
    T_cap = (w.T + 7) // 8 * 8
    ctx = [w.T] + [int(c) for c in np.random.default_rng(3).integers(1, w.T + 1, size=w.B - 1)]
    if w.B > 1:
        ctx[1] = min(ctx[1], max(M // 2, 1))     # a row shorter than the chunk
    log(f"prefill {name}: M={M}, G={w.G}, ctx {ctx}")
    model = OracleModel(w)
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, qjl=bool(w.k_qjl))
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    q, qn = _queries(w, M)
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    out = tq.prefill_attention(kc, vc, q, ctx_lens=cl, T=w.T)
    out4 = tq.prefill_attention(kc, vc, q, ctx_lens=cl, T=w.T, n_split=4)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    assert rel_l2(out4.cpu().numpy(), out.cpu().numpy()) <= TOL_RECUT
    got = out.cpu().numpy()
    kh, vh = model.heads("k"), model.heads("v")
    codes_k, norms_k = kc.codes.cpu().numpy(), kc.norms.cpu().numpy()
    codes_v, norms_v = vc.codes.cpu().numpy(), vc.norms.cpu().numpy()
    ref_e2e = np.zeros_like(got, dtype=np.float64)
    ref_kern = np.zeros_like(got, dtype=np.float64)
    sc = 1 / np.sqrt(128)
    for b in range(w.B):
        for kv in range(w.H_kv):
            gk = {"codes": unpack_head("k", codes_k[b, kv], w.k_bits, w.T),
                  "norm": norms_k[b, kv, : w.T].astype(np.float64)}
            if w.k_qjl:
                gk["signs"] = oq.unpack_signs(kc.signs[b, kv, : w.T].cpu().numpy().view(np.uint32), 128)
                gk["gamma"] = kc.gamma[b, kv, : w.T].cpu().numpy().astype(np.float64)
            gv = {"codes": unpack_head("v", codes_v[b, kv], w.v_bits, w.T),
                  "norm": norms_v[b, kv, : w.T].astype(np.float64)}
            qs = qn[b, :, kv * w.G:(kv + 1) * w.G]
            hs = slice(kv * w.G, (kv + 1) * w.G)
            ref_e2e[b, :, hs] = oa.attend_chunk_causal(qs, kh[(b, kv)], vh[(b, kv)], model.Pi, model.Pi, model.cK,
                                                       model.cV, 128, sc, ctx[b], S=model.S)
            ref_kern[b, :, hs] = oa.attend_chunk_causal(qs, gk, gv, model.Pi, model.Pi, model.cK, model.cV, 128, sc,
                                                        ctx[b], S=model.S)
    kern, e2e = rel_l2(got, ref_kern), rel_l2(got, ref_e2e)
    worst = assert_heads(got, ref_kern, TOL_ATTN, f"prefill {name}, kernel parity per (row, token, head)")
    log(f"  rel L2 over the output: kernel parity {kern:.2e} (worst (row, token, head) {worst:.2e}), "
        f"end to end {e2e:.2e}")
    assert kern <= TOL_ATTN and e2e <= TOL_ATTN
    for b in range(w.B):
        for i in range(M):
            if ctx[b] - M + i + 1 <= 0:
                assert np.all(got[b, i] == 0), (b, i)
    if M > 1:
        # the last token of the chunk is a decode over the whole context
        d = tq.decode_attention(kc, vc, q[:, -1].contiguous(), ctx_lens=cl, T=w.T)
        assert rel_l2(out[:, -1].cpu().numpy(), d.cpu().numpy()) <= TOL_RECUT


@pytest.mark.parametrize("name", ["stress70b_M16", "llama8b_M16"])
def test_prefill_dense_paged_equals_contiguous(tq, name):
    """The dense kernel on paged caches (32-token blocks through a seeded
    permutation) gives the contiguous result bit for bit."""
    w, M = CASES[name]
    T_cap = (w.T + 31) // 32 * 32
    bt, maxblk = 32, T_cap // 32
    perm = torch.randperm(w.B * maxblk, generator=torch.Generator().manual_seed(8), dtype=torch.int64)
    table = perm.to(torch.int32).reshape(w.B, maxblk).cuda()
    log(f"dense prefill paged {name}: M={M}")
    out = []
    for paged in (False, True):
        kw = dict(block_table=table, block_tokens=bt, n_blocks=w.B * maxblk) if paged else {}
        kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, **kw)
        vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, **kw)
        tq.quantize_kv(device_inputs(w, "k"), kc)
        tq.quantize_kv(device_inputs(w, "v"), vc)
        q, _ = _queries(w, M)
        cl = torch.tensor([w.T] + [max(w.T - 333 * b, M // 2) for b in range(1, w.B)], dtype=torch.int32,
                          device="cuda")
        out.append(tq.prefill_attention(kc, vc, q, ctx_lens=cl, T=w.T))
    torch.cuda.synchronize()
    assert torch.equal(out[0], out[1])


def test_prefill_single_token_is_decode(tq):
    w = W["stress70b"].scaled(B=2, T=1000)
    T_cap = (w.T + 7) // 8 * 8
    kc = tq.Cache(tq.KEYS, 3, w.B, w.H_kv, T_cap)
    vc = tq.Cache(tq.VALUES, 3, w.B, w.H_kv, T_cap)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    q, _ = _queries(w, 1)
    a = tq.prefill_attention(kc, vc, q, T=w.T)
    d = tq.decode_attention(kc, vc, q[:, 0].contiguous(), T=w.T)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], d)
