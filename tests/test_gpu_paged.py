"""Paged caches (block table): the same kernels addressing physical blocks
through a table, against the contiguous layout and the oracle.

For each case the workload is quantized into a contiguous cache and into a
paged cache whose logical blocks map to a seeded permutation of physical blocks
(with spare blocks, and table entries past the written tokens left at -1):
  * the paged arrays, gathered back through the table, equal the contiguous
    ones byte for byte (bulk prefill, then single-token appends);
  * their codes (outside the decision-boundary band) and norms match the
    oracle's quantization;
  * decode with ragged context lengths and dequantize give bitwise the
    contiguous results, and decode matches the oracle within 2e-3 relative L2.
"""
import numpy as np
import pytest

import tq_synth
from tqhelp import TOL_ATTN, OracleModel, code_mismatch, device_inputs, device_queries, log, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = tq_synth.WORKLOADS
CASES = {
    "llama8b_T2000": W["llama8b"].scaled(T=2000),    # G = 4, bf16
    "qwen_k4v2": W["qwen"].scaled(B=2, T=1500),      # G = 7, K4/V2
    "qjl_k2v3": W["qjl"].scaled(B=2, T=1024),        # QJL keys
    "tiny": W["tiny"],                               # fp32, G = 16
}
APPEND = 3   # single tokens written after the bulk prefill


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_tq_amd as lib
    return lib


def _table(B, maxblk, used, spare, seed):
    """[B, maxblk] int32: logical blocks < used map to a seeded permutation of
    B * used + spare physical blocks; the others are -1 (never written)."""
    rng = np.random.default_rng(seed)
    nb = B * used + spare
    perm = rng.permutation(nb)[: B * used].reshape(B, used)
    tab = np.full((B, maxblk), -1, dtype=np.int32)
    tab[:, :used] = perm
    return tab, nb


def _gather(arr, tab, used):
    """Paged array [n_blocks, H, per, ...] -> contiguous [B, H, used * per, ...] through the table."""
    B = tab.shape[0]
    x = arr[torch.as_tensor(tab[:, :used].reshape(-1).astype(np.int64), device=arr.device)]
    x = x.reshape(B, used, *arr.shape[1:])
    x = x.transpose(1, 2)
    return x.reshape(B, arr.shape[1], used * arr.shape[2], *arr.shape[3:])


@pytest.mark.parametrize("bt", [32, 256])
@pytest.mark.parametrize("name", list(CASES))
def test_paged_matches_contiguous_and_oracle(tq, name, bt):
    w0 = CASES[name]
    T = w0.T
    w = w0.scaled(T=T + APPEND)
    used = -(-(T + APPEND) // bt)        # blocks holding written tokens
    maxblk = used + 2                   # logical capacity beyond them (entries -1)
    T_cap = maxblk * bt
    log(f"paged {name}: block_tokens={bt}, {used} used + 2 unmapped logical blocks per row")
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    ktab, knb = _table(w.B, maxblk, used, 5, 101)
    vtab, vnb = _table(w.B, maxblk, used, 3, 202)
    dk = torch.as_tensor(ktab, device="cuda")
    dv = torch.as_tensor(vtab, device="cuda")
    caches = {}
    for kind in ("contig", "paged"):
        pk = dict(block_table=dk, block_tokens=bt, n_blocks=knb) if kind == "paged" else {}
        pv = dict(block_table=dv, block_tokens=bt, n_blocks=vnb) if kind == "paged" else {}
        kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, qjl=bool(w.k_qjl), **pk)
        vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, **pv)
        tq.quantize_kv(xk[:, :T], kc)
        tq.quantize_kv(xv[:, :T], vc)
        for t in range(T, T + APPEND):
            tq.quantize_kv(xk[:, t:t + 1].contiguous(), kc, t_offset=t)
            tq.quantize_kv(xv[:, t:t + 1].contiguous(), vc, t_offset=t)
        caches[kind] = (kc, vc)
    torch.cuda.synchronize()
    (kc, vc), (kp, vp) = caches["contig"], caches["paged"]
    n = used * bt
    gathered = {}
    for which, c, p, tab in (("k", kc, kp, ktab), ("v", vc, vp, vtab)):
        W_ = c.codes.shape[2] // T_cap
        g_codes = _gather(p.codes.view(p.codes.shape[0], w.H_kv, bt, W_), tab, used).reshape(w.B, w.H_kv, -1)
        g_norms = _gather(p.norms, tab, used)
        assert torch.equal(g_codes, c.codes[:, :, : n * W_]), which
        assert torch.equal(g_norms, c.norms[:, :, :n]), which
        if which == "k" and w.k_qjl:
            assert torch.equal(_gather(p.signs, tab, used), c.signs[:, :, :n])
            assert torch.equal(_gather(p.gamma, tab, used), c.gamma[:, :, :n])
        gathered[which] = (g_codes.cpu().numpy(), g_norms.cpu().numpy())
    # oracle: codes outside the band and norms of the gathered paged arrays
    model = OracleModel(w)
    for which in ("k", "v"):
        bits = w.k_bits if which == "k" else w.v_bits
        thr = model.tK if which == "k" else model.tV
        codes, norms = gathered[which]
        out = 0
        for (b, h), ref in model.heads(which).items():
            _, mo, _ = code_mismatch(which, codes[b, h], ref, bits, thr, w.T)
            out += mo
            want = ref["norm"].astype(np.float64)
            assert np.all(np.abs(norms[b, h, : w.T] - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)
        assert out == 0, which
    # decode (ragged contexts, automatic and forced splits) and dequantize
    q = device_queries(w)
    ctx = [w.T] + [int(c) for c in np.random.default_rng(7).integers(0, w.T + 1, size=w.B - 1)]
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    for ns in (0, 3):
        oc = tq.decode_attention(kc, vc, q, ctx_lens=cl, T=w.T, n_split=ns)
        op = tq.decode_attention(kp, vp, q, ctx_lens=cl, T=w.T, n_split=ns)
        assert torch.equal(oc, op), ns
    qn = tq_synth.queries_full(w)
    kh, vh = model.heads("k"), model.heads("v")
    out = op.cpu().numpy()
    for b in range(w.B):
        ref = np.concatenate([model.decode(kh, vh, qn, b, kv, ctx=ctx[b]) for kv in range(w.H_kv)])
        if ctx[b] == 0:
            assert np.all(out[b] == 0)
        else:
            assert rel_l2(out[b], ref) <= TOL_ATTN, b
    for c, p in ((kc, kp), (vc, vp)):
        assert torch.equal(tq.dequantize(c, 0, w.T), tq.dequantize(p, 0, w.T))
    log(f"  ctx {ctx}: paged == contiguous, decode within {TOL_ATTN:g} of the oracle")
