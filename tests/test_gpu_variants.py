"""Format variants through the same kernels: the sphere-exact Lloyd-Max
codebook and the randomized Hadamard rotation (host-generated, passed in the
cache like the defaults), against the oracle built with the same variant:
codes outside the decision-boundary band and norms bit-exact / 1e-6, decode
within 2e-3 relative L2 over the output tensor on the GPU's own codes and end to
end (the worst head is reported: with QJL keys one boundary code also changes
that token's residual signs, so single heads can move more)."""
import numpy as np
import pytest

import tq_synth
from tqhelp import (TOL_ATTN, OracleModel, assert_heads, band_report, code_mismatch, device_inputs, device_queries,
                    head_errors, log, rel_l2, shifted_codebook, unpack_head)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = tq_synth.WORKLOADS


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_tq_amd as lib
    return lib


@pytest.mark.parametrize("codebook,rotation",
                         [("sphere", "haar"), ("gaussian", "hadamard"), ("sphere", "hadamard"), ("shifted", "haar")])
@pytest.mark.parametrize("name", ["stress70b_B2", "qwen_k4v2", "qjl_k2v3"])
def test_variant_matches_oracle(tq, name, codebook, rotation):
    w = {"stress70b_B2": W["stress70b"].scaled(B=2, T=2048),
         "qwen_k4v2": W["qwen"].scaled(B=2, T=1500),
         "qjl_k2v3": W["qjl"].scaled(B=2, T=1024)}[name]
    log(f"variant {name}: {codebook} codebook, {rotation} rotation")
    model = OracleModel(w, codebook=codebook, rotation=rotation)
    rot = tq.make_rotation(tq_synth.ROT_SEED, tq.HADAMARD if rotation == "hadamard" else tq.HAAR)
    mk = {"sphere": tq.make_codebook_sphere, "gaussian": tq.make_codebook, "shifted": shifted_codebook}[codebook]
    T_cap = (w.T + 7) // 8 * 8
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, rot=rot, qjl=bool(w.k_qjl), centroids=mk(w.k_bits)[0])
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, rot=rot, centroids=mk(w.v_bits)[0])
    assert np.array_equal(kc.centroids.astype(np.float64), model.cK)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    out = tq.decode_attention(kc, vc, device_queries(w), T=w.T).cpu().numpy()
    qn = tq_synth.queries_full(w)
    got = {}
    for which, c in (("k", kc), ("v", vc)):
        bits = w.k_bits if which == "k" else w.v_bits
        thr = model.tK if which == "k" else model.tV
        codes, norms = c.codes.cpu().numpy(), c.norms.cpu().numpy()
        heads = model.heads(which)
        bad = 0
        gh = {}
        for (b, h), ref in heads.items():
            _, mo, _ = code_mismatch(which, codes[b, h], ref, bits, thr, w.T)
            bad += mo
            g = unpack_head(which, codes[b, h], bits, w.T)
            want = ref["norm"].astype(np.float64)
            assert np.all(np.abs(norms[b, h, : w.T] - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)
            gh[(b, h)] = dict(ref, codes=g, norm=norms[b, h, : w.T].astype(np.float64))
        assert bad == 0, which
        got[which] = (heads, gh)
    if w.k_qjl:
        # the QJL parts of the GPU cache (signs, gamma) come from its own bits
        from oracle import quantize as oq
        signs = kc.signs.cpu().numpy()
        gam = kc.gamma.cpu().numpy()
        for (b, h), d in got["k"][1].items():
            d["signs"] = oq.unpack_signs(signs[b, h, : w.T].view(np.uint32), 128)
            d["gamma"] = gam[b, h, : w.T].astype(np.float64)
    ref_e2e = np.zeros_like(out, dtype=np.float64)
    ref_kern = np.zeros_like(out, dtype=np.float64)
    for b in range(w.B):
        for kv in range(w.H_kv):
            ref_e2e[b, kv * w.G:(kv + 1) * w.G] = model.decode(got["k"][0], got["v"][0], qn, b, kv)
            ref_kern[b, kv * w.G:(kv + 1) * w.G] = model.decode(got["k"][1], got["v"][1], qn, b, kv)
    kern, e2e = rel_l2(out, ref_kern), rel_l2(out, ref_e2e)
    worst_k = assert_heads(out, ref_kern, TOL_ATTN, f"variant {name} {codebook}/{rotation}, kernel parity per (row, head)")
    e = head_errors(out, ref_e2e)
    b, h = np.unravel_index(int(np.nanargmax(e)), e.shape)
    kv = h // w.G
    log(f"  decode rel L2 over the output: kernel parity {kern:.2e} (worst head {worst_k:.2e}), end to end {e2e:.2e} "
        f"(worst head {e[b, h]:.2e} at row {b}, head {h}: {band_report(w, model, got['k'][0], got['k'][1], b, kv, 'k')}; "
        f"{band_report(w, model, got['v'][0], got['v'][1], b, kv, 'v')}; on the GPU's codes "
        f"{head_errors(out[b, h], ref_kern[b, h]):.2e})")
    assert kern <= TOL_ATTN and e2e <= TOL_ATTN


def test_shifted_codebook_bulk_kernel(tq):
    """A codebook that does not mirror around 0 through the bulk (32-vector tile)
    quantize kernel: 524,288 slots per cache, so every compute unit gets tiles.
    Codes of sampled heads match the oracle outside the decision-boundary band,
    norms to 1e-6."""
    w = W["stress70b"].scaled(B=32, T=2048)
    log("shifted codebook, bulk quantize: B=32 T=2048 H_kv=8, K3/V3")
    model = OracleModel(w, codebook="shifted")
    for which, bits, role in (("k", w.k_bits, tq.KEYS), ("v", w.v_bits, tq.VALUES)):
        c = tq.Cache(role, bits, w.B, w.H_kv, w.T, centroids=shifted_codebook(bits)[0])
        tq.quantize_kv(device_inputs(w, which), c)
        codes, norms = c.codes.cpu().numpy(), c.norms.cpu().numpy()
        thr = model.tK if which == "k" else model.tV
        for (b, h), ref in model.heads(which, bs=[0, 13, 31], hs=[0, 7]).items():
            _, mo, _ = code_mismatch(which, codes[b, h], ref, bits, thr, w.T)
            assert mo == 0, (which, b, h)
            want = ref["norm"].astype(np.float64)
            assert np.all(np.abs(norms[b, h, : w.T] - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)
