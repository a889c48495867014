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
from oracle import quantize as oq
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


@pytest.mark.parametrize("codebook,rotation", [("shifted", "haar"), ("gaussian", "hadamard"), ("shifted", "hadamard")])
@pytest.mark.parametrize("name", ["stress70b", "qwen"])
def test_bulk_kernel_variants(tq, name, codebook, rotation):
    """The bulk (32-vector tile) quantize kernel with a codebook that does not
    mirror around 0 (the general cell search) and with the randomized Hadamard
    rotation, whose entries all have one magnitude, so the kernel rotates by its
    sign matrix in one bfloat16 MFMA pass: 524,288 slots per cache (every compute
    unit gets tiles), K3/V3 and K4/V2. Codes of sampled heads match the oracle
    outside the decision-boundary band, norms to 1e-6."""
    w = W[name].scaled(B=32, T=2048, H_kv=8)
    log(f"bulk quantize {name}: {codebook} codebook, {rotation} rotation, B=32 T=2048 H_kv=8, "
        f"K{w.k_bits}/V{w.v_bits}")
    model = OracleModel(w, codebook=codebook, rotation=rotation)
    rot = tq.make_rotation(tq_synth.ROT_SEED, tq.HADAMARD if rotation == "hadamard" else tq.HAAR)
    mk = {"gaussian": tq.make_codebook, "shifted": shifted_codebook}[codebook]
    for which, bits, role in (("k", w.k_bits, tq.KEYS), ("v", w.v_bits, tq.VALUES)):
        c = tq.Cache(role, bits, w.B, w.H_kv, w.T, rot=rot, centroids=mk(bits)[0])
        tq.quantize_kv(device_inputs(w, which), c)
        codes, norms = c.codes.cpu().numpy(), c.norms.cpu().numpy()
        thr = model.tK if which == "k" else model.tV
        for (b, h), ref in model.heads(which, bs=[0, 13, 31], hs=[0, 7]).items():
            n, mo, _ = code_mismatch(which, codes[b, h], ref, bits, thr, w.T)
            assert mo == 0, (which, b, h, n, mo)
            want = ref["norm"].astype(np.float64)
            assert np.all(np.abs(norms[b, h, : w.T] - want) <= 1e-6 * np.maximum(want, 1e-30)), (which, b, h)


@pytest.mark.parametrize("rotation", ["haar", "hadamard"])
def test_bulk_kernel_edges(tq, rotation):
    """Edges of the bulk kernel at a size that takes it (B=8, H_kv=8, 2,050
    tokens written at t_offset 3 into caches of 2,064 slots): partial value
    blocks at both ends keep the bits of the tokens around the written range (the
    caches start as all ones), zero vectors get the code of z = 0 and norm 0, and
    vectors scaled by 1e-30 and 1e30 (squared norms outside float32's safe range,
    so the kernel rescales them by a power of two) match the oracle on the same
    bfloat16 values."""
    w = W["stress70b"].scaled(B=8, T=2050, H_kv=8)
    t0, T_cap = 3, 2064
    log(f"bulk quantize edges, {rotation} rotation: B=8 H_kv=8, tokens [3, 2053) of 2064")
    model = OracleModel(w, rotation=rotation)
    rot = tq.make_rotation(tq_synth.ROT_SEED, tq.HADAMARD if rotation == "hadamard" else tq.HAAR)
    for which, bits, role in (("k", w.k_bits, tq.KEYS), ("v", w.v_bits, tq.VALUES)):
        x = tq_synth.kv_full(w, which)
        x[1, 100:140] = 0.0                      # zero vectors (all heads)
        x[2, :, 3] *= np.float32(1e-30)          # one head of tiny vectors
        x[3, 500:900, 5] *= np.float32(1e30)     # a run of huge ones
        xb = torch.from_numpy(x).to(torch.bfloat16)
        c = tq.Cache(role, bits, w.B, w.H_kv, T_cap, rot=rot)
        c.codes.fill_(-1)
        tq.quantize_kv(xb.cuda(), c, t_offset=t0)
        codes, norms = c.codes.cpu().numpy(), c.norms.cpu().numpy()
        thr = model.tK if which == "k" else model.tV
        xf = xb.float().numpy().astype(np.float64)
        full = (1 << bits) - 1
        for b, h in [(0, 0), (1, 2), (2, 3), (3, 5), (7, 7)]:
            ref = model.quantize(which, xf[b, :, h])
            got = unpack_head(which, codes[b, h], bits, T_cap)
            # the written range against the oracle
            bad = got[t0:t0 + w.T] != ref["codes"]
            exempt = oq.boundary_distance(ref["u"], thr, 128) < 1e-6
            assert int((bad & ~exempt).sum()) == 0, (which, b, h, int(bad.sum()))
            # the tokens around it keep their bits
            assert np.all(got[:t0] == full) and np.all(got[t0 + w.T:] == full), (which, b, h)
            want = ref["norm"].astype(np.float64)
            nr = norms[b, h, t0:t0 + w.T].astype(np.float64)
            assert np.all(np.abs(nr - want) <= 1e-6 * np.maximum(want, 1e-300)), (which, b, h)
        # zero vectors: the code of z = 0 (2^(bits-1) for the mirrored codebook) and norm 0
        z = unpack_head(which, codes[1, 2], bits, T_cap)[t0 + 100:t0 + 140]
        assert np.all(z == 1 << (bits - 1)) and np.all(norms[1, 2, t0 + 100:t0 + 140] == 0), which
