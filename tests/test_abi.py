"""C-ABI checks that need no GPU: the library loads, exports every declared symbol,
its host-only functions agree with the oracle, and every argument error is
reported before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_attention_tq_amd as tq
from oracle import codebook as ocb
from oracle import rotation as orot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert set(names) == set(tq.EXPORTS)
    for n in names:
        assert hasattr(tq.lib(), n), n


def test_struct_layout_matches_header():
    # 4 x int32, 3 x int64, 6 pointers, 16 floats, then the paged-layout fields
    # (a pointer and 2 x int64)
    assert ctypes.sizeof(tq.TQCache) == 16 + 24 + 48 + 64 + 24
    assert tq.TQCache.centroids.offset == 88
    assert tq.TQCache.block_table.offset == 152
    assert tq.TQCache.n_blocks.offset == 168


def test_status_strings():
    for code in range(6):
        assert tq.status_string(code)
    assert tq.status_string(0) == "ok"
    assert "unknown" in tq.status_string(99)
    # no device call has failed on this thread (argument errors are not device errors)
    assert tq.lib().tq_last_hip_error() == b"hipSuccess"


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_oracle(bits):
    c, t = tq.make_codebook(bits)
    oc, ot = ocb.canonical(bits)
    assert np.array_equal(c.astype(np.float64), oc)
    assert np.array_equal(t.astype(np.float64), ot)
    assert not np.signbit(t[len(t) // 2])


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_sphere_codebook_matches_oracle(bits):
    c, t = tq.make_codebook_sphere(bits)
    oc, ot = ocb.canonical_sphere(bits, 128)
    assert np.array_equal(c.astype(np.float64), oc)
    assert np.array_equal(t.astype(np.float64), ot)
    # d = 3: the uniform quantizer of [-1, 1], in units of sqrt(3) (fp16-rounded)
    c3, _ = tq.make_codebook_sphere(bits, 3)
    L = 1 << bits
    want = ((-1.0 + (2 * np.arange(L) + 1) / L) * np.sqrt(3)).astype(np.float16).astype(np.float32)
    assert np.array_equal(c3, want)
    lib = tq.lib()
    buf = np.zeros(16, dtype=np.float32)
    assert lib.tq_make_codebook_sphere(bits, 2, buf.ctypes.data, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_make_codebook_sphere(5, 128, buf.ctypes.data, None) == tq.ERR_INVALID_ARGUMENT


def test_codebook_rejects_bad_arguments():
    lib = tq.lib()
    c = np.zeros(16, dtype=np.float32)
    assert lib.tq_make_codebook(0, 128, c.ctypes.data, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_make_codebook(5, 128, c.ctypes.data, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_make_codebook(3, 128, None, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_make_codebook(3, 96, c.ctypes.data, None) == tq.ERR_UNSUPPORTED
    # the Gaussian codebook (standard units) is the same at every head dimension
    for d in (64, 256):
        c64, t64 = tq.make_codebook(3, d)
        c128, t128 = tq.make_codebook(3)
        assert np.array_equal(c64, c128) and np.array_equal(t64, t128)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("seed", [42, 7, 2**63 + 5])
def test_rotation_matches_oracle(seed, d):
    P = tq.make_rotation(seed, tq.HAAR, d).astype(np.float64)
    assert np.abs(P - orot.haar_rotation(seed, d)).max() <= 1e-6
    assert np.abs(P.T @ P - np.eye(d)).max() <= 1e-5
    S = tq.make_rotation(seed, tq.GAUSSIAN, d).astype(np.float64)
    assert np.abs(S - orot.qjl_projection(seed, d)).max() <= 1e-6
    H = tq.make_rotation(seed, tq.HADAMARD, d).astype(np.float64)
    assert np.array_equal(H, orot.hadamard_rotation(seed, d))


def test_rotation_rejects_bad_arguments():
    lib = tq.lib()
    out = np.zeros((128, 128), dtype=np.float32)
    assert lib.tq_make_rotation(1, 128, 7, out.ctypes.data) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_make_rotation(1, 128, 0, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_make_rotation(1, 96, 0, out.ctypes.data) == tq.ERR_UNSUPPORTED


def test_decode_planning():
    # chunks are whole multiples of 512 tokens (32-token steps for up to 16
    # wavefronts) and together cover T; auto mode aims at one workgroup per
    # compute unit of a 256-CU part
    for B, H, T in [(1, 8, 32768), (32, 8, 32768), (4, 4, 131072), (1, 1, 1024), (2, 3, 1), (1, 1, 0)]:
        n = tq.decode_splits(B, H, T)
        assert n >= 1
        assert (n - 1) * 512 < max(T, 1) or n == 1
        assert tq.decode_workspace_bytes(B, 4 * H, H, T) > 0
    assert tq.decode_splits(32, 8, 32768) == 1              # 256 (row, KV head) pairs: one chunk each
    assert tq.decode_splits(1, 8, 32768) == 32              # 8 pairs: 32 chunks of 1024 tokens
    assert tq.decode_splits(1, 1, 4096, 3) == 3             # ceil(4096 / 3) -> 1536 tokens
    assert tq.decode_splits(1, 1, 1024, 3) == 2             # ceil(1024 / 3) -> 512 tokens
    assert tq.decode_splits(1, 1, 1024, 100000) == 2        # chunks never go below 512 tokens
    assert tq.decode_workspace_bytes(1, 7, 2, 100) == 0     # H_q % H_kv != 0
    assert tq.decode_workspace_bytes(1, 34, 2, 100) == 0    # G > 16


# ------------------------------------------------------------------------
# argument validation without a device: fake (never dereferenced) pointers

FAKE = 1 << 20   # 16-byte aligned, never touched


def _cache(role=tq.KEYS, bits=3, qjl=0, B=2, H=2, T_cap=64, d=128, **kw):
    s = tq.TQCache()
    s.role, s.bits, s.qjl, s.d = role, bits, qjl, d
    s.B, s.H_kv, s.T_cap = B, H, T_cap
    s.codes = s.norms = s.rot = FAKE
    if qjl:
        s.qjl_signs = s.qjl_gamma = s.qjl_proj = FAKE
    c, _ = tq.make_codebook(bits if 1 <= bits <= 4 else 3)
    for i, v in enumerate(c):
        s.centroids[i] = float(v)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _quant(s, x=FAKE, dtype=tq.BF16, B=2, T=4, H=2, strides=(4 * 2 * 128, 2 * 128, 128), t_offset=0):
    return tq.lib().tq_quantize_kv(x, dtype, B, T, H, *strides, ctypes.byref(s), t_offset, None)


def test_quantize_validation_paths():
    assert _quant(_cache(bits=5)) == tq.ERR_UNSUPPORTED
    assert _quant(_cache(bits=1)) == tq.ERR_UNSUPPORTED
    assert _quant(_cache(d=96)) == tq.ERR_UNSUPPORTED
    assert _quant(_cache(d=512)) == tq.ERR_UNSUPPORTED
    assert _quant(_cache(d=64, qjl=1)) == tq.ERR_UNSUPPORTED        # QJL keys: d = 128 only
    assert _quant(_cache(d=256, qjl=1)) == tq.ERR_UNSUPPORTED
    assert _quant(_cache(d=64), T=0) == tq.OK                      # d = 64 and 256 are taken
    assert _quant(_cache(d=256, role=tq.VALUES), T=0) == tq.OK
    assert _quant(_cache(role=7)) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(role=tq.VALUES, qjl=1)) == tq.ERR_UNSUPPORTED
    assert _quant(_cache(role=tq.VALUES, T_cap=60)) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(codes=None)) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(qjl=1, qjl_signs=None)) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(codes=FAKE + 4)) == tq.ERR_ALIGNMENT
    assert _quant(_cache(), x=None) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(), x=FAKE + 2) == tq.ERR_ALIGNMENT
    assert _quant(_cache(), strides=(4 * 2 * 128, 2 * 128, 100)) == tq.ERR_ALIGNMENT
    assert _quant(_cache(), dtype=9) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(), B=3) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(), H=1) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(), t_offset=62) == tq.ERR_INVALID_ARGUMENT       # 62 + 4 > T_cap
    assert _quant(_cache(), t_offset=-1) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(), T=-1) == tq.ERR_INVALID_ARGUMENT
    assert _quant(_cache(), T=0) == tq.OK                                   # no-op, no launch
    s = _cache()
    s.centroids[3] = 0.1   # not float16-exact
    assert _quant(s) == tq.ERR_INVALID_ARGUMENT
    s = _cache()
    s.centroids[2], s.centroids[3] = s.centroids[3], s.centroids[2]   # not ascending
    assert _quant(s) == tq.ERR_INVALID_ARGUMENT


def _append(kc, vc, k=FAKE, v=FAKE, dtype=tq.BF16, B=2, H=2, strides=(2 * 128, 128, 2 * 128, 128), t_offset=5):
    return tq.lib().tq_append_kv(k, v, dtype, B, H, *strides, ctypes.byref(kc), ctypes.byref(vc), t_offset, None)


def test_append_validation_paths():
    K, V = _cache(), _cache(role=tq.VALUES)
    assert _append(V, V) == tq.ERR_INVALID_ARGUMENT                        # roles
    assert _append(K, K) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, _cache(role=tq.VALUES, B=3)) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, V, B=3) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, V, H=1) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, V, t_offset=64) == tq.ERR_INVALID_ARGUMENT           # past T_cap
    assert _append(K, _cache(role=tq.VALUES, T_cap=8), t_offset=8) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, V, t_offset=-1) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, V, k=None) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, V, v=None) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, V, v=FAKE + 2) == tq.ERR_ALIGNMENT
    assert _append(K, V, strides=(2 * 128, 100, 2 * 128, 128)) == tq.ERR_ALIGNMENT
    assert _append(K, V, dtype=9) == tq.ERR_INVALID_ARGUMENT
    assert _append(_cache(bits=5), V) == tq.ERR_UNSUPPORTED
    assert _append(K, _cache(role=tq.VALUES, codes=None)) == tq.ERR_INVALID_ARGUMENT
    assert _append(K, _cache(role=tq.VALUES, d=64)) == tq.ERR_INVALID_ARGUMENT   # one head dimension


def _fused(K, V, kn=FAKE, vn=FAKE, ndt=tq.BF16, strides=(2 * 128, 128, 2 * 128, 128), q=FAKE, H_q=4, ctx=None,
           T=64, ws=FAKE, wsb=1 << 20):
    return tq.lib().tq_decode_attention_append(ctypes.byref(K), ctypes.byref(V), kn, vn, ndt, *strides, q, tq.BF16,
                                               H_q, ctx, T, 0.0, 0, FAKE, ws, wsb, None)


def test_decode_append_validation_paths():
    K, V = _cache(), _cache(role=tq.VALUES)
    assert _fused(V, K) == tq.ERR_INVALID_ARGUMENT                       # roles
    assert _fused(K, V, kn=None) == tq.ERR_INVALID_ARGUMENT
    assert _fused(K, V, vn=None) == tq.ERR_INVALID_ARGUMENT
    assert _fused(K, V, ndt=9) == tq.ERR_INVALID_ARGUMENT
    assert _fused(K, V, kn=FAKE + 2) == tq.ERR_ALIGNMENT
    assert _fused(K, V, strides=(2 * 128, 100, 2 * 128, 128)) == tq.ERR_ALIGNMENT
    assert _fused(K, V, strides=(-1, 128, 2 * 128, 128)) == tq.ERR_INVALID_ARGUMENT
    assert _fused(K, V, T=65) == tq.ERR_INVALID_ARGUMENT                 # past T_cap
    assert _fused(K, V, q=None) == tq.ERR_INVALID_ARGUMENT
    assert _fused(K, V, H_q=3) == tq.ERR_INVALID_ARGUMENT
    assert _fused(K, V, wsb=0) == tq.ERR_WORKSPACE_TOO_SMALL
    # QJL keys with ragged contexts: the separate append launch needs one position
    KQ = _cache(qjl=1)
    assert _fused(KQ, V, ctx=FAKE) == tq.ERR_UNSUPPORTED


def test_prefill_validation_paths():
    K, V = _cache(), _cache(role=tq.VALUES)
    lib = tq.lib()
    def call(M=4, H_q=8, T=64, n_split=0, ws_bytes=1 << 30):
        return lib.tq_prefill_attention(ctypes.byref(K), ctypes.byref(V), FAKE, tq.BF16, H_q, M, None, T, 0.0,
                                        n_split, FAKE, FAKE, ws_bytes, None)
    assert call(M=0) == tq.ERR_INVALID_ARGUMENT
    assert call(M=-3) == tq.ERR_INVALID_ARGUMENT
    assert call(M=70000) == tq.ERR_UNSUPPORTED
    assert call(ws_bytes=16) == tq.ERR_WORKSPACE_TOO_SMALL
    assert call(H_q=7) == tq.ERR_INVALID_ARGUMENT                 # H_q % H_kv
    # d = 256 takes chunked prefill only up to 8 (query token, head) columns per KV head
    K256, V256 = _cache(d=256), _cache(role=tq.VALUES, d=256)
    assert lib.tq_prefill_attention(ctypes.byref(K256), ctypes.byref(V256), FAKE, tq.BF16, 8, 4, None, 64, 0.0, 0,
                                    FAKE, FAKE, 1 << 30, None) == tq.ERR_UNSUPPORTED
    # workspace grows with M (chunk partials per query token and head)
    one = tq.prefill_workspace_bytes(2, 8, 2, 1, 4096, 4, 0)
    assert one == tq.decode_workspace_bytes(2, 8, 2, 4096, 4, 0)
    # M = 6 query tokens: at least 6 tokens' partials (2 + 128 floats per row, head and chunk)
    assert tq.prefill_workspace_bytes(2, 8, 2, 6, 4096, 4, 0) >= 6 * 2 * 8 * 4 * 130 * 4
    assert tq.prefill_workspace_bytes(2, 8, 2, 0, 4096, 4, 0) == 0


def test_paged_cache_validation_paths():
    """Paged layout: block_tokens a power of two in 32..65536 dividing T_cap,
    n_blocks > 0, a 4-byte aligned table, arrays below 2 GiB."""
    def paged(**kw):
        args = dict(T_cap=64, block_table=FAKE, block_tokens=32, n_blocks=4)
        args.update(kw)
        return _cache(**args)
    for bad in (0, 16, 48, 96, 1 << 17):
        assert _quant(paged(block_tokens=bad)) == tq.ERR_INVALID_ARGUMENT, bad
    assert _quant(paged(T_cap=96, block_tokens=64)) == tq.ERR_INVALID_ARGUMENT   # 96 % 64
    assert _quant(paged(n_blocks=0)) == tq.ERR_INVALID_ARGUMENT
    assert _quant(paged(block_table=FAKE + 2)) == tq.ERR_ALIGNMENT
    assert _quant(paged(n_blocks=1 << 22, block_tokens=64)) == tq.ERR_UNSUPPORTED   # codes >= 2 GiB
    # a contiguous cache ignores block_tokens / n_blocks
    assert _quant(_cache(block_tokens=48, n_blocks=-1), T=0) == tq.OK
    assert _quant(paged(), T=0) == tq.OK


def _decode(k, v, q=FAKE, H_q=8, T=64, scale=0.0, n_split=0, out=FAKE, ws=FAKE, ws_bytes=1 << 30, dtype=tq.BF16):
    return tq.lib().tq_decode_attention(ctypes.byref(k), ctypes.byref(v), q, dtype, H_q, None, T, scale, n_split,
                                        out, ws, ws_bytes, None)


def test_decode_validation_paths():
    K, V = _cache(), _cache(role=tq.VALUES)
    assert _decode(V, V) == tq.ERR_INVALID_ARGUMENT                 # keys must be keys
    assert _decode(K, K) == tq.ERR_INVALID_ARGUMENT
    assert _decode(K, _cache(role=tq.VALUES, B=3)) == tq.ERR_INVALID_ARGUMENT
    assert _decode(K, V, H_q=7) == tq.ERR_INVALID_ARGUMENT          # H_q % H_kv
    assert _decode(K, V, H_q=34) == tq.ERR_UNSUPPORTED              # G = 17 > 16
    assert _decode(K, V, T=65) == tq.ERR_INVALID_ARGUMENT           # T > T_cap
    assert _decode(K, V, q=None) == tq.ERR_INVALID_ARGUMENT
    assert _decode(K, V, out=FAKE + 4) == tq.ERR_ALIGNMENT
    assert _decode(K, V, ws_bytes=16) == tq.ERR_WORKSPACE_TOO_SMALL
    assert _decode(K, V, ws=None) == tq.ERR_WORKSPACE_TOO_SMALL
    assert _decode(K, V, ws=FAKE + 16) == tq.ERR_ALIGNMENT
    assert _decode(K, V, scale=float("nan")) == tq.ERR_INVALID_ARGUMENT
    assert _decode(K, V, n_split=-1) == tq.ERR_INVALID_ARGUMENT
    assert _decode(K, V, dtype=5) == tq.ERR_INVALID_ARGUMENT
    assert _decode(K, _cache(role=tq.VALUES, d=256)) == tq.ERR_INVALID_ARGUMENT   # K and V head dims differ
    assert _decode(_cache(d=64), _cache(role=tq.VALUES, d=64), H_q=34) == tq.ERR_UNSUPPORTED


def test_dequantize_validation_paths():
    lib = tq.lib()
    K = _cache()
    assert lib.tq_dequantize(ctypes.byref(K), 5, 4, FAKE, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_dequantize(ctypes.byref(K), 0, 65, FAKE, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_dequantize(ctypes.byref(K), 0, 8, None, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_dequantize(ctypes.byref(K), 0, 8, FAKE + 8, None) == tq.ERR_ALIGNMENT
    assert lib.tq_dequantize(ctypes.byref(K), 3, 3, FAKE, None) == tq.OK


def _decode_noalloc(k, v, q=FAKE, H_q=8, T=64, scale=0.0, n_split=0, out=FAKE, dtype=tq.BF16):
    return tq.lib().tq_decode_attention_noalloc(ctypes.byref(k), ctypes.byref(v), q, dtype, H_q, None, T, scale,
                                                n_split, out, None)


def test_decode_noalloc_validation_paths():
    """The allocation-free decode reports every argument error of
    tq_decode_attention before any HIP call, and a call whose chunk partials
    would not fit the library's static scratch as a workspace error."""
    K, V = _cache(), _cache(role=tq.VALUES)
    assert _decode_noalloc(V, V) == tq.ERR_INVALID_ARGUMENT
    assert _decode_noalloc(K, _cache(role=tq.VALUES, B=3)) == tq.ERR_INVALID_ARGUMENT
    assert _decode_noalloc(K, V, H_q=7) == tq.ERR_INVALID_ARGUMENT
    assert _decode_noalloc(K, V, H_q=34) == tq.ERR_UNSUPPORTED
    assert _decode_noalloc(K, V, T=65) == tq.ERR_INVALID_ARGUMENT
    assert _decode_noalloc(K, V, q=None) == tq.ERR_INVALID_ARGUMENT
    assert _decode_noalloc(K, V, out=FAKE + 4) == tq.ERR_ALIGNMENT
    assert _decode_noalloc(K, V, scale=float("nan")) == tq.ERR_INVALID_ARGUMENT
    assert _decode_noalloc(K, V, n_split=-1) == tq.ERR_INVALID_ARGUMENT
    assert _decode_noalloc(K, V, dtype=5) == tq.ERR_INVALID_ARGUMENT
    # 8 rows x 128 query heads x 64 chunks of partials (130 floats each) is
    # about 34 MB, beyond the 16 MiB scratch
    big_k = _cache(B=8, H=8, T_cap=32768)
    big_v = _cache(role=tq.VALUES, B=8, H=8, T_cap=32768)
    need = tq.decode_workspace_bytes(8, 128, 8, 32768, 64, 0)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    assert _decode_noalloc(big_k, big_v, H_q=128, T=32768, n_split=64) == tq.ERR_WORKSPACE_TOO_SMALL


def test_stream_read_validation_paths():
    lib = tq.lib()
    assert lib.tq_stream_read(None, 1 << 20, FAKE, 8, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_stream_read(FAKE, 0, FAKE, 8, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_stream_read(FAKE, 1 << 20, FAKE, 0, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_stream_read(FAKE + 8, 1 << 20, FAKE, 8, None) == tq.ERR_ALIGNMENT
    assert lib.tq_stream_read(FAKE, (1 << 20) + 4, FAKE, 8, None) == tq.ERR_ALIGNMENT
    assert lib.tq_stream_read(FAKE, 1 << 32, FAKE, 1, None) == tq.ERR_UNSUPPORTED
