"""The allocation-free decode entry point (tq_decode_attention_noalloc, called
through the C ABI) against tq_decode_attention with a caller workspace: the
same kernels and plan, so the outputs must be bitwise equal. Two calls in a
row on context-split plans (the partials live in the library's static scratch),
the second with smaller inputs, then a single-chunk plan and a ragged one."""
import ctypes

import pytest

import tq_synth
from tqhelp import device_inputs, device_queries, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = tq_synth.WORKLOADS


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_tq_amd as lib
    return lib


def _filled(tq, w):
    T_cap = (w.T + 7) // 8 * 8
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, qjl=bool(w.k_qjl))
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap)
    tq.quantize_kv(device_inputs(w, "k"), kc)
    tq.quantize_kv(device_inputs(w, "v"), vc)
    return kc, vc


def _noalloc(tq, kc, vc, q, T, out, ctx=None, n_split=0):
    sk, sv = kc.struct(), vc.struct()
    st = tq.lib().tq_decode_attention_noalloc(ctypes.byref(sk), ctypes.byref(sv), q.data_ptr(), tq.BF16
                                              if q.dtype == torch.bfloat16 else tq.F32, q.shape[1],
                                              None if ctx is None else ctx.data_ptr(), T, 0.0, n_split,
                                              out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == tq.OK, tq.status_string(st)


def test_noalloc_equals_workspace_call(tq):
    big = W["llama8b"].scaled(T=16384)       # 8 units -> 16 context chunks
    small = W["qjl"].scaled(B=2, T=3000)     # QJL keys, G = 4, ragged T -> smaller plan
    cases = [(big, None, 0), (small, None, 0), (small, [3000, 1777], 0), (big, None, 1)]
    outs = {}
    for w, ctx, ns in cases:
        kc, vc = _filled(tq, w)
        q = device_queries(w)
        cl = None if ctx is None else torch.tensor(ctx, dtype=torch.int32, device="cuda")
        plan = tq.decode_splits(w.B, w.H_kv, w.T, ns)
        need = tq.decode_workspace_bytes(w.B, w.H_q, w.H_kv, w.T, ns, w.k_qjl)
        log(f"noalloc {w.name}: B={w.B} H_q={w.H_q} T={w.T} ctx={ctx} n_split={plan} partials {need} B")
        assert need <= tq.NOALLOC_SCRATCH_BYTES
        want = tq.decode_attention(kc, vc, q, ctx_lens=cl, T=w.T, n_split=ns)
        got = torch.full_like(want, float("nan"))
        _noalloc(tq, kc, vc, q, w.T, got, cl, ns)
        got2 = tq.decode_attention_noalloc(kc, vc, q, ctx_lens=cl, T=w.T, n_split=ns)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert torch.equal(got2, want)
        outs[(w.name, w.T, str(ctx), ns)] = got
    assert len(outs) == len(cases)
