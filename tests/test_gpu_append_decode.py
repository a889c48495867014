"""One decode step in one call (tq_decode_attention_append) against the same
step in two calls (tq_append_kv at the row's last token, then
tq_decode_attention).

The one-call step writes the new key and value of every (row, KV head) to
token ctx_b - 1 (per row, from the context lengths) with the append kernel's
arithmetic, so the caches must hold the same bytes and the decode output must
be bitwise equal. Context lengths put the new token at the first token of a
wavefront's share, in a masked tail step, at a chunk boundary and in a row of
its own; rows with no context get no write and zeros. Keys with a QJL sketch
take the tiled quantize kernel; G = 16 and float32 inputs are covered too.
Every case also runs on paged caches (32-token blocks mapped through a seeded
permutation), where the outputs must again be bitwise equal: context splits,
a G = 4 ragged tail, K4/V2, QJL keys appended through the block table by the
tiled kernel, and float32 inputs with G = 16.
"""
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


def _caches(tq, w, T_cap, paged=False):
    kw = {}
    if paged:
        bt = 32
        maxblk = T_cap // bt
        perm = torch.randperm(w.B * maxblk, generator=torch.Generator().manual_seed(3), dtype=torch.int64)
        table = perm.to(torch.int32).reshape(w.B, maxblk).cuda()
        kw = dict(block_table=table, block_tokens=bt, n_blocks=w.B * maxblk)
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, qjl=bool(w.k_qjl), **kw)
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, **kw)
    return kc, vc


def _arrays(c):
    return [a for a in (c.codes, c.norms, c.signs, c.gamma) if a is not None]


def _clone(tq, c, w, T_cap):
    d = tq.Cache(c.role, c.bits, w.B, w.H_kv, T_cap, qjl=bool(c.qjl), block_table=c.block_table,
                 block_tokens=c.block_tokens, n_blocks=c.n_blocks)
    for a, b in zip(_arrays(d), _arrays(c)):
        a.copy_(b)
    return d


def _row_equal(tq, got, want, b):
    """Row b of two contiguous caches holds the same bytes (all of its token rows)."""
    return all(torch.equal(x[b].view(torch.int32), y[b].view(torch.int32)) for x, y in zip(_arrays(got), _arrays(want)))


CASES = {
    # name: (workload, T_cap, ctx per row (None: every row at T), n_split)
    "stress70b_full": (W["stress70b"].scaled(B=2, T=4096), 4096, None, 0),
    "stress70b_ragged": (W["stress70b"].scaled(B=4, T=4096), 4096, [4096, 33, 0, 1], 0),
    "stress70b_split4": (W["stress70b"].scaled(B=4, T=4096), 4096, [4096, 1025, 512, 2000], 4),
    "llama8b_tail": (W["llama8b"].scaled(T=2000), 2000, None, 0),
    "qwen_k4v2": (W["qwen"].scaled(B=2, T=1500), 1504, [1500, 737], 0),
    "qjl_two_launches": (W["qjl"].scaled(B=2, T=1024), 1024, None, 0),
    "tiny_f32_G16": (W["tiny"], 1024, None, 0),
}


@pytest.mark.parametrize("name,paged", [(n, p) for p in (False, True) for n in CASES])
def test_one_call_step_equals_two_calls(tq, name, paged):
    w, T_cap, ctx, n_split = CASES[name]
    if paged:
        T_cap = (T_cap + 31) // 32 * 32   # whole 32-token blocks
    log(f"one-call append + decode {name}{' paged' if paged else ''}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} "
        f"K{w.k_bits}/V{w.v_bits} ctx {ctx or [w.T] * w.B} n_split={n_split}")
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    kc, vc = _caches(tq, w, T_cap, paged)
    tq.quantize_kv(xk, kc)
    tq.quantize_kv(xv, vc)
    # new vectors: the recipe's vectors of a shifted token window, so they differ
    # from what the caches hold
    new_k = torch.roll(xk, 7, dims=1)[:, 0].contiguous()
    new_v = torch.roll(xv, 5, dims=1)[:, 0].contiguous()
    q = device_queries(w)
    cl = None if ctx is None else torch.tensor(ctx, dtype=torch.int32, device="cuda")
    rows = [w.T] * w.B if ctx is None else ctx

    refs = []
    for b in range(w.B):
        rk, rv = _clone(tq, kc, w, T_cap), _clone(tq, vc, w, T_cap)
        if rows[b] >= 1:
            tq.append_kv(new_k, new_v, rk, rv, rows[b] - 1)
        refs.append((rk, rv, tq.decode_attention(rk, rv, q, ctx_lens=cl, T=w.T, n_split=n_split)))
        if ctx is None:
            break   # every row appends at the same position: one reference serves all
    out = tq.decode_attention_append(kc, vc, new_k, new_v, q, ctx_lens=cl, T=w.T, n_split=n_split)
    torch.cuda.synchronize()
    for b in range(w.B):
        rk, rv, ro = refs[0] if ctx is None else refs[b]
        assert torch.equal(out[b], ro[b]), b
        # (with a block table the rows share the arrays and a reference appended
        # every row at row b's position, so only the outputs are compared)
        if not paged:
            assert _row_equal(tq, kc, rk, b) and _row_equal(tq, vc, rv, b), b
        if rows[b] == 0:
            assert torch.all(out[b] == 0)


def test_one_call_step_repeated(tq):
    """Steps that append token after token: the caches after the last step equal
    those built by tq_append_kv, and each step's output equals the two-call step."""
    w = W["stress70b"].scaled(B=2, T=96)
    T_cap = 128
    log("one-call append + decode, 40 consecutive steps")
    xk, xv = device_inputs(w, "k"), device_inputs(w, "v")
    kc, vc = _caches(tq, w, T_cap)
    rk, rv = _caches(tq, w, T_cap)
    for c, x in ((kc, xk), (vc, xv), (rk, xk), (rv, xv)):
        tq.quantize_kv(x[:, :56], c)
    q = device_queries(w)
    for t in range(56, 96):
        o1 = tq.decode_attention_append(kc, vc, xk[:, t], xv[:, t], q, T=t + 1)
        tq.append_kv(xk[:, t], xv[:, t], rk, rv, t)
        o2 = tq.decode_attention(rk, rv, q, T=t + 1)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), t
    for x, y in zip(_arrays(kc) + _arrays(vc), _arrays(rk) + _arrays(rv)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
