"""Benchmark of the TurboQuant packed-KV decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stress70b]

One step is one pass of the whole hot path for one new token per batch row, in
one call (tq_decode_attention_append): quantize the new token's key and value
vectors of every (row, KV head) into the packed caches at t = T-1 (one launch),
then decode attention of all query heads over the T-token packed caches (a
second launch). Inputs are resident in HBM before timing starts. Prints one
JSON line on stdout.

Extra fields: `roofline` (the decode launch vs the HBM peak), `cpu_baseline`
(the CPU oracle on a bounded sample of the same step, scaled to tokens/s),
`quantize_prefill` (bulk quantization of the whole context, HBM and MFMA view).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "decode attention tokens/s and packed-KV HBM GB/s (% of peak) at 32k ctx, 3-bit"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, AMD published


ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM traffic of the decode kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# (calibrated against a copy of known size), valid for the kernel sources whose
# hash it records
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_scan_stress70b_hbm_traffic.md")
KERNEL_SOURCES = ["decode_attention_tq_amd/csrc/tq_decode.hip", "decode_attention_tq_amd/csrc/tq_device.h",
                  "decode_attention_tq_amd/csrc/tq_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """Bytes per decode launch from the committed counter summary, or None when
    it is missing, covers another workload or predates the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split("=", 1) for line in (l.strip() for l in f) if "=" in line and " " not in line.split("=")[0])
    except OSError:
        return None
    if kv.get("workload") != workload or kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_bytes(w, T):
    """Algorithmic bytes of one decode call: packed K and V (codes + fp32 norms, QJL
    signs + gamma), the query in, the fp32 output, the two rotations."""
    d = w.d
    wk = d * w.k_bits // 8 + 4 + (d // 8 + 4 if w.k_qjl else 0)
    wv = d * w.v_bits // 8 + 4
    qb = 2 if w.dtype == "bf16" else 4
    return w.B * w.H_kv * T * (wk + wv) + w.B * w.H_q * d * (qb + 4) + 2 * d * d * 4


def append_bytes(w):
    """Algorithmic bytes of appending one token per (row, KV head): the new key and
    value in, the key record and norm out, the value block record read and written
    back (its other tokens' bits kept), the value norm out."""
    d = w.d
    xb = 2 if w.dtype == "bf16" else 4
    vblock = 8 * d * w.v_bits // 8
    return w.B * w.H_kv * (2 * d * xb + d * w.k_bits // 8 + 4 + 2 * vblock + 4)


def quantize_bytes(w, ntok, which):
    d = w.d
    bits = w.k_bits if which == "k" else w.v_bits
    inb = 2 if w.dtype == "bf16" else 4
    extra = (d // 8 + 4) if (which == "k" and w.k_qjl) else 0
    return w.B * w.H_kv * ntok * (d * inb + d * bits // 8 + 4 + extra)


def copy_cache(tq, c):
    """A second contiguous cache holding the same packed layer."""
    d = tq.Cache(c.role, c.bits, c.B, c.H_kv, c.T_cap, device=c.device, qjl=bool(c.qjl))
    for x, y in ((d.codes, c.codes), (d.norms, c.norms), (d.signs, c.signs), (d.gamma, c.gamma)):
        if x is not None:
            x.copy_(y)
    return d


def cpu_baseline(w, budget_s=12.0):
    """The CPU oracle, as it stands, on (row, KV head) slices of the same step:
    unpack the slice's packed key and value caches, quantize one new token of
    each, decode the G query heads over T tokens. Scaled to decode tokens/s of
    the whole batch."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import tq_synth
    from oracle import attention as oa
    from oracle import codebook as ocb
    from oracle import quantize as oq
    from oracle import rotation as orot

    Pi = orot.haar_rotation(tq_synth.ROT_SEED, w.d)
    cK, tK = ocb.canonical(w.k_bits)
    cV, tV = ocb.canonical(w.v_bits)
    step_times = []
    slices = 0
    t_setup = time.perf_counter()
    while True:
        b, h = divmod(slices, w.H_kv)
        if b >= w.B:
            break
        K = tq_synth.kv_head(w, "k", b, h)
        V = tq_synth.kv_head(w, "v", b, h)
        kq = oq.quantize_head(K, Pi, cK, tK)
        vq = oq.quantize_head(V, Pi, cV, tV)
        kwords = oq.pack_keys(kq["codes"], w.k_bits)
        vwords = oq.pack_values(vq["codes"], w.v_bits)
        q = tq_synth.queries(w, b)[h * w.G:(h + 1) * w.G]
        t0 = time.perf_counter()
        new = oq.quantize_head(K[-1:], Pi, cK, tK), oq.quantize_head(V[-1:], Pi, cV, tV)
        k = {"codes": oq.unpack_keys(kwords, w.k_bits, w.d), "norm": kq["norm"]}
        v = {"codes": oq.unpack_values(vwords, w.v_bits, w.d), "norm": vq["norm"]}
        k["codes"][-1], v["codes"][-1] = new[0]["codes"][0], new[1]["codes"][0]
        oa.attend_rotated(q, k, v, Pi, Pi, cK, cV, w.d, 1.0 / math.sqrt(w.d))
        step_times.append(time.perf_counter() - t0)
        slices += 1
        if sum(step_times) >= budget_s or time.perf_counter() - t_setup > 3 * budget_s:
            break
    per_slice = sum(step_times) / len(step_times)
    full_step = per_slice * w.B * w.H_kv
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": w.B / full_step,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{slices} of {w.B * w.H_kv} (row, KV head) slices of the same step: unpack the packed "
                   f"K/V slice ({w.T} tokens), quantize 1 new token each, rotated-domain decode of "
                   f"{w.G} query heads; {per_slice * 1e3:.1f} ms per slice, scaled by {w.B * w.H_kv} slices "
                   f"to the batch of {w.B} rows"),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stress70b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--prefill-iters", type=int, default=3)
    ap.add_argument("--formats", default="llama8b,qwen,qjl",
                    help="other workloads whose decode is also timed (their own bit widths); '' to skip")
    ap.add_argument("--prefill-m", default="2,16",
                    help="chunk sizes M of chunked causal attention timed on the same caches ('' to skip)")
    ap.add_argument("--paged-block", type=int, default=256,
                    help="also time decode on paged caches with this many tokens per block (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_attention_tq_amd as tq
    import tq_synth

    w = tq_synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = w.T
    T_cap = (T + 7) // 8 * 8

    log(f"[bench] workload {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} T={T} K{w.k_bits}/V{w.v_bits}")
    kc = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, device=dev, qjl=bool(w.k_qjl))
    vc = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, device=dev)

    # ---- prefill: bulk quantization of the whole context (also builds the caches)
    xk = tq_synth.torch_kv(w, "k", dev)
    xv = tq_synth.torch_kv(w, "v", dev)
    torch.cuda.synchronize()
    pre_ms = []
    for it in range(args.prefill_iters + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tq.quantize_kv(xk, kc)
        tq.quantize_kv(xv, vc)
        e1.record()
        torch.cuda.synchronize()
        if it > 0:
            pre_ms.append(e0.elapsed_time(e1))
    pre = sum(pre_ms) / len(pre_ms)
    ntok = w.B * w.H_kv * T * 2
    qbytes = quantize_bytes(w, T, "k") + quantize_bytes(w, T, "v")
    # algorithmic rotation flops (y = Pi x per vector, plus S r per QJL key); the MFMA
    # issues 2 fp16 passes per product (hi and lo halves of Pi), 3 for QJL's S r
    qflops = 2 * w.d * w.d * ntok + (2 * w.d * w.d * w.B * w.H_kv * T if w.k_qjl else 0)
    issued = 2 * 2 * w.d * w.d * ntok + (3 * 2 * w.d * w.d * w.B * w.H_kv * T if w.k_qjl else 0)
    new_k = xk[:, T - 1:T].contiguous()
    new_v = xv[:, T - 1:T].contiguous()
    del xk, xv
    torch.cuda.empty_cache()

    # ---- decode steps
    qs = [tq_synth.torch_queries(w, dev, seed_offset=i) for i in range(4)]
    out = torch.empty((w.B, w.H_q, w.d), dtype=torch.float32, device=dev)
    ws = tq.Workspace(tq.decode_workspace_bytes(w.B, w.H_q, w.H_kv, T, 0, w.k_qjl), dev)

    # one step = one call: the new key and value of every (row, KV head) go to
    # token T - 1 (one launch), then decode attention over T tokens
    def step(i):
        tq.decode_attention_append(kc, vc, new_k, new_v, qs[i % len(qs)], T=T, out=out, workspace=ws)

    for i in range(args.warmup):
        step(i)
    # the timed steps: nothing but the steps between the two synchronizations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    # the same steps again as their two launches with events around each, for
    # the split between append and decode and the decode launch's duration (the
    # roofline)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        a, b, c = evs[i]
        a.record()
        tq.append_kv(new_k, new_v, kc, vc, T - 1)
        b.record()
        tq.decode_attention(kc, vc, qs[i % len(qs)], T=T, out=out, workspace=ws)
        c.record()
    torch.cuda.synchronize()
    dec_list = sorted(b.elapsed_time(c) for a, b, c in evs)
    dec_ms = sum(dec_list) / args.steps
    app_ms = sum(a.elapsed_time(b) for a, b, c in evs) / args.steps
    dec_med = dec_list[len(dec_list) // 2]
    dec_p10, dec_p90 = dec_list[len(dec_list) // 10], dec_list[(9 * len(dec_list)) // 10]

    # decode alone, back to back (no appends in between), for reference
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(50):
        tq.decode_attention(kc, vc, qs[i % len(qs)], T=T, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    dec_only_us = e0.elapsed_time(e1) / 50 * 1e3
    dbytes = decode_bytes(w, T)
    n_split = tq.decode_splits(w.B, w.H_kv, T)
    achieved = dbytes / (dec_ms * 1e-3) / 1e9
    log(f"[bench] step {ms_step * 1e3:.1f} us (append {app_ms * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us); "
        f"decode {achieved:.0f} GB/s = {achieved / HBM_PEAK_GBS:.1%} of peak")

    # the same step on paged caches: logical blocks of every row mapped to a
    # seeded permutation of physical blocks (a runtime's block-table cache)
    paged = None
    bt = args.paged_block
    if bt > 0 and T_cap % bt == 0:
        maxblk = T_cap // bt
        perm = torch.randperm(w.B * maxblk, generator=torch.Generator().manual_seed(5), dtype=torch.int64)
        table = perm.to(torch.int32).reshape(w.B, maxblk).to(dev)
        pk = tq.Cache(tq.KEYS, w.k_bits, w.B, w.H_kv, T_cap, device=dev, qjl=bool(w.k_qjl),
                      block_table=table, block_tokens=bt, n_blocks=w.B * maxblk)
        pv = tq.Cache(tq.VALUES, w.v_bits, w.B, w.H_kv, T_cap, device=dev,
                      block_table=table, block_tokens=bt, n_blocks=w.B * maxblk)
        tq.quantize_kv(tq_synth.torch_kv(w, "k", dev), pk)
        tq.quantize_kv(tq_synth.torch_kv(w, "v", dev), pv)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        pout = torch.empty_like(out)
        for i in range(5):
            tq.decode_attention(pk, pv, qs[i % len(qs)], T=T, out=pout, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(50):
            tq.decode_attention_append(pk, pv, new_k, new_v, qs[i % len(qs)], T=T, out=pout, workspace=ws)
        e1.record()
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record()
        for i in range(50):
            tq.decode_attention(pk, pv, qs[i % len(qs)], T=T, out=pout, workspace=ws)
        e3.record()
        torch.cuda.synchronize()
        p_step = e0.elapsed_time(e1) / 50 * 1e3
        p_dec = e2.elapsed_time(e3) / 50 * 1e3
        paged = {"block_tokens": bt, "physical_blocks": w.B * maxblk, "table": "seeded permutation",
                 "step_us": p_step, "decode_us_back_to_back": p_dec,
                 "decode_GB_s": dbytes / (p_dec * 1e-6) / 1e9,
                 "decode_frac": dbytes / (p_dec * 1e-6) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] paged (block {bt}): step {p_step:.1f} us, decode {p_dec:.1f} us back to back")
        del pk, pv
        torch.cuda.empty_cache()

    # decode of the other workloads (other bit widths, QJL keys, G = 4 and 7,
    # context splits), each on its own caches, back to back
    formats = {}
    for name in [n for n in args.formats.split(",") if n]:
        fw = tq_synth.WORKLOADS[name]
        fcap = (fw.T + 7) // 8 * 8
        fk = tq.Cache(tq.KEYS, fw.k_bits, fw.B, fw.H_kv, fcap, device=dev, qjl=bool(fw.k_qjl))
        fv = tq.Cache(tq.VALUES, fw.v_bits, fw.B, fw.H_kv, fcap, device=dev)
        tq.quantize_kv(tq_synth.torch_kv(fw, "k", dev), fk)
        tq.quantize_kv(tq_synth.torch_kv(fw, "v", dev), fv)
        fq = tq_synth.torch_queries(fw, dev)
        fws = tq.Workspace(tq.decode_workspace_bytes(fw.B, fw.H_q, fw.H_kv, fw.T, 0, fw.k_qjl), dev)
        fo = torch.empty((fw.B, fw.H_q, fw.d), dtype=torch.float32, device=dev)
        fb = decode_bytes(fw, fw.T)
        # copies of the layer, so that one sweep over them (>= 1 GiB) cannot be
        # served from the 256 MB last-level cache: calls cycle through them
        n_layers = max(1, min(64, -(-(1 << 30) // fb)))
        layers = [(fk, fv)] + [(copy_cache(tq, fk), copy_cache(tq, fv)) for _ in range(n_layers - 1)]
        for i in range(5):
            tq.decode_attention(*layers[i % n_layers], fq, T=fw.T, out=fo, workspace=fws)
        n_calls = max(50, 2 * n_layers)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_calls):
            tq.decode_attention(*layers[i % n_layers], fq, T=fw.T, out=fo, workspace=fws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n_calls * 1e3
        formats[name] = {"B": fw.B, "H_q": fw.H_q, "H_kv": fw.H_kv, "T": fw.T, "k_bits": fw.k_bits,
                         "v_bits": fw.v_bits, "k_qjl": fw.k_qjl,
                         "n_split": tq.decode_splits(fw.B, fw.H_kv, fw.T), "layers_cycled": n_layers, "decode_us": us,
                         "bytes": fb, "GB_s": fb / (us * 1e-6) / 1e9, "frac": fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] {name}: decode {us:.1f} us, {fb / (us * 1e-6) / 1e9:.0f} GB/s")
        del fk, fv, fws, layers
        torch.cuda.empty_cache()

    # chunked causal (prefill) attention of the M newest tokens of every row over
    # the same caches; the cache is read once per tile of query tokens
    prefill = {}
    for M in [int(m) for m in args.prefill_m.split(",") if m]:
        pq = torch.randn((w.B, M, w.H_q, w.d), generator=torch.Generator(device=dev).manual_seed(M), device=dev)
        pq = pq.to(torch.bfloat16) if w.dtype == "bf16" else pq
        pws = tq.Workspace(tq.prefill_workspace_bytes(w.B, w.H_q, w.H_kv, M, T, 0, w.k_qjl), dev)
        po = torch.empty((w.B, M, w.H_q, w.d), dtype=torch.float32, device=dev)
        for _ in range(3):
            tq.prefill_attention(kc, vc, pq, T=T, out=po, workspace=pws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            tq.prefill_attention(kc, vc, pq, T=T, out=po, workspace=pws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 20 * 1e3
        Mt = M if M * w.G <= 8 else min(M, 16 // w.G)
        tiles = -(-M // Mt)
        pb = tiles * (decode_bytes(w, T) - w.B * w.H_q * w.d * 6) + w.B * M * w.H_q * w.d * 6
        prefill[str(M)] = {"us": us, "query_tokens_per_s": w.B * M / (us * 1e-6), "tiles_per_row": tiles,
                           "bytes": pb, "GB_s": pb / (us * 1e-6) / 1e9, "frac": pb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] prefill attention M={M}: {us:.1f} us, {w.B * M / (us * 1e-6):.0f} query tokens/s, "
            f"{pb / (us * 1e-6) / 1e9:.0f} GB/s")
        del pws, po, pq

    # calibration copy of known size for the rocprofv3 byte counters (256 MiB read + write)
    cal = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    torch.cuda.synchronize()
    del cal, cal2

    res = {
        "metric": METRIC,
        "value": w.B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "d": w.d, "T": T,
                   "k_bits": w.k_bits, "v_bits": w.v_bits, "k_qjl": w.k_qjl, "input_dtype": w.dtype,
                   "step": "quantize 1 new K,V token per (row, KV head) + decode attention over T tokens",
                   "n_split": n_split},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(w.name),
                     "kernel": (f"decode_scan_kernel<{w.k_bits},{w.v_bits},{int(bool(w.k_qjl))},{int(w.G > 8)},0>"
                                + (" (the whole tq_decode_attention launch)" if n_split == 1
                                   else f" + combine_kernel ({n_split} context chunks)")),
                     "bytes_per_launch": dbytes, "launch_us": dec_ms * 1e3},
        "decode": {"us": dec_ms * 1e3, "us_median": dec_med * 1e3, "us_p10": dec_p10 * 1e3,
                   "us_p90": dec_p90 * 1e3, "us_back_to_back": dec_only_us,
                   "kv_tokens_per_s": w.B * T / (dec_ms * 1e-3),
                   "tokens_per_s": w.B / (dec_ms * 1e-3), "append_us": app_ms * 1e3,
                   "append_bytes": append_bytes(w)},
        "quantize_prefill": {"ms": pre, "vectors": ntok, "GB_s": qbytes / (pre * 1e-3) / 1e9,
                             "hbm_frac": qbytes / (pre * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "rotation_TFLOP_s": qflops / (pre * 1e-3) / 1e12,
                             "mfma_issued_TFLOP_s": issued / (pre * 1e-3) / 1e12,
                             "mfma_frac": issued / (pre * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS},
    }
    if paged is not None:
        res["paged"] = paged
    if formats:
        res["formats"] = formats
    if prefill:
        res["prefill_attention"] = prefill
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
