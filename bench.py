#!/usr/bin/env python3
"""Benchmark of the block-sparse landmark attention path on one MI355X.

One step = one pass of the whole prefill path over the SAS workload at 128K tokens
(B=1, 32 query / 8 kv heads, D=128, bf16, top-K=32 plus sink and two local blocks):
landmark pooling, selector vectors, MFMA block scoring, top-K selection and the gated
block-sparse attention.  Inputs are synthetic (clustered keys, aimed queries), generated on
the device before the timed region.  `value` is prefill tokens/s over the timed steps.

Reported beside it, measured in the same run:
* the attention kernel's attended TFLOP/s and its fraction of the bf16 MFMA peak (HIP events
  around that kernel on the stream it is launched on);
* the decode path (32 sequences x 128K cached tokens, 64 query / 8 kv heads, top-K=64):
  selection + split-K attention, algorithmic HBM GB/s and fraction of the HBM peak, with the
  caches flushed (a 1 GiB read) between timed steps;
* the same decode step over a ragged batch held in a paged cache (32 sequences of 16K..128K
  tokens in shuffled 64-token pages);
* the backward of the SAS prefill (dq, dk, dv and the selector-score gradient) on the same
  workload, and the HiLS backward (dq, dk, dv and the landmark gradient) on the same shape and
  attended sets, each timed per call (--no-backward skips both);
* the same prefill step with the flat clustered (LSA) index -- pool, Ward index build,
  selection over the index, attention -- each part timed, and again with the tree index (beam
  search over groups of segments, segments and clusters) (--no-lsa skips both);
* the HiLS prefill step at 1M tokens (pool, selection, per-chunk attention; --no-hils skips it);
* the float64 oracle timed on the host cores on a bounded sample of the prefill workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-hils]
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tok/s + attended TFLOP/s at 128K; decode HBM GB/s (top-K block attn)"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def attended_flops(B, Hq, D, T, K, n_sink=1, n_local=2):
    """4*D flops (QK^T and PV) per visible (query, key) pair per query head."""
    total = 0
    nqb = (T + 63) // 64
    for c in range(nqb):
        n_att = min(c + 1, K + n_sink + n_local)
        diag = 64 * 65 // 2 if (c + 1) * 64 <= T else (T - 64 * c) * (T - 64 * c + 1) // 2
        total += 64 * min(64, T - 64 * c) * (n_att - 1) + diag
    return 4 * D * Hq * B * total


def decode_bytes(B, Hq, Hkv, Tk, D, K, elem=2, n_sink=1, n_local=2):
    """Bytes a decode step must move: candidate landmarks, the attended K and V blocks, q, o."""
    c = (Tk - 1) // 64
    n_cand = max(0, c - n_local - n_sink + 1)
    n_att = min(c + 1, K + n_sink + n_local)
    G = Hq // Hkv
    per = n_cand * D * elem + n_att * 64 * D * elem * 2 + 2 * G * D * elem
    return per * B * Hkv


def profiled_traffic(summary, key):
    """HBM bytes per launch from a committed rocprofv3 counter summary under profiles/, or None
    if there is none or the kernel sources changed since the counters were taken."""
    try:
        text = open(os.path.join(ROOT, "profiles", summary)).read()
        val = int(re.search(key + r": (\d+)", text).group(1))
        for src, sha in re.findall(r"kernel_source(?:_\d+)?: (\S+)\s+kernel_source(?:_\d+)?_sha256_16: (\w+)",
                                   text):
            cur = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()[:16]
            if cur != sha:
                return None
        return val
    except (OSError, AttributeError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-lsa", action="store_true")
    ap.add_argument("--no-hils", action="store_true", help="skip the HiLS workload at 1M tokens")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip measuring the bf16 MFMA and 16 KB gather ceilings")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stat(xs, kind):
    xs = sorted(xs)
    if kind == "median":
        n = len(xs)
        return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    raise ValueError(kind)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Events:
    """Pairs of HIP events on the current stream (where libbsa launches its kernels)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def bench_prefill(torch, bsa, synth, name, steps, warmup):
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, T, D, K, mode = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["topk"], w["mode"]
    log(f"[bench] {name}: generating inputs")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, w["dtype"], w["data"], seed=0, device="cuda",
                                 n_centres=w["n_centres"], n_aim=w["n_aim"])
    NB = (T + 63) // 64
    NA = K + 3
    lm = torch.empty((B, Hkv, NB, D), dtype=q.dtype, device="cuda")
    idx = torch.empty((B, Hkv, NB, NA), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hkv, NB, NA), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    p = bsa.make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=T, seq_k=T, dtype=q.dtype, topk=K)
    ws = torch.empty(max(bsa.select_workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
    ev_attn, ev_sel, ev_pool = Events(torch), Events(torch), Events(torch)

    def step(record):
        if record:
            ev_pool.start()
        bsa.pool_landmarks(k, out=lm)
        if record:
            ev_pool.stop()
            ev_sel.start()
        bsa.select_topk(q, lm, topk=K, ws=ws, idx=idx, sc=sc)
        if record:
            ev_sel.stop()
            ev_attn.start()
        bsa.attend_prefill(q, k, v, idx, sc, lm if mode == "hils" else None, mode=mode, topk=K,
                           out=out)
        if record:
            ev_attn.stop()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] {name}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flops = attended_flops(B, Hq, D, T, K)
    attn = ev_attn.ms()
    attn_ms = sum(attn) / steps
    # the same steps once more, each after a 1 GiB read that evicts L2 and the memory-side
    # cache (outside the timed region above), timed step by step with HIP events
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    ev_attn.pairs, ev_sel.pairs, ev_pool.pairs = [], [], []
    for _ in range(steps):
        flush.sum()
        step(True)
    torch.cuda.synchronize()
    del flush
    f_attn = ev_attn.ms()
    f_step = [a + b + c for a, b, c in zip(ev_pool.ms(), ev_sel.ms(), f_attn)]
    res = {
        "ms_per_step": wall * 1e3 / steps,
        "tok_per_s": B * T * steps / wall,
        "attn_ms": attn_ms,
        "attn_ms_median": stat(attn, "median"),
        "attn_ms_min": min(attn),
        "select_ms": sum(ev_sel.ms()) / steps,
        "pool_ms": sum(ev_pool.ms()) / steps,
        "attended_flops": flops,
        "attended_tflops_kernel": flops / (attn_ms * 1e-3) / 1e12,
        "attended_tflops_e2e": flops * steps / wall / 1e12,
        "flushed": {"step_ms_median": stat(f_step, "median"), "step_ms_min": min(f_step),
                    "attend_ms_median": stat(f_attn, "median"), "attend_ms_min": min(f_attn),
                    "how": "each step after a 1 GiB read that evicts L2 and the memory-side "
                           "cache; pool + select + attend summed from HIP events"},
    }
    log(f"[bench] {name}: {json.dumps(res)}")
    tensors = (q, k, v, lm, idx, sc, out, ws)
    return res, tensors


def bench_backward(torch, bsa, synth, name, tensors, steps, warmup, mode=None):
    """The backward of the prefill (dq, dk, dv, and the score or landmark gradient) on the
    forward's own outputs; mode defaults to the workload's."""
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, T, D, K = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["topk"]
    mode = mode or w["mode"]
    q, k, v, lm, idx, sc = tensors[:6]
    out, lse = bsa.attend_prefill(q, k, v, idx, sc, lm if mode == "hils" else None, mode=mode,
                                  topk=K, want_lse=(mode != "hils"))
    g = torch.Generator(device="cuda").manual_seed(5)
    dout = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(q.dtype)
    p = bsa.make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=T, seq_k=T, dtype=q.dtype, topk=K,
                        mode=mode)
    ws = torch.empty(bsa.backward_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsc = torch.empty(idx.shape, dtype=torch.float32, device="cuda")
    dlm = torch.empty(lm.shape, dtype=torch.float32, device="cuda") if mode == "hils" else None
    ev = Events(torch)

    def step(record):
        if record:
            ev.start()
        bsa.attend_prefill_backward(q, k, v, idx, sc, out, lse, dout, mode=mode,
                                    lm=lm if mode == "hils" else None, topk=K, ws=ws, dq=dq,
                                    dk=dk, dv=dv, dsc=dsc, dlm=dlm)
        if record:
            ev.stop()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] backward {name}: timing {steps} calls")
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    ms = sum(ev.ms()) / steps
    flops = attended_flops(B, Hq, D, T, K) // 4 * 10
    tf = flops / (ms * 1e-3) / 1e12
    what = ("HiLS prefill on the same shape and attended sets (dq, dk, dv, landmark gradient)"
            if mode == "hils" else "SAS prefill (dq, dk, dv, selector-score gradient) given the "
            "forward's out and lse")
    res = {"workload": f"{name}: backward of the {what}",
           "ms_per_call": ms, "tok_per_s": B * T / (ms * 1e-3),
           "algorithmic_flops": flops,
           "flops_definition": "10*D per visible (query, key) pair per query head: "
                               "recomputed S, dP, dQ, dK, dV (2*D each)",
           "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                        "traffic": profiled_traffic("attend_backward_sas_bf16_128k.md",
                                                    "traffic_bytes_per_call" if mode == "sas"
                                                    else "traffic_bytes_per_call_hils"),
                        "traffic_unit": "bytes per call (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)",
                        "scope": "whole backward call (all its kernels)"}}
    log(f"[bench] backward: {json.dumps(res)}")
    del ws, dq, dk, dv, dsc, dlm, dout, out, lse
    return res


def bench_lsa(torch, bsa, synth, name, tensors, steps, warmup, seg_blocks=64, n_clusters=16,
              tree=False, fanout=8, beam=8):
    """The prefill step with the clustered index in place of the per-block top-K: pool, Ward
    index build (and, for the tree, its node centres), selection over the index (flat, or beam
    search over the tree), attention; each part timed with HIP events."""
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, T, D, K, mode = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["topk"], w["mode"]
    q, k, v, lm, idx, sc, out = tensors[:7]
    index = bsa.lsa_build_index(lm, seg_blocks=seg_blocks, n_clusters=n_clusters)
    if tree:
        bsa.lsa_build_tree(lm, index, fanout=fanout)
    p = bsa.make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=T, seq_k=T, dtype=q.dtype, topk=K)
    ws = torch.empty(max(bsa.lsa_select_workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
    ev = {n: Events(torch) for n in ("pool", "build", "select", "attend")}
    exact_idx, _ = bsa.select_topk(q, lm, topk=K)  # the per-block top-K, for the agreement figure

    def step(record):
        def timed(n, fn):
            if record:
                ev[n].start()
            fn()
            if record:
                ev[n].stop()
        timed("pool", lambda: bsa.pool_landmarks(k, out=lm))
        def build():
            bsa.lsa_build_index(lm, seg_blocks=seg_blocks, n_clusters=n_clusters)
            if tree:
                bsa.lsa_build_tree(lm, index, fanout=fanout)

        def select():
            if tree:
                bsa.lsa_tree_select(q, lm, index, topk=K, beam=beam, ws=ws, idx=idx, sc=sc)
            else:
                bsa.lsa_select(q, lm, index, topk=K, ws=ws, idx=idx, sc=sc)
        timed("build", build)
        timed("select", select)
        timed("attend", lambda: bsa.attend_prefill(q, k, v, idx, sc,
                                                   lm if mode == "hils" else None, mode=mode,
                                                   topk=K, out=out))

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] lsa {name}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {n: sum(e.ms()) / steps for n, e in ev.items()}
    NB = (T + 63) // 64
    NS = NB // seg_blocks
    if tree:
        scored = (NS // fanout + fanout) + beam * fanout + beam * n_clusters + beam + seg_blocks
        what = (f"the tree index (groups of {fanout} segments, beam {beam}) over {NS} segments of "
                f"{seg_blocks} landmarks x {n_clusters} Ward clusters per kv group; a query block "
                f"scores at most {scored} nodes and units instead of {NB} landmarks")
    else:
        what = (f"the flat clustered index: {NS} segments of {seg_blocks} landmarks x "
                f"{n_clusters} Ward clusters per kv group; a query block scores at most "
                f"{NS * n_clusters + seg_blocks} units instead of {NB} landmarks")
    # rows past the first K + 3 blocks choose exactly K candidates (after the one sink block):
    # the share of the exact top-K's blocks that the index chooses too, over 512 spread rows
    rows = torch.linspace(K + 3, NB - 1, 512, device="cuda").long().unique()
    a = exact_idx[:, :, rows, 1:1 + K]
    b = idx[:, :, rows, 1:1 + K]
    agree = (a.unsqueeze(-1) == b.unsqueeze(-2)).any(-1).float().mean().item()
    res = {"workload": f"{name} with {what}",
           "tok_per_s": B * T * steps / wall, "ms_per_step": wall * 1e3 / steps,
           "breakdown_ms": ms,
           "agreement_with_exact_topk": {
               "value": agree, "rows": int(rows.numel()) * B * Hkv,
               "what": "share of the blocks the per-block top-K chooses that the index chooses "
                       "too (synthetic keys: each block drawn round its own random centre, so "
                       "a cluster's centre averages unrelated blocks)"}}
    del exact_idx
    log(f"[bench] lsa: {json.dumps(res)}")
    return res


def bench_decode(torch, bsa, synth, steps, warmup):
    w = synth.WORKLOADS["decode_bf16_32x128k"]
    B, Hq, Hkv, Tk, D, K = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["topk"]
    log("[bench] decode: generating inputs")
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, w["dtype"], w["data"], seed=0, device="cuda",
                                  n_centres=w["n_centres"], n_aim=w["n_aim"])
    q = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks(kc)                  # cache-fill time, not timed
    NA = K + 3
    idx = torch.empty((B, Hkv, 1, NA), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hkv, 1, NA), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    p = bsa.make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=Tk, dtype=q.dtype, topk=K)
    ws_sel = torch.empty(bsa.select_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ws_dec = torch.empty(bsa.decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ws_step = torch.empty(max(256, bsa.decode_step_workspace_bytes(p)), dtype=torch.uint8,
                          device="cuda")
    # evicting the caches with a read leaves them full of clean lines; a write would leave dirty
    # lines whose write-back the timed step would then pay for
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    ev_step, ev_two, ev_attn = Events(torch), Events(torch), Events(torch)

    def step(record):                            # one call: selection + attention fused
        if record:
            ev_step.start()
        bsa.decode_step(q, kc, vc, lm, topk=K, idx=idx, sc=sc, out=out, ws=ws_step)
        if record:
            ev_step.stop()

    def two_calls(record):                       # the selection call, then the attention call
        if record:
            ev_two.start()
        bsa.select_topk(q, lm, topk=K, seq_k=Tk, ws=ws_sel, idx=idx, sc=sc)
        if record:
            ev_attn.start()
        bsa.attend_decode(q, kc, vc, idx, sc, None, mode="plain", topk=K, out=out, ws=ws_dec)
        if record:
            ev_attn.stop()
            ev_two.pairs[-1][1] = ev_attn.pairs[-1][1]

    for fn in (step, two_calls):
        for _ in range(warmup):
            fn(False)
        for _ in range(steps):
            flush.sum()                          # evict L2 and the MALL between steps
            fn(True)
    torch.cuda.synchronize()
    nbytes = decode_bytes(B, Hq, Hkv, Tk, D, K)
    step_us = 1e3 * sum(ev_step.ms()) / steps
    two_us = 1e3 * sum(ev_two.ms()) / steps
    attn_us = 1e3 * sum(ev_attn.ms()) / steps
    med_us = 1e3 * stat(ev_step.ms(), "median")
    res = {"us_per_step": step_us, "us_per_step_median": med_us,
           "us_per_step_min": 1e3 * min(ev_step.ms()), "two_call_us_per_step": two_us,
           "two_call_breakdown_us": {"select": two_us - attn_us, "attend": attn_us},
           "algorithmic_bytes": nbytes, "hbm_gbps": nbytes / (med_us * 1e-6) / 1e9,
           "hbm_gbps_mean": nbytes / (step_us * 1e-6) / 1e9}
    res["hbm_frac"] = res["hbm_gbps"] / PEAK_HBM_GBPS
    log(f"[bench] decode: {json.dumps(res)}")
    del q, kc, vc, lm, flush
    return res


def bench_decode_paged(torch, bsa, synth, steps, warmup):
    """Ragged batch in a paged cache: one paged decode step call (fused selection + attention)
    per step; the paged selection and attention calls one after the other for comparison."""
    import numpy as np
    name = "decode_paged_bf16_32x16k_128k"
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, D, K = w["B"], w["Hq"], w["Hkv"], w["D"], w["topk"]
    lens = np.random.default_rng(11).integers(w["T_min"], w["T"] + 1, size=B).tolist()
    log(f"[bench] decode paged: generating inputs ({sum(lens)} cached tokens)")
    q, k_pool, v_pool, table, seq_lens = synth.make_paged_decode(
        lens, Hq, Hkv, D, w["dtype"], w["data"], seed=0, device="cuda",
        n_centres=w["n_centres"], n_aim=w["n_aim"])
    q = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks_paged(k_pool, table, seq_lens)     # cache-fill time, not timed
    NB = table.shape[1]
    NA = K + 3
    idx = torch.empty((B, Hkv, 1, NA), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hkv, 1, NA), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    p = bsa.make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=NB * 64, dtype=q.dtype, topk=K)
    ws_dec = torch.empty(max(256, bsa.decode_workspace_bytes(p)), dtype=torch.uint8, device="cuda")
    ws_step = torch.empty(max(256, bsa.decode_step_workspace_bytes(p)), dtype=torch.uint8,
                          device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    ev_step, ev_two, ev_attn = Events(torch), Events(torch), Events(torch)

    def step(record):
        if record:
            ev_step.start()
        bsa.decode_step_paged(q, k_pool, v_pool, table, seq_lens, lm, topk=K, idx=idx, sc=sc,
                              out=out, ws=ws_step)
        if record:
            ev_step.stop()

    def two_calls(record):
        if record:
            ev_two.start()
        bsa.select_topk_paged(q, lm, seq_lens, topk=K, idx=idx, sc=sc)
        if record:
            ev_attn.start()
        bsa.attend_decode_paged(q, k_pool, v_pool, table, seq_lens, idx, sc, None, mode="plain",
                                topk=K, out=out, ws=ws_dec)
        if record:
            ev_attn.stop()
            ev_two.pairs[-1][1] = ev_attn.pairs[-1][1]

    ev_ref, ev_refresh = Events(torch), Events(torch)

    def step_with_refresh(record):
        # a decode loop's step: the landmark of each sequence's newest token's block is
        # refreshed (one block per sequence and kv head), then selection and attention
        if record:
            ev_ref.start()
        bsa.update_landmarks_paged(k_pool, table, seq_lens, lm, 1)
        if record:
            ev_refresh.start()
            ev_refresh.stop()
        bsa.decode_step_paged(q, k_pool, v_pool, table, seq_lens, lm, topk=K, idx=idx, sc=sc,
                              out=out, ws=ws_step)
        if record:
            ev_ref.stop()
            ev_refresh.pairs[-1][0] = ev_ref.pairs[-1][0]

    for fn in (step, two_calls, step_with_refresh):
        for _ in range(warmup):
            fn(False)
        for _ in range(steps):
            flush.sum()
            fn(True)
    torch.cuda.synchronize()
    nbytes = sum(decode_bytes(1, Hq, Hkv, L, D, K) for L in lens)
    step_us = 1e3 * sum(ev_step.ms()) / steps
    two_us = 1e3 * sum(ev_two.ms()) / steps
    attn_us = 1e3 * sum(ev_attn.ms()) / steps
    res = {"workload": f"{name}: {B} seqs of {min(lens)}..{max(lens)} cached tokens (seeded "
                       f"uniform), shuffled 64-token pages, Hq={Hq}, Hkv={Hkv}, D={D}, "
                       f"top-K={K} + sink + 2 local, bf16",
           "us_per_step": step_us, "us_per_step_median": 1e3 * stat(ev_step.ms(), "median"),
           "us_per_step_min": 1e3 * min(ev_step.ms()), "two_call_us_per_step": two_us,
           "two_call_breakdown_us": {"select": two_us - attn_us, "attend": attn_us},
           "hbm_gbps": nbytes / (stat(ev_step.ms(), "median") * 1e-3) / 1e9,
           "hbm_gbps_mean": nbytes / (step_us * 1e-6) / 1e9,
           "with_landmark_refresh": {
               "us_per_step": 1e3 * sum(ev_ref.ms()) / steps,
               "refresh_us": 1e3 * sum(ev_refresh.ms()) / steps,
               "what": "bsa_update_landmarks_paged (n_new = 1: the newest token's block of every "
                       "sequence and kv head) then the one-launch paged step; re-pooling the whole "
                       "cache instead is bsa_pool_landmarks_paged"}}
    res["roofline"] = {"bound": "hbm", "achieved": res["hbm_gbps"], "peak": PEAK_HBM_GBPS,
                       "unit": "GB/s", "frac": res["hbm_gbps"] / PEAK_HBM_GBPS,
                       "achieved_from": "median of the flushed steps (HIP events)",
                       "algorithmic_bytes": nbytes,
                       "traffic": profiled_traffic("decode_paged_bf16_32x16k_128k.md",
                                                   "traffic_bytes_per_step")}
    log(f"[bench] decode paged: {json.dumps(res)}")
    del q, k_pool, v_pool, table, seq_lens, lm, flush
    return res


def cpu_baseline(torch, tensors, name, synth, budget_s=12.0):
    """The float64 oracle on a sample of the prefill workload, extrapolated to tok/s."""
    import numpy as np
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)     # BLAS threads = every core of this process
    except Exception:  # noqa: BLE001
        limiter = None
    try:
        return _cpu_baseline(torch, tensors, name, synth, budget_s, cores, np, O)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()


def _cpu_baseline(torch, tensors, name, synth, budget_s, cores, np, O):
    w = synth.WORKLOADS[name]
    q, k, v = tensors[:3]
    B, Hq, Hkv, T, D, K = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["topk"]
    G = Hq // Hkv
    NQB = (T + 63) // 64
    h = lambda t: t.float().cpu().numpy().astype(np.float64)
    K64, V64 = h(k[0, 0]), h(v[0, 0])
    rng = np.random.default_rng(7)
    t0 = time.perf_counter()
    lm = O.landmarks(K64[None, None], w["dtype"])[0, 0]
    t_lm = time.perf_counter() - t0
    n_rows, t_rows = 0, 0.0
    scale = 1 / math.sqrt(D)
    while t_rows < budget_s and n_rows < 4096:
        c = int(rng.integers(NQB))
        qs = h(q[0, 0:G, c * 64:(c + 1) * 64])
        t1 = time.perf_counter()
        qbar = O.selector_vectors(qs[None], 1)[0, 0, 0]
        s_row = O.block_scores(qbar[None], lm)[0]
        A, sA = O.select_row(s_row, c, K)
        gates = O.sas_gates(A, sA, c) if w["mode"] == "sas" else np.zeros(A.size)
        tpos = np.arange(c * 64, c * 64 + 64)
        for hh in range(G):
            O.attend_rows(qs[hh], tpos, K64, V64, A, gates, scale)
        t_rows += time.perf_counter() - t1
        n_rows += 1
    per_step = B * Hkv * (t_lm + t_rows / n_rows * NQB)
    return {"value": B * T / per_step, "unit": "tok/s", "cores": cores, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": (f"kv group 0 of {name}: its landmarks plus {n_rows} random query blocks "
                       f"(all {G} heads x 64 tokens: scores, top-K, gates, attention) in "
                       f"{t_lm + t_rows:.1f} s; extrapolated linearly to {B * Hkv} groups x "
                       f"{NQB} query blocks"),
            "seconds_per_step_extrapolated": per_step}


def measured_peaks(torch):
    """Ceilings of this GPU measured with the probes of libbsa_peak.so: back-to-back 32x32x16 bf16
    MFMAs on every SIMD (TFLOP/s), and random 16 KB blocks of a 4 GiB buffer gathered straight
    into LDS (GB/s, read bytes).  Best of 3 timed launches each, HIP events on the launch stream."""
    import ctypes
    from block_sparse_attention_landmark_amd import build as B
    if not os.path.exists(B.PEAK_LIB):
        raise RuntimeError(f"{B.PEAK_LIB} is missing; build the package first")
    lib = ctypes.CDLL(B.PEAK_LIB)
    lib.bsa_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.bsa_peak_mfma.restype = ctypes.c_int
    lib.bsa_peak_gather.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.bsa_peak_gather.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def best_ms(launch, reps=3):
        launch()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    n_wg, iters = 1024, 4000                      # 4 workgroups of 4 waves per CU
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")

    def mfma():
        if lib.bsa_peak_mfma(ctypes.c_void_p(out.data_ptr()), n_wg, iters, stream) != 0:
            raise RuntimeError("bsa_peak_mfma failed")
    ms = best_ms(mfma)
    mfma_tflops = n_wg * 4 * iters * 16 * 32768 / (ms * 1e-3) / 1e12
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    n_blocks = src.numel() // 16384
    g_wg, bpw = 256, 512                          # 256 x 4 waves x 512 blocks x 16 KB = 8 GiB
    outg = torch.empty(g_wg * 256, dtype=torch.int32, device="cuda")

    def gather():
        if lib.bsa_peak_gather(ctypes.c_void_p(src.data_ptr()), n_blocks, g_wg, bpw,
                               ctypes.c_void_p(outg.data_ptr()), stream) != 0:
            raise RuntimeError("bsa_peak_gather failed")
    ms_g = best_ms(gather)
    gather_gbps = g_wg * 4 * bpw * 16384 / (ms_g * 1e-3) / 1e9
    del src, out, outg
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": mfma_tflops, "gather_16k_gbps": gather_gbps,
            "how": "libbsa_peak.so: 1024 workgroups x 4 waves of back-to-back 32x32x16 bf16 MFMAs; "
                   "256 workgroups x 4 waves gathering random 16 KB blocks of a 4 GiB buffer "
                   "into LDS (8 GiB read); best of 3 launches"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is "
              "not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_attention_landmark_amd as bsa
    from block_sparse_attention_landmark_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    bsa.load_library()

    name = "sas_bf16_128k"
    pre, tensors = bench_prefill(torch, bsa, synth, name, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores")
        cpu = cpu_baseline(torch, tensors, name, synth)
        log(f"[bench] cpu baseline: {cpu['value']:.1f} tok/s")
    lsa = lsa_tree = None
    if not args.no_lsa:
        lsa = bench_lsa(torch, bsa, synth, name, tensors, max(3, args.steps // 2), 1)
        lsa_tree = bench_lsa(torch, bsa, synth, name, tensors, max(3, args.steps // 2), 1,
                             tree=True)
        torch.cuda.empty_cache()
    bwd = bwd_hils = None
    if not args.no_backward:
        bwd = bench_backward(torch, bsa, synth, name, tensors, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
        bwd_hils = bench_backward(torch, bsa, synth, name, tensors, max(3, args.steps // 4), 1,
                                  mode="hils")
    del tensors
    torch.cuda.empty_cache()
    dec = None
    if not args.no_decode:
        dec = bench_decode(torch, bsa, synth, args.steps, args.warmup)
        torch.cuda.empty_cache()
    dec_paged = None
    if not args.no_decode:
        dec_paged = bench_decode_paged(torch, bsa, synth, args.steps, args.warmup)
        torch.cuda.empty_cache()
    hils = lsa_1m = lsa_tree_1m = None
    if not args.no_hils:
        hils, t = bench_prefill(torch, bsa, synth, "hils_bf16_1m", max(2, args.steps // 4), 1)
        if not args.no_lsa:
            # the clustered indexes where the pages motivate them: the scan over every landmark
            # grows with the context (16384 landmarks per query block at 1M tokens)
            lsa_1m = bench_lsa(torch, bsa, synth, "hils_bf16_1m", t, max(2, args.steps // 4), 1)
            lsa_tree_1m = bench_lsa(torch, bsa, synth, "hils_bf16_1m", t,
                                    max(2, args.steps // 4), 1, tree=True)
        del t
        torch.cuda.empty_cache()
    peaks = None
    if not args.no_peak_probe:
        peaks = measured_peaks(torch)
        log(f"[bench] measured ceilings: {peaks['mfma_bf16_tflops']:.0f} TFLOP/s bf16 MFMA, "
            f"{peaks['gather_16k_gbps']:.0f} GB/s 16 KB gathers")
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    w = synth.WORKLOADS[name]
    line = {
        "metric": METRIC,
        "value": pre["tok_per_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (clustered keys, aimed queries; seeded)",
        "config": {"workload": f"{name}: SAS-gated block-sparse prefill, B={w['B']}, "
                               f"Hq={w['Hq']}, Hkv={w['Hkv']}, D={w['D']}, T={w['T']}, block=64, "
                               f"top-K={w['topk']} + sink + 2 local",
                   "step": "pool + select (selector, scores, top-K) + attend"},
        "attended_tflops": pre["attended_tflops_e2e"],
        "attended_tflops_attention_kernel": pre["attended_tflops_kernel"],
        "breakdown_ms": {"pool": pre["pool_ms"], "select": pre["select_ms"],
                         "attend": pre["attn_ms"]},
        "attend_ms_median": pre["attn_ms_median"],
        "attend_ms_min": pre["attn_ms_min"],
        "flushed": pre["flushed"],
        "roofline": {"bound": "mfma", "achieved": pre["attended_tflops_kernel"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": pre["attended_tflops_kernel"] / PEAK_BF16_TFLOPS,
                     "traffic": profiled_traffic("attend_prefill_sas_bf16_128k.md",
                                                 "traffic_bytes_per_launch"),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)",
                     "kernel": "attend_prefill_pp_kernel<128, SAS>"},
    }
    if dec is not None:
        line["decode"] = {
            "workload": "decode_bf16_32x128k: 32 seqs x 131072 cached tokens, Hq=64, Hkv=8, "
                        "D=128, top-K=64 + sink + 2 local, bf16",
            "step": "one decode step call: selection and attention in one fused kernel",
            "hbm_gbps": dec["hbm_gbps"], "us_per_step": dec["us_per_step"],
            "us_per_step_median": dec["us_per_step_median"],
            "us_per_step_min": dec["us_per_step_min"],
            "two_call_us_per_step": dec["two_call_us_per_step"],
            "two_call_breakdown_us": dec["two_call_breakdown_us"],
            "hbm_gbps_mean_step": dec["hbm_gbps_mean"],
            "roofline": {"bound": "hbm", "achieved": dec["hbm_gbps"], "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": dec["hbm_frac"],
                         "achieved_from": "median of the flushed steps (HIP events)",
                         "algorithmic_bytes": dec["algorithmic_bytes"],
                         "traffic": profiled_traffic("decode_bf16_32x128k.md",
                                                     "traffic_bytes_per_step")}}
    if dec_paged is not None:
        line["decode_paged"] = dec_paged
    if lsa is not None:
        line["lsa_prefill"] = lsa
    if lsa_tree is not None:
        line["lsa_tree_prefill"] = lsa_tree
    if bwd is not None:
        line["backward"] = bwd
    if bwd_hils is not None:
        line["backward_hils"] = bwd_hils
    if hils is not None:
        line["hils_1m"] = {"workload": "hils_bf16_1m: HiLS prefill, B=1, Hq=32, Hkv=8, D=128, "
                                       "T=1048576, top-K=32 + sink + 2 local, per-chunk softmax "
                                       "merged by softmax(q.L/sqrt(D))",
                           "tok_per_s": hils["tok_per_s"], "ms_per_step": hils["ms_per_step"],
                           "breakdown_ms": {"pool": hils["pool_ms"], "select": hils["select_ms"],
                                            "attend": hils["attn_ms"]},
                           "select_path": "one-pass kernel (selector vectors, scores and top-K of "
                                          "each tile row in one launch; no score workspace)",
                           "attended_tflops_attention_kernel": hils["attended_tflops_kernel"],
                           "frac_of_bf16_peak": hils["attended_tflops_kernel"] / PEAK_BF16_TFLOPS}
    if lsa_1m is not None:
        line["lsa_prefill_1m"] = dict(lsa_1m, scan_select_ms=hils["select_ms"])
    if lsa_tree_1m is not None:
        line["lsa_tree_prefill_1m"] = dict(lsa_tree_1m, scan_select_ms=hils["select_ms"])
    if peaks is not None:
        # the same achieved rates against the ceilings measured on this GPU in this run
        line["measured_peaks"] = peaks
        line["roofline"]["frac_of_measured"] = \
            line["roofline"]["achieved"] / peaks["mfma_bf16_tflops"]
        for key in ("decode", "decode_paged"):
            if key in line:
                r = line[key]["roofline"]
                r["frac_of_measured"] = r["achieved"] / peaks["gather_16k_gbps"]
        for key in ("backward", "backward_hils"):
            if key in line and "roofline" in line[key]:
                r = line[key]["roofline"]
                r["frac_of_measured"] = r["achieved"] / peaks["mfma_bf16_tflops"]
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
