#!/usr/bin/env python3
"""Benchmark of the Flash-LoRA-Attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-mixed] [--no-cpu-baseline]

Headline (the JSON line's `value`): bf16 Flash-LoRA-Attention prefill throughput in
TFLOP/s (algorithmic FLOP) on the Llama-3-8B-shaped single-layer workload: 1024 new causal
queries after an 8192-token shared context (9216 keys), 32 q / 8 kv heads, head_dim 128,
LoRA rank 16, agent 0 of 3.  A step is one lra_attn_prefill call on it; K steps are timed
back to back between device synchronisations.

Also reported, each timed on its own (HIP events around every call, the 256 MB MALL
flushed between calls of the HBM-bound ones):
  tiny_fp32   16 queries over 256 keys, 4 heads, head_dim 64, 2 agents of rank 8, fp32
              (latency only)
  decode      64 requests x 16384 keys, one query each, rank 16, 4 agents  (HBM GB/s)
  decode_shared  16 contexts x 16384 keys, each read by all 4 agents (rank 16):
              64 requests whose K/V tiles are streamed once per context (HBM GB/s,
              shared rows counted once), also timed with grouping switched off
  append      decode-step LR append: 64 new tokens x 4096 into 4 rank-16 caches (HBM GB/s)
  precompute  L = X·[A_1..A_3], X [32768, 4096], ranks 3 x 64              (HBM GB/s)
  longctx     512 queries over 32768 keys, rank 64, L from the precompute   (TFLOP/s)
  naive_expansion  the regrouped kernels beside the naive route (V_full = V_base + L·B
              materialised, then plain attention) and the in-tile expansion route, on the
              Llama prefill, the decode batch and the long-context prefill
  mixed       32 layers of a 32-request batch, ranks 8/16/32/64 (--no-mixed skips it)
and the CPU fp64 oracle timed on a bounded sample of the headline workload.

Prints ONE JSON line on stdout.  Inputs are seeded synthetic tensors resident in HBM
before timing starts.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import shutil
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Flash-LoRA-Attn prefill TFLOP/s + decode HBM GB/s (% of MI355X roofline)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


class Flusher:
    """Evicts the 256 MB Infinity Cache (MALL) by reading a 512 MB buffer.  A read leaves
    clean lines behind; a write-based flush would leave dirty lines whose write-backs
    then compete with the timed kernel's reads."""

    def __init__(self):
        import torch
        self.buf = torch.ones(64 << 20, dtype=torch.int64, device="cuda")

    def __call__(self):
        self.buf.sum()


def settle(fn, seconds=0.5):
    """Runs fn back to back for about `seconds` of wall time before anything is timed.  The
    headline is the first workload a fresh process runs, and an idle GPU takes some
    milliseconds of load to reach its working clock; the W warm-up steps alone (about 1 ms
    of work) do not cover that."""
    import torch
    t_end = time.time() + seconds
    while time.time() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def time_calls(fn, steps, warmup, flush=None):
    """Per-call durations (ms) from HIP events on the current stream, and the total (ms).

    Without a flush the K calls run back to back between two events and every call gets
    total/K: an event recorded between calls costs a cache write-back of its own, which
    would otherwise be charged to the calls.  With a flush (a kernel that evicts the inputs
    from the caches between calls), each call is bracketed by its own pair of events and
    the total is their sum."""
    import torch
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
    torch.cuda.synchronize()
    if flush is None:
        t0, t1 = _events(2)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        total = t0.elapsed_time(t1)
        return np.full(steps, total / steps), total
    st, en = _events(steps), _events(steps)
    for i in range(steps):
        flush()
        st[i].record()
        fn()
        en[i].record()
    torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) for s, e in zip(st, en)])
    return per, float(per.sum())


# HBM bytes per call measured with rocprofv3 FETCH_SIZE and WRITE_SIZE (each calibrated by
# what the same counter reads for a plain 1 GiB device copy); the per-kernel summaries and
# the commands are under profiles/.  The figures describe the kernels built from sources
# with this digest and are reported as null for any other sources.
TRAFFIC_SOURCES_SHA256 = "8a0a8b7a2b4f4913477a2ab1d7e9b7ffe77b95682309a27a0dd836c3c5eaed56"
TRAFFIC_BYTES = {
    "llama8b-prefill-1024q-9216k-r16": 125446549,
    "decode-64x16384-r16": 4418541634,
    "decode-shared-16x4x16384-r16": 1164516375,
    "lr-precompute-32768x4096-3x64": 293973223,
    "lr-append-64x4096-4x16": 1652094,
    "longctx-prefill-512q-32768k-r64": 244838087,
}


def sources_sha256():
    """Digest of the C ABI header and every source liblra.so is built from."""
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "shared_rank_kv_amd", "csrc")
    files = [os.path.join(here, "include", "lra.h")] + sorted(
        os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes(workload):
    if sources_sha256() != TRAFFIC_SOURCES_SHA256:
        return None
    return TRAFFIC_BYTES.get(workload)


def roof(achieved, peak, unit, bound, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def upload(prob, L=None):
    cpu = {"Q": prob.Q(), "K": prob.K(), "V": prob.V()}
    dev = {k: v.cuda() for k, v in cpu.items()}
    dev["L"] = L if L is not None else [prob.L(a).cuda() if prob.ranks[a] else None
                                        for a in range(prob.n_agents)]
    dev["B"] = [prob.B(a).cuda() if prob.ranks[a] else None for a in range(prob.n_agents)]
    return cpu, dev


def prefill_call(prob, dev, ws):
    """The C call with its arguments marshalled once (only the call itself is timed)."""
    from shared_rank_kv_amd import lra
    return lra.prepare_attn_prefill(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                    prob.q_start, prob.q_len, prob.k_start, prob.k_len,
                                    prob.agent_idx, O=torch_empty_like(dev["Q"]), workspace=ws)


def torch_empty_like(t):
    import torch
    return torch.empty_like(t)


def workspace_for(prob, decode):
    import torch
    from shared_rank_kv_amd import lra
    n = lra.lra_attn_workspace_bytes(torch.bfloat16 if prob.dtype == "bf16" else torch.float32,
                                     decode, None if decode else prob.q_len, prob.k_len,
                                     prob.n_q_heads, prob.n_kv_heads, prob.head_dim,
                                     max(prob.ranks))
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda") if n else None


def bench_llama_prefill(steps, warmup):
    from shared_rank_kv_amd import accounting, workloads
    prob = workloads.llama_prefill(agents=(0,))
    cpu, dev = upload(prob)
    ws = workspace_for(prob, False)
    fn = prefill_call(prob, dev, ws)
    settle(fn)
    per, total = time_calls(fn, steps, warmup)
    flop, nbytes = accounting.attention_work(prob)
    return prob, cpu, dev, {"flop": flop, "bytes": nbytes, "per_ms": per, "total_ms": total}


def bench_tiny_fp32(steps, warmup):
    """The tiny fp32 workload (both agents in one call): launch- and latency-bound, so the
    time is reported with neither roofline."""
    from shared_rank_kv_amd import accounting, workloads
    prob = workloads.tiny_fp32()
    _, dev = upload(prob)
    fn = prefill_call(prob, dev, workspace_for(prob, False))
    per, _ = time_calls(fn, max(steps, 100), warmup)
    flop, nbytes = accounting.attention_work(prob)
    us = float(np.median(per)) * 1e3
    return {"workload": prob.name, "dtype": "f32", "us_per_call": round(us, 2), "flop": flop,
            "bytes": nbytes, "bound": "latency (launch of one small kernel)"}


def bench_decode(steps, warmup, flush):
    from shared_rank_kv_amd import accounting, lra, workloads
    prob = workloads.decode_batch()
    t = time.time()
    cpu, dev = upload(prob)
    log(f"[bench] decode inputs ready in {time.time() - t:.1f}s")
    ws = workspace_for(prob, True)
    fn = lra.prepare_attn_decode(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"], prob.k_start,
                                 prob.k_len, prob.agent_idx, O=torch_empty_like(dev["Q"]),
                                 workspace=ws)
    per, _ = time_calls(fn, steps, warmup, flush)
    flop, nbytes = accounting.attention_work(prob)
    del dev, cpu
    ms = float(np.median(per))
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": prob.name, "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_call": round(ms, 4), "ms_min": round(float(per.min()), 4),
            "ms_max": round(float(per.max()), 4), "bytes": nbytes, "flop": flop,
            "roofline": roof(gbs, accounting.PEAK_HBM_GBS, "GB/s", "hbm", traffic_bytes(prob.name))}


def bench_decode_shared(steps, warmup, flush):
    from shared_rank_kv_amd import accounting, lra, workloads
    prob = workloads.decode_shared_batch()
    t = time.time()
    cpu, dev = upload(prob)
    log(f"[bench] shared-context decode inputs ready in {time.time() - t:.1f}s")
    ws = workspace_for(prob, True)
    fn = lra.prepare_attn_decode(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"], prob.k_start,
                                 prob.k_len, prob.agent_idx, O=torch_empty_like(dev["Q"]),
                                 workspace=ws)
    per, _ = time_calls(fn, steps, warmup, flush)
    # the same calls with one work item per request (each request streams its context)
    os.environ["LRA_DECODE_GROUP"] = "0"
    try:
        per1, _ = time_calls(fn, steps, warmup, flush)
    finally:
        del os.environ["LRA_DECODE_GROUP"]
    flop, nbytes = accounting.attention_work(prob)
    del dev, cpu
    ms, ms1 = float(np.median(per)), float(np.median(per1))
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": prob.name, "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_call": round(ms, 4), "ms_min": round(float(per.min()), 4),
            "ms_max": round(float(per.max()), 4), "bytes": nbytes, "flop": flop,
            "ungrouped_ms_per_call": round(ms1, 4), "speedup_vs_ungrouped": round(ms1 / ms, 2),
            # analytic KV-cache bytes of the batch's 16 contexts over 32 layers, per scheme
            "cache_GB_32_layers": {k: round(16 * v / 1e9, 3) for k, v in accounting.cache_memory(
                16384, prob.ranks, prob.n_kv_heads, prob.head_dim, 32).items()},
            "roofline": roof(gbs, accounting.PEAK_HBM_GBS, "GB/s", "hbm", traffic_bytes(prob.name))}


def bench_append(steps, warmup, flush):
    import torch
    from shared_rank_kv_amd import accounting, lra, workloads
    p = workloads.decode_append()
    X = p.X().cuda()
    A_cat = torch.cat([p.A(a) for a in range(len(p.ranks))], 1).contiguous().cuda()
    l_rows = 64 * 16384
    Ls = [torch.zeros(l_rows, r, dtype=torch.bfloat16, device="cuda") for r in p.ranks]
    rows = np.arange(64) * 16384 + 16383
    fn = lra.prepare_append_lr(X, A_cat, p.ranks, Ls, rows)
    per, _ = time_calls(fn, steps, warmup, flush)
    flop, nbytes = accounting.append_work(p)
    del Ls
    ms = float(np.median(per))
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": p.name, "value": round(gbs, 1), "unit": "GB/s",
            "us_per_call": round(ms * 1e3, 2), "us_min": round(float(per.min()) * 1e3, 2),
            "bytes": nbytes, "flop": flop,
            "roofline": roof(gbs, accounting.PEAK_HBM_GBS, "GB/s", "hbm", traffic_bytes(p.name))}


def bench_longctx(steps, warmup, flush):
    import torch
    from shared_rank_kv_amd import accounting, lra, workloads
    pre = workloads.longctx_precompute()
    X = pre.X().cuda()
    A_cat = torch.cat([pre.A(a) for a in range(3)], 1).contiguous().cuda()
    Ls = [torch.empty(pre.T, r, dtype=torch.bfloat16, device="cuda") for r in pre.ranks]

    pfn = lra.prepare_precompute_lr(X, A_cat, pre.ranks, Ls)
    per, _ = time_calls(pfn, steps, warmup, flush)
    pflop, pbytes = accounting.precompute_work(pre)
    pms = float(np.median(per))
    pgbs = pbytes / (pms * 1e-3) / 1e9
    precompute = {"workload": pre.name, "value": round(pgbs, 1), "unit": "GB/s",
                  "tflops": round(pflop / (pms * 1e-3) / 1e12, 1), "ms_per_call": round(pms, 4),
                  "ms_min": round(float(per.min()), 4), "ms_max": round(float(per.max()), 4),
                  "bytes": pbytes, "flop": pflop,
                  "roofline": roof(pgbs, accounting.PEAK_HBM_GBS, "GB/s", "hbm",
                                   traffic_bytes(pre.name))}
    del X, pfn
    prob = workloads.longctx_prefill(agents=(0,))
    _, dev = upload(prob, L=Ls)
    ws = workspace_for(prob, False)
    fn = prefill_call(prob, dev, ws)
    settle(fn)      # the flushed precompute timing leaves the GPU below its working clock
    per, _ = time_calls(fn, steps, warmup)
    flop, nbytes = accounting.attention_work(prob)
    ms = float(np.median(per))
    tf = flop / (ms * 1e-3) / 1e12
    longctx = {"workload": prob.name, "value": round(tf, 1), "unit": "TFLOP/s",
               "ms_per_call": round(ms, 4), "flop": flop, "bytes": nbytes,
               "roofline": roof(tf, accounting.PEAK_BF16_TFLOPS, "TFLOP/s", "mfma",
                                traffic_bytes(prob.name))}
    return precompute, longctx


def bench_naive_expansion(steps, warmup, flush):
    """The regrouped kernels against the two comparators of the regrouping, on the Llama
    prefill, the decode batch and the long-context prefill (its LR caches from the
    precompute): the naive route (lra_expand_values writes V_full = V_base + L·B, then plain
    attention reads it) and the in-tile expansion route (each V tile expanded in LDS before
    P·V).  Compute-bound prefills run back to back; the decode batch is timed with the
    caches flushed before every call.  FLOP and bytes are what each route's LR term adds to
    plain attention (accounting.lr_term_work)."""
    import torch
    from shared_rank_kv_amd import accounting, lra, workloads
    out = {}
    for key in ("llama_prefill", "decode", "longctx_prefill"):
        if key == "llama_prefill":
            prob = workloads.llama_prefill(agents=(0,))
            _, dev = upload(prob)
        elif key == "decode":
            prob = workloads.decode_batch()
            _, dev = upload(prob)
        else:
            pre = workloads.longctx_precompute()
            X = pre.X().cuda()
            A_cat = torch.cat([pre.A(a) for a in range(3)], 1).contiguous().cuda()
            Ls = [torch.empty(pre.T, r, dtype=torch.bfloat16, device="cuda") for r in pre.ranks]
            lra.lra_precompute_lr(X, A_cat, pre.ranks, Ls)
            del X, A_cat
            prob = workloads.longctx_prefill(agents=(0,))
            _, dev = upload(prob, L=Ls)
        decode = key == "decode"
        ws = workspace_for(prob, decode)
        zero = np.zeros(prob.batch, np.int32)
        Vf = torch.empty_like(dev["V"])
        expand = lra.prepare_expand_values(dev["V"], dev["L"], dev["B"], prob.k_start,
                                           prob.k_len, prob.agent_idx, Vf)
        if decode:
            mk = lambda V, L, B, ag, ex=False: lra.prepare_attn_decode(  # noqa: E731
                dev["Q"], dev["K"], V, L, B, prob.k_start, prob.k_len, ag,
                O=torch.empty_like(dev["Q"]), workspace=ws, expand=ex)
        else:
            mk = lambda V, L, B, ag, ex=False: lra.prepare_attn_prefill(  # noqa: E731
                dev["Q"], dev["K"], V, L, B, prob.q_start, prob.q_len, prob.k_start, prob.k_len,
                ag, O=torch.empty_like(dev["Q"]), workspace=ws, expand=ex)
        fla = mk(dev["V"], dev["L"], dev["B"], prob.agent_idx)
        settle(fla)
        plain = mk(Vf, [None], [None], zero)
        intile = mk(dev["V"], dev["L"], dev["B"], prob.agent_idx, True)

        def naive():
            expand()
            plain()
        fl = flush if decode else None
        ms = {}
        for name, fn in (("regrouped", fla), ("naive", naive), ("naive_expand_only", expand),
                         ("naive_attention_only", plain), ("in_tile", intile)):
            per, _ = time_calls(fn, steps, warmup, fl)
            ms[name] = float(np.median(per))
        flop, nbytes = accounting.attention_work(prob)
        work = {r: accounting.lr_term_work(prob, r) for r in ("regrouped", "naive", "in_tile")}
        out[key] = {
            "workload": prob.name, "ms": {k: round(v, 4) for k, v in ms.items()},
            "regrouped_speedup_vs_naive": round(ms["naive"] / ms["regrouped"], 3),
            "regrouped_speedup_vs_in_tile": round(ms["in_tile"] / ms["regrouped"], 3),
            "expand_GBps": round(work["naive"][1] / (ms["naive_expand_only"] * 1e-3) / 1e9, 1),
            "attention_flop": flop, "attention_bytes": nbytes,
            "lr_term_flop": {k: v[0] for k, v in work.items()},
            "lr_term_bytes": {k: v[1] for k, v in work.items()},
        }
        del dev, Vf, expand, fla, plain, intile
        torch.cuda.empty_cache()
    return out


def bench_mixed(steps, warmup):
    import torch
    from shared_rank_kv_amd import accounting, lra, workloads
    layers = []
    t = time.time()
    tflop = tbytes = 0
    req_ms = 0.0
    for layer in range(workloads.MIXED_LAYERS):
        prob = workloads.mixed_batch_layer(layer)
        _, dev = upload(prob)
        dev["ws"] = workspace_for(prob, False)
        dev["O"] = torch.empty_like(dev["Q"])
        f, b = accounting.attention_work(prob)
        tflop += f
        tbytes += b
        # per-request bound: each request on its own at whichever roofline binds it
        req_ms += sum(max(fr / (accounting.PEAK_BF16_TFLOPS * 1e12),
                          br / (accounting.PEAK_HBM_GBS * 1e9))
                      for fr, br in accounting.attention_work_per_request(prob)) * 1e3
        layers.append((prob, dev))
    log(f"[bench] mixed-batch inputs (32 layers) ready in {time.time() - t:.1f}s")

    calls = [lra.prepare_attn_prefill(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                      prob.q_start, prob.q_len, prob.k_start, prob.k_len,
                                      prob.agent_idx, O=dev["O"], workspace=dev["ws"])
             for prob, dev in layers]

    def fn():
        for c in calls:
            c()
    settle(fn, 1.0)
    per, _ = time_calls(fn, max(3, steps // 4), max(1, warmup // 2))
    ms = float(np.median(per))
    ideal_ms = max(tflop / (accounting.PEAK_BF16_TFLOPS * 1e12),
                   tbytes / (accounting.PEAK_HBM_GBS * 1e9)) * 1e3
    del layers, calls
    torch.cuda.empty_cache()
    return {"workload": "mixed32-32req-ranks8-16-32-64", "ms_per_32_layers": round(ms, 3),
            "flop": tflop, "bytes": tbytes, "tflops": round(tflop / (ms * 1e-3) / 1e12, 1),
            "roofline_ms": round(ideal_ms, 3), "frac_of_roofline": round(ideal_ms / ms, 4),
            "per_request_roofline_ms": round(req_ms, 3),
            "frac_of_per_request_roofline": round(req_ms / ms, 4)}


def cpu_baseline(prob, cpu, target_s=10.0):
    """The fp64 oracle on the first n query rows (all heads) of the headline workload,
    n chosen for ~target_s seconds of host time; reported in the headline's unit."""
    import oracle
    from shared_rank_kv_amd import accounting, inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    lk, lq = int(prob.k_len[0]), int(prob.q_len[0])
    Q = inputs.to_f64(cpu["Q"][:lq])
    K = inputs.to_f64(cpu["K"])
    V = inputs.to_f64(cpu["V"])
    L = inputs.to_f64(prob.L(0))
    B = inputs.to_f64(prob.B(0))

    def run(n):
        rows = np.arange(n)
        t = time.perf_counter()
        oracle.attention_request(Q[rows], K, V, L, B, positions=(lk - lq) + rows)
        return time.perf_counter() - t

    n0 = 32
    t0 = run(n0)
    n = int(min(lq, max(n0, n0 * target_s / max(t0, 1e-3))))
    t = run(n)
    r = prob.ranks[0]
    D, Hq = prob.head_dim, prob.n_q_heads
    pairs = sum(lk - lq + i + 1 for i in range(n))
    flop = Hq * pairs * (4 * D + 2 * r) + Hq * n * 2 * r * D
    return {"value": round(flop / t / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(t, 2),
            "sample": f"{prob.name}, agent 0, query rows 0..{n - 1} of {lq}, all {Hq} q heads, "
                      f"fp64 numpy/BLAS on {platform.processor() or platform.machine()}"}


def ceilings(steps, warmup):
    """Attainable rates on this GPU, for context only (not targets): a 512 MiB streaming
    read (torch reduction), a 1 GiB device copy, and torch.matmul in bf16 at 8192^3."""
    import torch
    buf = torch.ones(64 << 20, dtype=torch.int64, device="cuda")
    per, _ = time_calls(lambda: buf.sum(), steps, warmup)
    read = buf.numel() * 8 / float(np.median(per)) / 1e6
    del buf
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    per, _ = time_calls(lambda: dst.copy_(src), steps, warmup)
    copy = 2 * (1 << 30) / float(np.median(per)) / 1e6
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    per, _ = time_calls(lambda: torch.matmul(a, b), max(5, steps // 2), warmup)
    mm = 2 * n ** 3 / float(np.median(per)) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"read_GBps": round(read, 1), "copy_GBps": round(copy, 1),
            "torch_matmul_bf16_8192_TFLOPs": round(mm, 1), "note": "context only"}


def environment():
    import subprocess
    import torch
    props = torch.cuda.get_device_properties(0)
    env = {"device": props.name, "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count,
           "torch": torch.__version__, "hip": torch.version.hip}
    try:
        # rocm-smi is a Python script: run it with this interpreter, so no launcher (env)
        # sits between this process and the child
        smi = os.path.realpath(shutil.which("rocm-smi"))
        r = subprocess.run([sys.executable, smi, "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        clk = json.loads(r.stdout)
        card = next(iter(clk.values()))
        env["clocks"] = {k: v for k, v in card.items() if k.lower().startswith(("sclk", "mclk"))}
    except Exception:  # noqa: BLE001
        env["clocks"] = None
    return env


def bench_sdpa_context(steps, warmup):
    """Context only, not part of the default line: torch's scaled_dot_product_attention with
    the flash backend forced (it raises rather than falling back to another backend), beside
    lra_attn_prefill at ranks 0 and 16, on square causal problems of n tokens with 32 q heads
    and head_dim 128.  SDPA gets 32 kv heads, the lra calls 8 (GQA): the same FLOP.  Calls run
    back to back, as for the headline."""
    import torch
    import torch.nn.functional as F
    from shared_rank_kv_amd import accounting, workloads
    rows = []
    for n in (4096, 9216):
        row = {"n": n, "flop_rank0": 4 * 128 * (n * (n + 1) // 2) * 32}
        try:
            from torch.nn.attention import SDPBackend, sdpa_kernel
            g = torch.Generator(device="cuda").manual_seed(n)
            q, k, v = (torch.randn(1, 32, n, 128, dtype=torch.bfloat16, device="cuda",
                                   generator=g) for _ in range(3))
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                fn = lambda: F.scaled_dot_product_attention(q, k, v, is_causal=True)  # noqa: E731
                settle(fn)
                per, _ = time_calls(fn, steps, warmup)
            ms = float(np.median(per))
            row["sdpa_flash"] = {"ms": round(ms, 4),
                                 "TFLOP/s": round(row["flop_rank0"] / ms / 1e9, 1)}
            del q, k, v
        except Exception as ex:  # noqa: BLE001  (no flash kernel for this part)
            row["sdpa_flash"] = {"error": str(ex)[:200]}
        for r in (0, 16):
            prob = workloads.custom(f"square-{n}-r{r}", "bf16", 32, 8, 128, (r,), [n], [n], [0],
                                    seed=900 + n + r)
            _, dev = upload(prob)
            fn = prefill_call(prob, dev, workspace_for(prob, False))
            settle(fn)
            per, _ = time_calls(fn, steps, warmup)
            ms = float(np.median(per))
            flop, _ = accounting.attention_work(prob)
            row[f"lra_rank{r}"] = {"ms": round(ms, 4), "TFLOP/s": round(flop / ms / 1e9, 1)}
            del dev
        rows.append(row)
    return {"workload": "square causal prefill, 32 q heads, head_dim 128", "rows": rows}


def run_only(args):
    if args.only == "copy":
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        per, _ = time_calls(lambda: dst.copy_(src), args.steps, args.warmup)
        ms = float(np.median(per))
        return {"workload": "device copy 1 GiB", "ms": ms, "GB/s": 2 * (1 << 30) / ms / 1e6,
                "read_bytes": 1 << 30, "write_bytes": 1 << 30}
    if args.only == "decode":
        return bench_decode(args.steps, args.warmup, Flusher())
    if args.only == "decode_shared":
        return bench_decode_shared(args.steps, args.warmup, Flusher())
    if args.only == "append":
        return bench_append(args.steps, args.warmup, Flusher())
    if args.only == "tiny":
        return bench_tiny_fp32(args.steps, args.warmup)
    if args.only == "sdpa":
        return bench_sdpa_context(args.steps, args.warmup)
    if args.only == "naive":
        return bench_naive_expansion(args.steps, args.warmup, Flusher())
    if args.only == "longctx":
        pre, lc = bench_longctx(args.steps, args.warmup, Flusher())
        return {"precompute": pre, "longctx_prefill": lc}
    return bench_mixed(args.steps, args.warmup)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mixed", action="store_true",
                    help="time the 32-layer mixed batch (the default; kept for old command lines)")
    ap.add_argument("--no-mixed", action="store_true", help="skip the 32-layer mixed batch")
    ap.add_argument("--only", choices=["prefill", "tiny", "decode", "decode_shared", "append",
                                       "longctx", "naive", "mixed", "copy", "sdpa"],
                    help="time one workload only (for profiling); prints its JSON object. "
                         "'copy' times a 1 GiB device copy, the reference for HBM counters; "
                         "'sdpa' times torch's flash attention beside the prefill (context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    from shared_rank_kv_amd import accounting
    if args.only and args.only != "prefill":
        print(json.dumps(run_only(args)), flush=True)
        return

    log("[bench] llama prefill (headline)")
    prob, cpu, dev, r = bench_llama_prefill(args.steps, args.warmup)
    ms_step = r["total_ms"] / args.steps
    value = r["flop"] / (ms_step * 1e-3) / 1e12
    kern_ms = float(np.mean(r["per_ms"]))
    achieved = r["flop"] / (kern_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Gaussian Llama-3-8B-shaped base K/V, LR caches and B",
        "config": {"workload": prob.name, "q_len": 1024, "k_len": 9216, "q_heads": 32,
                   "kv_heads": 8, "head_dim": 128, "rank": 16, "agents": 3, "timed_agent": 0,
                   "flop_per_step": r["flop"], "bytes_per_step": r["bytes"]},
        "roofline": roof(achieved, accounting.PEAK_BF16_TFLOPS, "TFLOP/s", "mfma",
                         traffic_bytes(prob.name)),
        "roofline_kernel": "lra_attn_prefill call (attention kernel, plus the combine pass "
                           "when the planner splits keys)",
    }
    del dev
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(prob, cpu)
    if not args.only:
        log("[bench] tiny fp32")
        out["tiny_fp32"] = bench_tiny_fp32(args.steps, args.warmup)
        flush = Flusher()
        log("[bench] decode")
        out["decode"] = bench_decode(args.steps, args.warmup, flush)
        log("[bench] shared-context decode")
        out["decode_shared"] = bench_decode_shared(args.steps, args.warmup, flush)
        log("[bench] decode-step LR append")
        out["append"] = bench_append(args.steps, args.warmup, flush)
        log("[bench] precompute + long-context prefill")
        out["precompute"], out["longctx_prefill"] = bench_longctx(args.steps, args.warmup, flush)
        log("[bench] naive and in-tile expansion comparators")
        out["naive_expansion"] = bench_naive_expansion(args.steps, args.warmup, flush)
        del flush
        torch.cuda.empty_cache()
        if not args.no_mixed:
            log("[bench] mixed 32-layer batch")
            out["mixed"] = bench_mixed(args.steps, args.warmup)
        log("[bench] ceilings")
        out["ceilings"] = ceilings(args.steps, args.warmup)
        out["env"] = environment()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
