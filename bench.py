#!/usr/bin/env python3
"""Benchmark of the position-independent KV-reuse hot path on one MI355X.

One step = one batch through the whole path: plan + gather/re-rotate the
prefix (pic_assemble), then the query prefill of every layer
(pic_query_prefill: rotate and append the new tokens, attention over prefix +
new rows).  Inputs (pool, span tables, every layer's q/k/v) are resident in
HBM before the timed region.  Steps cycle through pre-generated batch layouts
over the same pool.

Prints one JSON line.  `value` is the whole step's attention throughput
(algorithmic attention FLOPs of a step / step time, so assembly and prologue
time count against it); per-kernel rates, latency percentiles, the roofline of
the dominant kernel and the CPU-oracle baseline ride along.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant M|F]

Variants: M gathers the prefix (assembly kernel) and attends over it; F
reads the pool inside attention, rotating keys on load.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HERE = os.path.dirname(os.path.abspath(__file__))
METRIC = "assembly GB/s + query-prefill attn TFLOP/s (% roofline), p99 µs/request"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector
KERNEL_GATHER, KERNEL_PROLOGUE, KERNEL_ATTN, KERNEL_PLAN = 0, 1, 2, 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="turborag_b16")
    ap.add_argument("--variant", default="M", choices=["M", "F"])
    ap.add_argument("--layouts", type=int, default=8, help="pre-generated batch layouts to cycle through")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of each oracle sample (all cores, then one thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--values-in-pool", action="store_true",
                    help="variant M: gather keys only and let attention read the prefix values in the pool "
                         "(the same bits)")
    ap.add_argument("--pipelined", action="store_true",
                    help="gather layer l+1 on a second stream while layer l's attention runs")
    ap.add_argument("--host-pool", action="store_true",
                    help="keep the pool in pinned host memory (the staging tier): assembly reads the "
                         "covered rows over the host link")
    ap.add_argument("--hot-pages", type=int, default=0,
                    help="with --host-pool: an HBM hot set of this many page slots in front of the pool "
                         "(least recently used pages evicted); reports the cold first pass over the layouts")
    ap.add_argument("--store-dir", default=None,
                    help="with --host-pool: write the pool to one file per chunk in this directory and let "
                         "assembly read the pages each batch covers from the files; reports cold steps "
                         "(every page read from the files, the OS cache dropped first)")
    ap.add_argument("--store-threads", type=int, default=8, help="host threads reading chunk files")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="also time this many decode steps (every layer, one token per request) after a prefill")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM counters), then exit")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
    the factor between counter units and bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 5}), flush=True)


def percentile(xs, q):
    """Nearest-rank percentile."""
    s = sorted(xs)
    k = max(0, min(len(s) - 1, int(-(-q * len(s) // 100)) - 1))
    return s[k]


def _oracle_sample(wl, pool, dw, budget_s: float):
    """Time the fp64 oracle on requests in order, every layer of each, until
    the time budget is spent (or the whole batch is done).  Only the oracle's
    own work is timed, not the read-back of its inputs.  Returns (attention
    FLOPs of the sample, seconds, (request, layer) pairs, requests touched)."""
    import numpy as np
    from oracle import pic_oracle as orc
    import workloads as W
    m = wl.model
    flops = 0
    spent = 0.0
    pairs = 0
    done_reqs = 0
    cache = {}
    for b, r in enumerate(wl.requests):
        spans = [tuple(int(x) for x in s) for s in r.spans]
        planned = orc.plan_spans(spans, wl.pool.chunk_orig)
        pos_new = orc.new_token_positions(planned, r.n_new, r.new_pos)
        nb = int(wl.new_ptr()[b])
        n_visible = None
        for l in range(m.layers):
            ck, cv = {}, {}
            for c in sorted(set(int(c) for c in r.spans[:, 0])):
                k, v = W.chunk_kv(wl, pool, c, [l])
                ck[c], cv[c] = k.numpy(), v.numpy()
            if l not in cache:
                cache[l] = dw.layer_inputs(l)
            q, kn, vn = cache[l]
            sl = slice(nb, nb + r.n_new)
            qn, kk, vv = (t[sl].float().cpu().double().numpy() for t in (q, kn, vn))
            t0 = time.perf_counter()
            kp, vp, pp = orc.assemble(ck, cv, spans, m.theta, m.dtype, chunk_orig=wl.pool.chunk_orig)
            orc.query_prefill_layer(kp[0], vp[0], pp, qn, kk, vv, pos_new, m.theta, m.dtype, m.kv_heads)
            spent += time.perf_counter() - t0
            pairs += 1
            if n_visible is None:
                rows = np.concatenate([pp, pos_new])
                n_visible = int(sum(int((rows <= p).sum()) for p in pos_new))
            flops += 4 * m.head_dim * m.q_heads * n_visible
            if spent >= budget_s:
                break
        done_reqs = b + 1
        if spent >= budget_s:
            break
    return flops, spent, pairs, done_reqs


def cpu_baseline(wl, pool, dw, budget_s: float):
    """The fp64 oracle as it stands, on the host cores: once with every BLAS
    thread numpy has, once limited to one thread, each on a sample of about
    `budget_s` seconds of oracle time.  `value` is the all-threads rate."""
    import threadpoolctl
    affinity = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    threads = max((d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()), default=1)
    fl, sec, pairs, reqs = _oracle_sample(wl, pool, dw, budget_s)
    with threadpoolctl.threadpool_limits(1):
        fl1, sec1, pairs1, _ = _oracle_sample(wl, pool, dw, budget_s)
    return {"value": fl / sec / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{pairs} (request, layer) pairs of {wl.name} ({reqs} of {wl.batch} requests, "
                      f"{wl.model.layers} layers each): gather, re-rotation and attention in fp64 numpy, "
                      f"{sec:.1f} s of oracle time; value = the sample's attention FLOPs / that time",
            "single_thread": {"value": fl1 / sec1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": f"{pairs1} (request, layer) pairs, {sec1:.1f} s"},
            "host": {"logical_cpus": os.cpu_count(), "affinity_cpus": len(affinity),
                     "affinity": _ranges(affinity), "blas_threads": int(threads)}}


def _ranges(cpus) -> str:
    """CPU list as ranges, e.g. '0-15,32-47'."""
    out, i = [], 0
    while i < len(cpus):
        j = i
        while j + 1 < len(cpus) and cpus[j + 1] == cpus[j] + 1:
            j += 1
        out.append(f"{cpus[i]}-{cpus[j]}" if j > i else f"{cpus[i]}")
        i = j + 1
    return ",".join(out)


def kernel_source_hash() -> str:
    """sha256 of the HIP kernel sources; counter-based traffic figures are only
    valid for the kernels they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in ("pic_kernels.hip", "pic_kernels.h"):
        with open(os.path.join(HERE, "position_independent_kv_pic_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, variant: str) -> dict:
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE,
    WRITE_SIZE, scaled by a plain copy of known size), read from the committed
    profile summary of this workload; empty when none exists or the kernels
    changed since it was taken."""
    path = os.path.join(HERE, "profiles", f"traffic_{workload}_{variant}.txt")
    if not os.path.exists(path):
        return {}
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return {}
    out = {}
    for key in ("attention", "gather"):
        if f"{key}_bytes_per_launch" in vals:
            out[key] = int(vals[f"{key}_bytes_per_launch"])
    return out


def decode_bench(args, wl, dw, inputs, variant, stream) -> dict:
    """Decode after a prefill of layout 0: K steps of one token per request over
    every layer, timed with events on the launch stream.  The rows a step
    reads (K and V of every earlier row of every request, all layers and kv
    heads) give the effective HBM rate of this HBM-bound step."""
    import torch
    import workloads as W
    m = wl.model
    sess = dw.session
    plan = sess.plan
    K = args.decode_steps
    plan.set_decode_rows(K)
    sess.ensure_capacity(wl.rows_total + K * wl.batch)
    plan_flag = 1 if variant == 1 else 0
    plan.assemble(wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat(), sess.asm_k, sess.asm_v,
                  sess.capacity, plan_flag, stream)
    n = wl.n_new_total
    for l in range(m.layers):
        q, k, v = inputs[l]
        plan.query_prefill(l, q[:n], k[:n], v[:n], torch.empty_like(q[:n]), variant, stream)
    dec_in = [[W.decode_tokens(wl, l, st, dw.kscale, dw.vscale, dw.kscale.device) for l in range(m.layers)]
              for st in range(K)]
    dout = torch.empty_like(dec_in[0][0][0])
    dptr = [[tuple(t.data_ptr() for t in dec_in[st][l]) for l in range(m.layers)] for st in range(K)]
    optr, sptr = dout.data_ptr(), stream.cuda_stream
    dl = plan.decode_layer
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    gc.collect()
    gc.disable()   # (as in the prefill's timed region)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for st in range(K):
        for l in range(m.layers):
            dl(l, st, *dptr[st][l], optr, variant, sptr)
        ev[st + 1].record(stream)
    torch.cuda.synchronize()
    gc.enable()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(K)]
    plan.set_decode_rows(0)
    rows = wl.rows_total
    bytes_step = (rows + wl.batch * (K + 1) / 2) * 2 * m.layers * m.kv_heads * m.head_dim * m.elem_bytes
    ms_med = sorted(ms)[len(ms) // 2]
    return {"steps": K, "ms_per_step_median": round(ms_med, 4), "tokens_per_s": round(wl.batch / (ms_med * 1e-3), 1),
            "kv_read_GBps": round(bytes_step / (ms_med * 1e-3) / 1e9, 1),
            "note": "one token per request per step over all layers; kv_read counts each earlier row's K and V once"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path would shard "
              f"requests or kv heads across GPUs with no exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import workloads as W
    from workloads.device import open_workload
    from position_independent_kv_pic_amd import (DEFER_GATHER, PLAN_ONLY, VALUES_IN_POOL,
                                                  VARIANT_FUSED, VARIANT_MATERIALIZED)

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    variant = VARIANT_MATERIALIZED if args.variant == "M" else VARIANT_FUSED
    wls = [W.get(args.workload, layout=i) for i in range(args.layouts)]
    wl = wls[0]
    m = wl.model
    log(f"[bench] workload {wl.name}: batch {wl.batch}, layers {m.layers}, rows {wl.rows_total}")
    if args.store_dir and not args.host_pool:
        sys.exit("--store-dir needs --host-pool")
    if args.store_dir:
        os.makedirs(args.store_dir, exist_ok=True)
    t_open = time.perf_counter()
    dw = open_workload(wl, host_pool=args.host_pool, hot_pages=args.hot_pages, store_dir=args.store_dir,
                       store_threads=args.store_threads)
    if args.store_dir:
        log(f"[bench] pool written to {len(wl.pool.chunk_len)} chunk files in {time.perf_counter() - t_open:.1f} s")
    sess = dw.session
    cap = max(w.rows_total for w in wls)
    sess.ensure_capacity(cap)
    # inputs sized for the layout with the most new tokens; each step passes
    # the leading rows its own layout needs
    wl_max = max(wls, key=lambda w: w.n_new_total)
    inputs = [W.new_tokens(wl_max, l, dw.kscale, dw.vscale, dw.kscale.device) for l in range(m.layers)]
    outs = [torch.empty_like(inputs[l][0]) for l in range(m.layers)]
    tables = [(w.span_ptr(), w.spans_flat(), w.new_ptr(), w.new_pos_flat(), w.n_new_total) for w in wls]
    stream = torch.cuda.current_stream()
    # device pointers of each layer's inputs and output, taken once: a step
    # reads the leading rows its layout needs, which start at the same address
    lptr = [(inputs[l][0].data_ptr(), inputs[l][1].data_ptr(), inputs[l][2].data_ptr(), outs[l].data_ptr())
            for l in range(m.layers)]
    sptr = stream.cuda_stream
    plan = sess.plan
    plan_flag = 0 if args.variant == "M" else PLAN_ONLY
    vpool = args.values_in_pool and args.variant == "M"
    if vpool:
        plan_flag |= VALUES_IN_POOL

    side = torch.cuda.Stream() if args.pipelined else None

    def step(i):
        sp, spans, npt, npos, n = tables[i % len(tables)]
        if args.pipelined and variant != VARIANT_FUSED:
            # per-layer gathers on a second stream, one layer ahead of attention
            plan.assemble(sp, spans, npt, npos, sess.asm_k, sess.asm_v, sess.capacity,
                          DEFER_GATHER | (VALUES_IN_POOL if vpool else 0), stream)
            plan.gather_layers(0, 1, side)
            for l in range(m.layers):
                if l + 1 < m.layers:
                    plan.gather_layers(l + 1, l + 2, side)
                plan.query_prefill(l, *lptr[l], variant, sptr)
            # the next step's planes may only be overwritten after this one is done
            stream.wait_stream(side)
            return
        plan.assemble(sp, spans, npt, npos, sess.asm_k, sess.asm_v, sess.capacity, plan_flag, stream)
        qp = plan.query_prefill
        for l in range(m.layers):
            qp(l, *lptr[l], variant, sptr)

    # with chunk files: each layout once from cold files (pages forgotten and
    # the OS cache dropped first), host wall time to the end of the step
    store = None
    if sess.store is not None:
        cold, nbytes, waits = [], [], []
        for i in range(len(tables)):
            torch.cuda.synchronize()
            sess.store.forget(drop_os_cache=True)
            s0 = sess.store.stats()
            t0 = time.perf_counter()
            step(i)
            torch.cuda.synchronize()
            cold.append((time.perf_counter() - t0) * 1e3)
            s1 = sess.store.stats()
            nbytes.append(s1["bytes_read"] - s0["bytes_read"])
            waits.append(s1["wait_seconds"] - s0["wait_seconds"])
        store = {"threads": args.store_threads, "cold_step_ms": [round(x, 2) for x in cold],
                 "cold_bytes_read": nbytes, "cold_read_seconds": [round(x, 4) for x in waits],
                 "read_GBps": round(sum(nbytes) / max(sum(waits), 1e-9) / 1e9, 2),
                 "after_cold_pass": sess.store.stats()}
        log(f"[bench] chunk files, cold steps: {store}")
        # the timed steps below find every page loaded
        for t in tables:
            sess.store.request(t[0], t[1])
        sess.store.wait()

    # with a hot set: a cold first pass over the layouts, each step timed (the
    # first misses every page; later ones may find pages an earlier layout
    # brought in)
    hot = None
    if sess.cache is not None:
        cold = []
        for i in range(len(tables)):
            ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ce0.record(stream)
            step(i)
            ce1.record(stream)
            torch.cuda.synchronize()
            cold.append(ce0.elapsed_time(ce1))
        hot = {"pages": args.hot_pages, "first_step_ms": round(cold[0], 3),
               "first_pass_ms_per_step": round(sum(cold) / len(cold), 3), "first_pass_steps": len(cold),
               "after_first_pass": sess.cache.stats()}
        log(f"[bench] hot set cold pass: {hot}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    hot_before = sess.cache.stats() if sess.cache is not None else None

    # timed region: K steps, per-step events on the launch stream.  Python's
    # cyclic garbage collector stays off inside it: a full collection stalls
    # the issuing thread for tens of milliseconds at a step fixed by the
    # allocation count, longer than the one step the host runs ahead, and
    # the GPU would wait (measured: one step of 36-39 ms in 200)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
        ev[i + 1].record(stream)
    issued = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    if hot is not None:
        after = sess.cache.stats()
        hot["timed_bytes_copied_per_step"] = (after["bytes_copied"] - hot_before["bytes_copied"]) / args.steps
        hot["timed_misses"] = after["misses"] - hot_before["misses"]
        hot["timed_evictions"] = after["evictions"] - hot_before["evictions"]
    total_ms = ev[0].elapsed_time(ev[-1])
    log(f"[bench] timed {args.steps} steps: {total_ms:.2f} ms (host wall {wall * 1e3:.2f} ms, "
        f"issued in {issued * 1e3:.2f} ms)")
    srt = sorted(step_ms)
    log(f"[bench] step ms: min {srt[0]:.3f} p50 {srt[len(srt) // 2]:.3f} p90 {srt[int(0.9 * (len(srt) - 1))]:.3f} "
        f"max {srt[-1]:.3f}; slowest {[round(x, 2) for x in srt[-5:]]} at steps "
        f"{sorted(range(len(step_ms)), key=lambda i: step_ms[i])[-5:]}")

    # per-kernel durations: the same K steps again with the library's HIP-event
    # brackets around each kernel class on the launch stream (kept out of the
    # timed region: about a hundred extra event records per step lengthen it)
    plan.timing(True)
    plan.timing_reset()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kt = {k: plan.timing_read(k) for k in (KERNEL_GATHER, KERNEL_PROLOGUE, KERNEL_ATTN, KERNEL_PLAN)}
    plan.timing(False)

    # practical HBM ceiling for reference: a plain device copy of 2 GiB
    src = torch.empty(1 << 30, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    for _ in range(5):
        dst.copy_(src)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() * 2 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del src, dst

    asm_bytes = sum(W.assembly_bytes(w) for w in (wls * args.steps)[:args.steps]) / args.steps
    if vpool:
        asm_bytes /= 2   # keys only
    attn_flops = sum(W.attention_flops(w) for w in (wls * args.steps)[:args.steps]) / args.steps
    ms_step = total_ms / args.steps
    n_g, t_g = kt[KERNEL_GATHER]
    n_a, t_a = kt[KERNEL_ATTN]
    n_p, t_p = kt[KERNEL_PROLOGUE]
    gather_ms = t_g / max(n_g, 1)
    attn_ms = t_a / max(n_a, 1)
    asm_gbps = asm_bytes / (gather_ms * 1e-3) / 1e9 if n_g else None
    attn_launch_flops = attn_flops / m.layers
    attn_tflops = attn_launch_flops / (attn_ms * 1e-3) / 1e12 if n_a else None
    value = attn_flops / (ms_step * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if m.dtype == "bf16" else FP32_PEAK_TFLOPS
    traffic = measured_traffic(wl.name, args.variant)

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        # host time to issue one step (plan, upload, one call per layer); at or
        # above the GPU's per-step time (p50 below) the step waits for the host
        "host_issue_ms_per_step": round(issued * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "model_shape": f"L{m.layers} Hq{m.q_heads} Hkv{m.kv_heads} d{m.head_dim}",
                   "batch": wl.batch, "prefix_rows_per_step": wl.prefix_rows_total,
                   "new_tokens_per_step": wl.n_new_total, "variant": args.variant,
                   "values": "read in the pool by attention" if vpool else "gathered with the keys",
                   "layouts": args.layouts, "parallelism": "none (1 GPU)",
                   "pipelined": bool(args.pipelined), "pool": "pinned host" if args.host_pool else "HBM",
                   "hot_pages": args.hot_pages if args.host_pool else 0},
        "assembly_GBps": None if asm_gbps is None else round(asm_gbps, 1),
        "assembly_frac_hbm": None if asm_gbps is None else round(asm_gbps / HBM_PEAK_GBPS, 4),
        "hbm_copy_GBps": round(copy_gbps, 1),
        "attention_TFLOPs": None if attn_tflops is None else round(attn_tflops, 2),
        "attention_frac_peak": None if attn_tflops is None else round(attn_tflops / peak, 4),
        "p50_us_per_request": round(percentile(step_ms, 50) * 1e3, 1),
        "p99_us_per_request": round(percentile(step_ms, 99) * 1e3, 1),
        "amortized_us_per_request": round(ms_step * 1e3 / wl.batch, 2),
        "kernel_ms": {"gather": round(gather_ms, 4), "attention_per_layer": round(attn_ms, 4),
                      "prologue_per_layer": round(t_p / max(n_p, 1), 4),
                      "plan": round(kt[KERNEL_PLAN][1] / max(kt[KERNEL_PLAN][0], 1), 4)},
        "roofline": {"bound": "mfma", "achieved": None if attn_tflops is None else round(attn_tflops, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": None if attn_tflops is None else round(attn_tflops / peak, 4),
                     "traffic": traffic.get("attention"), "kernel": "attention_bf16_kernel (+ merge_kernel when split)",
                     "per_launch_flops": int(attn_launch_flops)},
        "roofline_assembly": {"bound": "hbm", "achieved": None if asm_gbps is None else round(asm_gbps, 1),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": None if asm_gbps is None else round(asm_gbps / HBM_PEAK_GBPS, 4),
                              "traffic": traffic.get("gather"), "kernel": "gather_kernel",
                              "per_launch_bytes": int(asm_bytes)},
        "not_ttft": "assembly + per-layer attention only; no projections, MLP or sampling",
    }
    if variant == VARIANT_FUSED:
        res["roofline_assembly"]["achieved"] = None
        res["assembly_GBps"] = None
        res["roofline_assembly"]["note"] = "fused variant gathers inside attention; no gather kernel"
    if args.decode_steps > 0:
        res["decode"] = decode_bench(args, wl, dw, inputs, variant, stream)
    if hot is not None:
        res["hot_set"] = hot
    if store is not None:
        res["chunk_files"] = store
        res["config"]["pool"] = "pinned host, filled from chunk files"
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        res["cpu_baseline"] = cpu_baseline(wl, dw.pool, dw, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    dw.close()


if __name__ == "__main__":
    main()
