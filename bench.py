#!/usr/bin/env python3
"""Benchmark of the causal GQA flash-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line. The headline step is fa_prefill on the prefill-q4kv-8k
workload (8192 query rows, 16 q heads / 2 kv heads, head_dim 256, Q4_0 KV
written by fa_kv_append, full causal), inputs and cache resident in HBM:
`value` is key-set-counted prefill FLOPs (4*head_dim per attended (query,
head, key)) per second of step time. The append that fills the cache is timed
on its own (`config.append_ms`) and kept out of the metric. The line also
carries a `roofline` object for the prefill kernel and a `roofline_decode`
object for the 64-slot Q4_0 decode (the metric's second half: KV-read GB/s
against HBM and against the fp32 compute ceiling), both timed with HIP events
on the launch stream; the other workloads as `legs` (the tiny and 2k
prefills, the 32k sliding-window prefill, the 64-slot decode on the opt-in fp16 hi/lo
lane, both Q4_0 workloads with the fp16 sink/window shadow, the 64-slot
decode over an fp32 cache, a varlen batch
over a paged fp32 cache, the 64-slot decode as 64 one-token requests over a
paged fp32 cache, and the LSE merge of two attention states); and the CPU
oracle timed on the host cores as `cpu_baseline`. Decode legs evict the
cache between timed calls by reading a 512 MB buffer (--evict write zero-fills
it instead, whose dirty lines are then written back inside the timed call).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "prefill causal attn TFLOP/s + decode KV-read GB/s (fraction of roofline)"
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


CSRC = os.path.join(ROOT, "causal_gqa_flash_fa_amd", "csrc")
# Sources that define each measured launch: a change to any of them makes the
# committed HBM counter figures stale.
KERNEL_SOURCES = {
    "prefill": ["fa_prefill.hip", "fa_device.hpp", "fa_internal.hpp", "fa_api.hip"],
    "decode": ["fa_decode.hip", "fa_decode_hilo.hip", "fa_decode_sched.hpp", "fa_device.hpp",
               "fa_internal.hpp", "fa_api.hip", "fa_shadow.hpp"],
    "merge": ["fa_paged.hip", "fa_device.hpp", "fa_internal.hpp", "fa_api.hip"],
}


def kernel_source_digest(which: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[which]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def measured_traffic(which: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (copy-calibrated), or None when the kernel sources have changed
    since the counters were taken (or no summary exists)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic__{workload}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    rec = None
    for line in text.splitlines():
        line = line.strip()
        if line.startswith("{") and "source_digest" in line:
            rec = json.loads(line)
    if rec is None or rec.get("source_digest") != kernel_source_digest(which):
        return None
    return rec


def keyset_pairs(n: int, pos0: int, sink: int, win: int) -> int:
    """Sum over query positions p of |K(p)| (attended keys of one q head)."""
    p = np.arange(pos0, pos0 + n, dtype=np.int64)
    if win <= 0:
        return int((p + 1).sum())
    lo = np.maximum(0, p - win + 1)
    sink = max(sink, 0)
    return int(np.minimum(p + 1, np.minimum(sink, lo) + (p - lo + 1)).sum())


def prefill_flops(w) -> float:
    return 4.0 * w.head_dim * w.n_head * keyset_pairs(w.n, w.pos0, w.attn_sink, w.attn_win)


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


# Legs warm up for at least this much wall time (the headline keeps exactly
# its W steps): the shader clock ramps up under sustained load, and the 2k
# prefill (a 0.3 ms kernel) ran ~12% slower after 3 warm-up steps than after
# 300, while the 4 ms headline kernel times the same after 3 or 40.
LEG_WARM_MS = 150.0


def warm(torch, step, warmup: int, min_ms: float = 0.0) -> int:
    """Runs `warmup` untimed steps, then more until `min_ms` of wall time has
    passed with the GPU kept busy; returns the number of steps run."""
    n = 0
    t0 = time.perf_counter()
    while n < warmup:
        step()
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    return n


class CacheEvict:
    """Evicts a leg's data from L2 and the 256 MB MALL between timed calls by
    READING a 512 MB buffer. A write-based flush (zero-filling the buffer)
    leaves up to ~290 MB of dirty lines whose write-back then runs inside the
    next timed call: on a plain 642 MB read stream it cost ~60 us (3.8 TB/s
    measured instead of 6.0 TB/s)."""

    def __init__(self, torch, dev):
        self.buf = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    mode = "read"             # bench.py --evict write restores the zero-fill

    def __call__(self):
        if CacheEvict.mode == "write":
            self.buf.zero_()
        else:
            self.buf.max()    # a reduction: reads every line, writes one byte


def spread(kms, key: str) -> dict:
    """Median, 90th percentile and relative standard deviation of the per-call
    HIP-event times `kms` (ms); the leg's headline figure stays the mean, the
    average launch duration the roofline is defined on."""
    a = np.asarray(kms, dtype=np.float64)
    return {key + "_median": float(np.median(a)), key + "_p90": float(np.percentile(a, 90)),
            key + "_rel_std": float(np.std(a) / np.mean(a))}


def prefill_leg(fa, torch, w, steps: int, warmup: int, graph: bool = False,
                warm_ms: float = LEG_WARM_MS) -> dict:
    """fa_prefill of one workload over a cache filled by fa_kv_append. The
    append is timed on its own (HIP events, `append_ms`) and is not part of
    the step. Kernel time: HIP events around each eager fa_prefill. Step
    time: fa_prefill launched eagerly, or, with `graph`, captured once in a
    HIP graph and replayed (same kernels, same work, no per-launch host
    overhead)."""
    dev = torch.device("cuda:0")
    q = torch.from_numpy(workloads.prefill_q(w)).to(dev)
    k_np, v_np = workloads.prefill_kv(w)
    kd, vd = torch.from_numpy(k_np).to(dev), torch.from_numpy(v_np).to(dev)
    del k_np, v_np
    cache, kt, vt = fa.make_cache(w.kv_format, 1, w.n_kv_head, w.head_dim, w.max_seq, dev)
    shadow = fa.add_shadow(cache, w.shadow_sink, w.shadow_win, dev) \
        if (w.shadow_sink or w.shadow_win) else None   # holds the shadow tensors alive
    out = torch.empty_like(q)
    rows = w.pos0 + w.n
    ws_bytes = fa.fa_prefill_workspace_bytes(w.n, w.n_head, w.n_kv_head, w.head_dim)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    # the append, timed apart from the step
    aev = _events(torch, max(3, steps // 4))
    for i in range(-1, len(aev)):
        if i >= 0:
            aev[i][0].record()
        fa.fa_kv_append(cache, 0, 0, rows, kd, vd)
        if i >= 0:
            aev[i][1].record()
    torch.cuda.synchronize()
    append_ms = float(np.mean([a.elapsed_time(b) for a, b in aev]))

    ev = _events(torch, steps)

    def step(i=None):
        if i is not None:
            ev[i][0].record()
        fa.fa_prefill(cache, 0, q, w.pos0, w.n, w.n_head, w.attn_sink, w.attn_win, w.scale, out,
                      ws, ws_bytes)
        if i is not None:
            ev[i][1].record()

    warm_steps = warm(torch, step, warmup, warm_ms)
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms = [a.elapsed_time(b) for a, b in ev]
    flops = prefill_flops(w)
    eager_ms = (t1 - t0) * 1e3 / steps
    step_ms = eager_ms
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step_ms = (t1 - t0) * 1e3 / steps
    kern_ms = float(np.mean(kms))
    return {
        "workload": w.name, "kind": "prefill", "kv": "q4_0" if w.kv_format else "f32",
        "n": w.n, "n_head": w.n_head, "n_kv_head": w.n_kv_head, "head_dim": w.head_dim,
        "attn_sink": w.attn_sink, "attn_win": w.attn_win,
        "shadow_sink": w.shadow_sink, "shadow_win": w.shadow_win,
        "step": "fa_prefill", "append_ms": append_ms, "warmup_steps": warm_steps,
        "launch": "hip_graph" if graph else "eager", "ms_per_step_eager": eager_ms,
        "flops": flops, "ms_per_step": step_ms, "tflops_step": flops / step_ms / 1e9,
        "prefill_kernel_ms": kern_ms, "prefill_kernel_ms_min": float(np.min(kms)),
        **spread(kms, "prefill_kernel_ms"),
        "tflops_kernel": flops / kern_ms / 1e9,
        "frac_fp32_mfma_peak": flops / kern_ms / 1e9 / PEAK_FP32_MFMA_TFLOPS,
    }


def paged_flops(w) -> float:
    """4 * head_dim FLOPs per attended (query, head, key), bottom-right
    aligned positions, full causal."""
    pairs = sum(keyset_pairs(n, c, 0, 0) for c, n in workloads.paged_requests(w))
    return 4.0 * w.head_dim * w.n_head * pairs


def paged_leg(fa, torch, w, steps: int, warmup: int) -> dict:
    """One varlen step over the paged cache: fa_paged_append of the batch's
    new K/V rows (the last query_len rows of every request), then
    fa_paged_attention with the LSE output. The earlier context rows are
    written once before timing."""
    dev = torch.device("cuda:0")
    reqs = workloads.paged_requests(w)
    table, num_blocks, seq, qsl = workloads.paged_layout(w)
    bs = w.block_size
    cache, kt, vt = fa.make_paged_cache(num_blocks, bs, w.n_kv_head, w.head_dim, dev)
    new_k, new_v, new_slots = [], [], []
    for r, (c, n) in enumerate(reqs):
        k, v = workloads.paged_kv(w, r, c + n)
        rows = np.arange(c + n)
        sm = workloads.paged_slots(table, r, rows, bs)
        fa.fa_paged_append(cache, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                           torch.from_numpy(sm).to(dev), c + n)
        new_k.append(k[c:])
        new_v.append(v[c:])
        new_slots.append(sm[c:])
    kn = torch.from_numpy(np.concatenate(new_k)).to(dev)
    vn = torch.from_numpy(np.concatenate(new_v)).to(dev)
    sn = torch.from_numpy(np.concatenate(new_slots)).to(dev)
    T = int(qsl[-1])
    q = torch.from_numpy(workloads.paged_q(w)).to(dev)
    d_qsl, d_seq, d_bt = (torch.from_numpy(x).to(dev) for x in (qsl, seq, table))
    out = torch.empty_like(q)
    lse = torch.empty((w.n_head, T), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_paged_workspace_bytes(w.head_dim)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ev = _events(torch, steps)

    def step(i=None):
        fa.fa_paged_append(cache, kn, vn, sn, T)
        if i is not None:
            ev[i][0].record()
        fa.fa_paged_attention(cache, q, T, w.n_head, d_qsl, d_seq, len(reqs), d_bt,
                              table.shape[1], -1, 0, w.scale, out, lse, ws, ws_bytes)
        if i is not None:
            ev[i][1].record()

    warm_steps = warm(torch, step, warmup, LEG_WARM_MS)
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms = [a.elapsed_time(b) for a, b in ev]
    flops = paged_flops(w)
    step_ms = (t1 - t0) * 1e3 / steps
    kern_ms = float(np.mean(kms))
    return {
        "workload": w.name, "kind": "paged", "kv": "f32", "tokens": T, "requests": len(reqs),
        "warmup_steps": warm_steps,
        "decode_requests": sum(1 for _, n in reqs if n == 1), "block_size": bs,
        "n_head": w.n_head, "n_kv_head": w.n_kv_head, "head_dim": w.head_dim,
        "flops": flops, "ms_per_step": step_ms, "tflops_step": flops / step_ms / 1e9,
        "attention_kernel_ms": kern_ms, "attention_kernel_ms_min": float(np.min(kms)),
        **spread(kms, "attention_kernel_ms"),
        "tflops_kernel": flops / kern_ms / 1e9,
        "frac_fp32_mfma_peak": flops / kern_ms / 1e9 / PEAK_FP32_MFMA_TFLOPS,
    }


def paged_decode_leg(fa, torch, w, steps: int, warmup: int) -> dict:
    """fa_paged_decode over the decode workload's rows in a paged fp32 cache
    (one query token per request), timed like the decode leg: HIP events,
    the last-level cache flushed between reps."""
    dev = torch.device("cuda:0")
    ctx = workloads.decode_ctx(w)
    table, num_blocks = workloads.decode_page_table(w, ctx)
    bs = w.block_size
    cache, kt, vt = fa.make_paged_cache(num_blocks, bs, w.n_kv_head, w.head_dim, dev)
    for s in range(w.n_slots):
        k, v = workloads.decode_kv(w, s, int(ctx[s]))
        sm = workloads.paged_slots(table, s, np.arange(int(ctx[s])), bs)
        fa.fa_paged_append(cache, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                           torch.from_numpy(sm).to(dev), int(ctx[s]))
    q = torch.from_numpy(workloads.decode_q(w)).to(dev)
    seq = torch.from_numpy(ctx.astype(np.int32)).to(dev)
    bt = torch.from_numpy(table).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.n_head, w.n_slots), dtype=torch.float32, device=dev)
    hint = int(ctx.max())
    ws_bytes = fa.fa_paged_decode_workspace_bytes(w.n_slots, w.n_head, w.n_kv_head, w.head_dim,
                                                  hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    flush = CacheEvict(torch, dev)
    ev = _events(torch, steps)

    def step(i=None):
        if i is not None:
            ev[i][0].record()
        fa.fa_paged_decode(cache, q, w.n_slots, w.n_head, seq, bt, table.shape[1], hint, -1, 0,
                           w.scale, out, lse, ws, ws_bytes)
        if i is not None:
            ev[i][1].record()

    # warm-up calls evict too, so that they match the timed ones
    warm_steps = warm(torch, lambda: (flush(), step()), warmup, LEG_WARM_MS)
    for i in range(steps):
        flush()
        step(i)
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.mean(kms))
    kv_bytes = int(ctx.sum()) * w.n_kv_head * 2 * w.head_dim * 4
    nbytes = kv_bytes + 2 * w.n_slots * w.n_head * w.head_dim * 4
    gbs = nbytes / ms / 1e6
    return {"workload": w.name, "kind": "paged_decode", "kv": "f32", "requests": w.n_slots,
            "warmup_steps": warm_steps, "evict": CacheEvict.mode,
            "block_size": bs, "num_blocks": num_blocks, "ctx_sum": int(ctx.sum()),
            "bytes": nbytes, "decode_ms": ms, "decode_ms_min": float(np.min(kms)),
            **spread(kms, "decode_ms"), "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS}


def merge_leg(fa, torch, steps: int, warmup: int, T: int = 8192, H: int = 16,
              D: int = 256) -> dict:
    """fa_merge_attn_states on [T][H][D] states: an HBM-bound pass reading
    two outputs and two LSEs and writing one of each."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(workloads.SEED_BASE + 900)
    po = torch.randn((T, H, D), device=dev, generator=g)
    so = torch.randn((T, H, D), device=dev, generator=g)
    pl = torch.randn((H, T), device=dev, generator=g)
    sl = torch.randn((H, T), device=dev, generator=g)
    out = torch.empty_like(po)
    out_lse = torch.empty_like(pl)
    ev = _events(torch, steps)

    def step(i=None):
        if i is not None:
            ev[i][0].record()
        fa.fa_merge_attn_states(out, out_lse, po, pl, so, sl, T, H, D)
        if i is not None:
            ev[i][1].record()

    warm_steps = warm(torch, step, warmup, LEG_WARM_MS)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in ev]
    nbytes = 3 * T * H * D * 4 + 3 * T * H * 4
    ms = float(np.mean(kms))
    rec = measured_traffic("merge", "merge-attn-states")
    return {"workload": f"merge-attn-states-{T}x{H}x{D}", "kind": "merge", "bytes": nbytes,
            "warmup_steps": warm_steps,
            "kernel_ms": ms, "kernel_ms_min": float(np.min(kms)), **spread(kms, "kernel_ms"),
            "gbs": nbytes / ms / 1e6, "frac_hbm_peak": nbytes / ms / 1e6 / PEAK_HBM_GBS,
            "traffic_bytes": round(rec["traffic_bytes"]) if rec else None}


def decode_leg(fa, torch, w, steps: int, warmup: int, lane: str = "fp32") -> dict:
    """fa_decode (lane "fp32") or fa_decode_q4_hilo (lane "hilo": the Q4_0
    decode on fp16 MFMA with hi/lo-split operands) over the slots' cache,
    timed with HIP events, the last-level cache flushed between reps."""
    dev = torch.device("cuda:0")
    call = fa.fa_decode_q4_hilo if lane == "hilo" else fa.fa_decode
    ctx = workloads.decode_ctx(w)
    cache, kt, vt = fa.make_cache(w.kv_format, w.n_slots, w.n_kv_head, w.head_dim, w.max_seq, dev)
    shadow = fa.add_shadow(cache, w.shadow_sink, w.shadow_win, dev) \
        if (w.shadow_sink or w.shadow_win) else None   # holds the shadow tensors alive
    for s in range(w.n_slots):
        k, v = workloads.decode_kv(w, s, int(ctx[s]))
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), torch.from_numpy(k).to(dev),
                        torch.from_numpy(v).to(dev))
    q = torch.from_numpy(workloads.decode_q(w)).to(dev)
    pos = torch.from_numpy(ctx - 1).to(dev)
    out = torch.empty_like(q)
    hint = int(ctx.max())
    ws_bytes = fa.fa_decode_workspace_bytes(cache, w.n_slots, w.n_head, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    flush = CacheEvict(torch, dev)
    ev = _events(torch, steps)

    def step(i=None):
        if i is not None:
            ev[i][0].record()
        call(cache, q, pos, w.n_slots, hint, w.n_head, 0, 0, w.scale, out, ws, ws_bytes)
        if i is not None:
            ev[i][1].record()

    # warm-up calls evict too, so that they match the timed ones
    warm_steps = warm(torch, lambda: (flush(), step()), warmup, LEG_WARM_MS)
    for i in range(steps):
        flush()                # evict the KV cache from L2 / MALL between reps (not timed)
        step(i)
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.mean(kms))
    row_bytes = w.head_dim // 32 * 18 if w.kv_format else w.head_dim * 4
    kv_bytes = int(ctx.sum()) * w.n_kv_head * 2 * row_bytes
    qo_bytes = 2 * w.n_slots * w.n_head * w.head_dim * 4
    flops = 4.0 * w.head_dim * w.n_head * float(ctx.sum())
    gbs = (kv_bytes + qo_bytes) / ms / 1e6
    compute_ceiling_gbs = PEAK_FP32_MFMA_TFLOPS * 1e12 / (flops / (kv_bytes + qo_bytes)) / 1e9
    return {
        "workload": w.name + ("-hilo" if lane == "hilo" else ""), "kind": "decode",
        "lane": "fp16 MFMA, hi/lo-split operands" if lane == "hilo" else "fp32 MFMA",
        "kv": "q4_0" if w.kv_format else "f32",
        "evict": CacheEvict.mode, "warmup_steps": warm_steps, "n_slots": w.n_slots,
        "ctx_sum": int(ctx.sum()),
        "ctx_min": int(ctx.min()),
        "ctx_max": int(ctx.max()), "launch_splits": fa.fa_decode_plan(hint)[0],
        "shadow_sink": w.shadow_sink, "shadow_win": w.shadow_win,
        "kv_bytes": kv_bytes, "bytes": kv_bytes + qo_bytes, "flops": flops,
        "decode_ms": ms, "decode_ms_min": float(np.min(kms)), **spread(kms, "decode_ms"),
        "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS, "tflops": flops / ms / 1e9,
        # the same call against the fp32 MFMA peak: a Q4_0 cache puts the decode
        # above the fp32 ridge (28.4 FLOP/B at hd 256), so this is its bound
        "frac_fp32_mfma_peak": flops / ms / 1e9 / PEAK_FP32_MFMA_TFLOPS,
        "fp32_compute_ceiling_gbs": compute_ceiling_gbs,
        "frac_of_min_ceiling": gbs / min(PEAK_HBM_GBS, compute_ceiling_gbs),
        "traffic_bytes": (round(rec["traffic_bytes"])
                          if (rec := measured_traffic("decode", w.name + ("-hilo" if lane == "hilo"
                                                                          else "")))
                          else None),
    }


def cpu_baseline(w) -> dict:
    """The oracle (plain C, double precision, single-threaded per call) over
    every row of the workload, rows spread over the host threads: all of the
    host's cores up to 16, the CPU share of one GPU on the benchmark machines
    (their os.cpu_count() reports the whole node, which other GPUs' jobs use)."""
    import oracle
    q = workloads.prefill_q(w)
    k, v = workloads.prefill_kv(w)
    kt = np.ascontiguousarray(k.transpose(1, 0, 2))
    vt = np.ascontiguousarray(v.transpose(1, 0, 2))
    if w.kv_format:
        kt = oracle.q4_dequantize(oracle.q4_quantize(kt), w.head_dim)
        vt = oracle.q4_dequantize(oracle.q4_quantize(vt), w.head_dim)
    host_cpus = os.cpu_count() or 1
    threads = min(16, host_cpus)
    t0 = time.perf_counter()
    oracle.prefill(q, kt, vt, w.pos0, w.attn_sink, w.attn_win, w.scale, threads=threads)
    dt = time.perf_counter() - t0
    value = prefill_flops(w) / dt / 1e12
    # one thread on a fixed subset: every 64th (position, head) row
    sel = np.arange(0, w.n * w.n_head, 64, dtype=np.int64)
    pos = w.pos0 + sel // w.n_head
    sel_flops = 4.0 * w.head_dim * sum(keyset_pairs(1, int(p), w.attn_sink, w.attn_win) for p in pos)
    t0 = time.perf_counter()
    oracle.prefill(q, kt, vt, w.pos0, w.attn_sink, w.attn_win, w.scale, sel=sel, threads=1)
    dt1 = time.perf_counter() - t0
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "host_cpu_count": host_cpus,
            "kind": "oracle", "seconds": dt,
            "sample": f"all {w.n * w.n_head} rows of {w.name} (fp64 global-max softmax over "
                      f"the oracle's own dequantised K/V)",
            "per_core_gflops": value * 1e3 / threads,
            "single_thread": {"gflops": sel_flops / dt1 / 1e9, "seconds": dt1,
                              "sample": f"every 64th row ({sel.size} rows) of {w.name}"},
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or ""."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def copy_calibration(torch, nbytes: int = 1 << 30) -> dict:
    """A plain device copy of known size, for scaling HBM byte counters."""
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="tiny-prefill-128,prefill-f32kv-2k,window-prefill-32k,"
                                      "decode-64slots-q4kv,decode-64slots-q4kv-hilo,"
                                      "prefill-q4kv-8k-shadow,decode-64slots-q4kv-shadow,"
                                      "decode-64slots-f32kv,"
                                      "paged-varlen-8k,paged-decode-64req-f32kv,merge-attn-states",
                    help="comma-separated extra workloads ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch the headline step eagerly instead of replaying a HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for counter scaling)")
    ap.add_argument("--evict", choices=("read", "write"), default="read",
                    help="how decode legs evict the cache between timed calls: read a 512 MB "
                         "buffer, or zero-fill it (its dirty lines are then written back during "
                         "the next call)")
    ap.add_argument("--only", default="",
                    help="run just this workload and print its leg as the JSON line "
                         "(for profiling one kernel)")
    args = ap.parse_args()
    CacheEvict.mode = args.evict
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        return 2

    import torch
    import causal_gqa_flash_fa_amd as fa
    torch.cuda.set_device(0)
    fa.fa_init()

    def run_leg(name):
        if name == "merge-attn-states":
            return merge_leg(fa, torch, args.steps, args.warmup)
        if name.endswith("-hilo"):
            return decode_leg(fa, torch, workloads.BY_NAME[name[:-len("-hilo")]], args.steps,
                              args.warmup, lane="hilo")
        w = workloads.BY_NAME[name]
        fn = {"prefill": prefill_leg, "decode": decode_leg, "paged": paged_leg,
              "paged_decode": paged_decode_leg}[w.kind]
        return fn(fa, torch, w, args.steps, args.warmup)

    if args.only:
        leg = run_leg(args.only)
        if args.copy_calibration:
            leg["copy_calibration"] = copy_calibration(torch)
        print(json.dumps(leg), flush=True)
        return 0

    head = workloads.BY_NAME["prefill-q4kv-8k"]
    print(f"[bench] {head.name}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    main_leg = prefill_leg(fa, torch, head, args.steps, args.warmup, graph=not args.eager,
                           warm_ms=0.0)
    torch.cuda.empty_cache()
    legs = []
    for name in [s for s in args.legs.split(",") if s]:
        print(f"[bench] leg {name}", file=sys.stderr, flush=True)
        legs.append(run_leg(name))
        torch.cuda.empty_cache()
    extra = {}
    if args.copy_calibration:
        extra["copy_calibration"] = copy_calibration(torch)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(head)

    kern_tflops = main_leg["tflops_kernel"]
    rec = measured_traffic("prefill", head.name)
    traffic_bytes = round(rec["traffic_bytes"]) if rec else None
    traffic_src = f"profiles/hbm_traffic__{head.name}.md" if rec else None
    # the metric's decode half: the 64-slot Q4_0 decode leg (run here if the
    # leg list left it out)
    dec = next((g for g in legs if g.get("workload") == "decode-64slots-q4kv"), None)
    if dec is None:
        print("[bench] decode-64slots-q4kv (decode roofline)", file=sys.stderr, flush=True)
        dec = run_leg("decode-64slots-q4kv")
    drec = measured_traffic("decode", dec["workload"])
    roofline_decode = {
        "bound": "hbm", "workload": dec["workload"],
        "kernel": "fa_decode: decode_partial_kernel<256,8,q4_0> + decode_combine_kernel<256,8>",
        "achieved": round(dec["gbs"], 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(dec["gbs"] / PEAK_HBM_GBS, 4),
        "traffic": round(drec["traffic_bytes"]) if drec else None,
        "traffic_source": f"profiles/hbm_traffic__{dec['workload']}.md" if drec else None,
        "kernel_ms": round(dec["decode_ms"], 5), "bytes_per_launch": dec["bytes"],
        # a Q4_0 cache at G = 8 needs 28.4 FLOP per KV byte, past the fp32 ridge:
        # the fp32 MFMA peak caps this call below 8 TB/s
        "fp32_compute_ceiling_gbs": round(dec["fp32_compute_ceiling_gbs"], 1),
        "frac_of_fp32_ceiling": round(dec["frac_of_min_ceiling"], 4),
        "frac_fp32_mfma_peak": round(dec["frac_fp32_mfma_peak"], 4),
    }
    line = {
        "metric": METRIC,
        "value": round(main_leg["tflops_step"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_leg["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head.name, "n": head.n, "pos0": head.pos0,
                   "n_head": head.n_head, "n_kv_head": head.n_kv_head,
                   "head_dim": head.head_dim, "kv": "q4_0", "attn_sink": head.attn_sink,
                   "attn_win": head.attn_win, "step": "fa_prefill",
                   "append_ms": round(main_leg["append_ms"], 5),
                   "launch": main_leg["launch"],
                   "ms_per_step_eager": round(main_leg["ms_per_step_eager"], 4)},
        "roofline": {"bound": "mfma",
                     "kernel": "fa_prefill: prefill_kernel<256,8,q4_0> + prefill_combine_kernel<256,8>",
                     "achieved": round(kern_tflops, 3), "peak": PEAK_FP32_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_FP32_MFMA_TFLOPS, 4),
                     "traffic": traffic_bytes,
                     "traffic_source": traffic_src,
                     "kernel_ms": round(main_leg["prefill_kernel_ms"], 5),
                     "flops_per_launch": main_leg["flops"]},
        "roofline_decode": roofline_decode,
        "cpu_baseline": cpu,
        "legs": legs,
        **extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
