#!/usr/bin/env python3
"""MoE-stack decode benchmark on one MI355X.

A step is one token row (T = 1) through the whole 40-layer 35B-A3B-shaped MoE
stack (H 2048, 256 experts of intermediate 512, top-8 + shared expert of 512,
6-bit routed experts, 8-bit shared expert and router, groups of 64), with
distinct generated weights per layer resident in HBM and a fresh synthetic x
row per step (seed 1000 + step). Prints one JSON line:

* value: tokens/s through the stack (T * steps / timed seconds);
* achieved GB/s of touched bytes: the routed experts actually selected (from
  the routing the GPU returned; duplicates across rows counted once), the
  shared expert, the router and the gate vector, at their packed size
  (codes + one bf16 scale and bias per 64 weights);
* roofline: the dominant kernel, the streaming stack kernel (one launch per
  step runs all layers, preceded by a clear kernel of about 2 us), against the
  8 TB/s HBM peak: touched bytes per launch / mean launch duration, the
  duration taken with HIP events recorded around every step on the stream the
  library launches on; traffic: the HBM bytes one launch fetched and wrote,
  from rocprofv3 FETCH_SIZE and WRITE_SIZE passes scaled by what the same
  counters read for a plain device copy of known size (--copy-probe), stored
  below with a hash of the kernel sources and reported only while the sources
  still hash the same;
* step_us: median, 10th and 90th percentile of the per-step call durations
  (the same HIP events); unique_experts_per_layer: the mean size of the union
  of the rows' selected experts per layer and step;
* config0_gpu (a3b only): GPU microseconds per layer of the small one-layer
  shape through the same entry point;
* cpu_baseline: the fp64 oracle timed on this host on a bounded sample, single
  core (value) and all cores, split into compute and weight regeneration per
  layer, for the bench workload and the one-layer and 397B-A17B shapes, with
  the CPU model, os.cpu_count(), the affinity-mask cores and BLAS threads.

Usage: python bench.py [--steps K] [--warmup W] [--workload a3b] [--no-cpu]
       python bench.py --copy-probe MIB   (PMC calibration: 5 device copies)
       python bench.py --phase-trace      (the phase-trace build libmoe_trace.so: per-phase
                                           timestamps of the streaming stack kernel, T = 1;
                                           prints a table, no JSON line)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["stack1.hip", "gemv.h", "device_common.h", "internal.h"]  # the stack kernel's device code

# HBM traffic of one stack-kernel launch, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over
# `bench.py --steps 5 --warmup 2 --no-cpu`, each scaled by bytes/counter of a
# 256 MiB device copy measured the same way. Keyed by workload; valid only
# for the kernel sources whose hash is stored with it.
TRAFFIC = {
    "a3b": {"src_hash": "2b7bd0a3e4f4f1c0", "fetch_bytes": 997_514_166, "write_bytes": 13_120_471},
}


def kernel_source_hash() -> str:
    """Hash of the stack kernel's device sources with // comments and blank lines removed."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_moe_decode_softmax_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def kernel_path(w) -> str:
    """What one moe_decode_stack call launches for this workload."""
    if w.T == 1:
        return f"stack1_kernel: all {w.n_layers} layers in one launch (timed with its clear kernel)"
    if w.T > 8 and w.router_bits == 8 and w.shared_bits == 8:
        return (f"per-layer kernels: mfma_pack, route_mfma, down_mfma, select, expert, down per layer ({w.n_layers} "
                f"layers, timed together)")
    return f"per-layer kernels: route, select, expert, down per layer ({w.n_layers} layers, timed together)"


def copy_probe(mib: int) -> int:
    """Five copies of a MIB-MiB device buffer: the known-size kernel the PMC byte counters are scaled by."""
    import torch

    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
    return 0


def _matrix_alg_bytes(bits: int, rows: int, cols: int) -> int:
    rb = 4 * ((cols + 9) // 10) if bits == 3 else cols * bits // 8
    return rows * rb + rows * (cols // 64) * 4


def _ffn_bytes(bits: int, h: int, inter: int) -> int:
    return 2 * _matrix_alg_bytes(bits, inter, h) + _matrix_alg_bytes(bits, h, inter)


def touched_bytes(w, ids: np.ndarray) -> int:
    """ids: [steps, layers, T, k] -> total algorithmic bytes over all steps."""
    per_expert = _ffn_bytes(w.expert_bits, w.hidden, w.inter)
    router = w.n_experts * w.hidden * 2 if w.router_bits == 16 else _matrix_alg_bytes(w.router_bits, w.n_experts,
                                                                                        w.hidden)
    static = _ffn_bytes(w.shared_bits, w.hidden, w.shared_inter) + router + 2 * w.hidden
    total = 0
    for s in range(ids.shape[0]):
        for l in range(ids.shape[1]):
            total += len(np.unique(ids[s, l])) * per_expert + static
    return total


def _host_info():
    """CPU model, os.cpu_count() and the cores of this process's affinity mask."""
    model = None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count()
    return model, os.cpu_count(), aff


def _oracle_pass(w, threads: int, budget_s: float):
    """The oracle as it stands: token rows through w's layer stack in order,
    BLAS limited to `threads`, until the budget is spent (at least one layer).
    Each layer runs twice on the same input: the first pass regenerates from
    the seed the weights the layer touches, the second reuses them, so the
    difference is the regeneration time. Returns per-layer means."""
    import oracle
    from oracle.gen import GeneratedLayer, MoEShape, gen_x
    from threadpoolctl import threadpool_info, threadpool_limits

    sh = MoEShape(hidden=w.hidden, n_experts=w.n_experts, inter=w.inter, top_k=w.top_k,
                  shared_inter=w.shared_inter, router_bits=w.router_bits, expert_bits=w.expert_bits,
                  shared_bits=w.shared_bits, eps=w.rms_eps)
    with threadpool_limits(limits=threads):
        blas = sorted({i["num_threads"] for i in threadpool_info()})
        t_start = time.perf_counter()
        comp = regen = 0.0
        n = token = 0
        done = False
        while not done:
            h = gen_x(1000 + token, 1, w.hidden)
            for layer in range(w.n_layers):
                gl = GeneratedLayer(sh, 0, layer)
                t0 = time.perf_counter()
                oracle.layer_forward(gl, h)
                t1 = time.perf_counter()
                r = oracle.layer_forward(gl, h)
                t2 = time.perf_counter()
                comp += t2 - t1
                regen += max(0.0, (t1 - t0) - (t2 - t1))
                n += 1
                h = oracle.bf16_round(r["y"])
                if time.perf_counter() - t_start > budget_s:
                    done = True
                    break
            token += 1
    per_token = (comp + regen) / n * w.n_layers
    return {"tok_s": round(1.0 / per_token, 5), "s_per_token": round(per_token, 3),
            "compute_s_per_layer": round(comp / n, 4), "regen_s_per_layer": round(regen / n, 4),
            "layers_timed": n, "layers_per_token": w.n_layers, "blas_threads": blas,
            "extrapolated": n < w.n_layers}


def cpu_baseline(w, budget_s: float = 10.0):
    """The oracle timed on this host, single core and all cores, for the bench
    workload and for the small one-layer shape and the 397B-A17B shape."""
    from quantized_moe_decode_softmax_amd import WORKLOADS

    model, n_cpu, aff = _host_info()
    one = _oracle_pass(w, 1, budget_s)
    allc = _oracle_pass(w, aff, budget_s)
    others = {}
    for name, share in (("tiny", 0.2), ("a17b", 1.0)):
        if name == w.name:
            continue
        ow = WORKLOADS[name]
        others[name] = {"single_core": _oracle_pass(ow, 1, budget_s * share),
                        "all_cores": dict(_oracle_pass(ow, aff, budget_s * share), cores=aff)}
    return {
        "value": one["tok_s"],
        "unit": "tok/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{one['layers_timed']} layer passes of the {w.n_layers}-layer {w.name} stack (token rows from "
                   f"x seed 1000, layers in order), fp64 numpy, BLAS limited to 1 thread; per layer "
                   f"{one['compute_s_per_layer']} s of steps O2-O8 plus {one['regen_s_per_layer']} s regenerating "
                   f"the touched weights from the seed; scaled to {w.n_layers} layers per token"),
        "single_core": one,
        "all_cores": dict(allc, cores=aff),
        "other_configs": others,
        "cpu_model": model,
        "os_cpu_count": n_cpu,
        "affinity_cores": aff,
    }


def config0_gpu(K: int = 200, W: int = 20):
    """GPU time per layer of the small one-layer shape (moe_stack_decode, T = 1)."""
    import torch

    from quantized_moe_decode_softmax_amd import WORKLOADS
    from quantized_moe_decode_softmax_amd import _lib as Lb
    from quantized_moe_decode_softmax_amd.runtime import DeviceStack

    w = WORKLOADS["tiny"]
    ds = DeviceStack.from_workload(w)
    st = ds.state()
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty((1, w.hidden), dtype=torch.bfloat16, device="cuda")
    xs = [ds.rows(1000 + s, 1) for s in range(W + K)]
    for s in range(W):
        Lb.moe_stack_decode(st, 1, xs[s].data_ptr(), out.data_ptr(), None, None, None, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
    for s in range(K):
        ev[2 * s].record()
        Lb.moe_stack_decode(st, 1, xs[W + s].data_ptr(), out.data_ptr(), None, None, None, stream)
        ev[2 * s + 1].record()
    torch.cuda.synchronize()
    us = np.array([ev[2 * s].elapsed_time(ev[2 * s + 1]) for s in range(K)]) * 1e3 / w.n_layers
    return {"workload": "tiny: 1 layer, H 256, 16 experts of I 128, top-2 + shared, 4-bit experts, bf16 router, T=1",
            "us_per_layer": {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
                             "p90": round(float(np.percentile(us, 90)), 2)}}


PHASES = ["layer start", "h staged", "phase A computed", "all logits seen", "top-k done",
          "routed loads issued", "routed pairs computed (wave 0)", "routed pairs computed (wave 7)",
          "routed activations stored", "first down inputs in LDS", "down rows done", "combine done",
          "shared down inputs fetched (wave 7)", "down rows requested", "down rows in LDS"]


def phase_trace(w, K: int, W: int) -> int:
    """Per-phase timestamps of the streaming stack kernel (phase-trace build only)."""
    import ctypes

    import torch

    from quantized_moe_decode_softmax_amd import _lib as Lb
    from quantized_moe_decode_softmax_amd.build import TRACE_LIB

    Lb.use_library(TRACE_LIB)
    from quantized_moe_decode_softmax_amd.runtime import DeviceStack

    if w.T != 1:
        print("--phase-trace covers the one-row streaming kernel (T = 1)", file=sys.stderr)
        return 2
    ds = DeviceStack.from_workload(w)
    f = Lb.lib().moe_phase_trace_offset
    f.argtypes = [ctypes.POINTER(Lb.moe_shape_t), ctypes.c_int32]
    f.restype = ctypes.c_int64
    off = f(ctypes.byref(ds.shape), 1)
    if off < 0:
        print("this library build records no phase timestamps", file=sys.stderr)
        return 2
    L, n_ph = w.n_layers, 16
    region = ds.ws[off:off + 64 * 512 * n_ph * 8].view(torch.int64).view(64, 512, n_ph)
    st = ds.state()
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty((1, w.hidden), dtype=torch.bfloat16, device="cuda")
    xs = [ds.rows(1000 + s, 1) for s in range(W + K)]
    recs = []
    for s in range(W + K):
        region.zero_()
        Lb.moe_stack_decode(st, 1, xs[s].data_ptr(), out.data_ptr(), None, None, None, stream)
        if s >= W:
            recs.append(region[:L].clone())
    torch.cuda.synchronize()
    if ds.status(1) != 0:
        print("a cross-workgroup wait timed out", file=sys.stderr)
        return 1
    r = torch.stack(recs).cpu().numpy()  # [K, 64, 512, 16]
    used = r[:, :, :, 0].any(axis=(0, 1))
    nwg = int(used.sum())
    r = r[:, :, :nwg].astype(np.float64)
    t0 = r[:, :, :, 0].min(axis=2, keepdims=True)  # earliest layer start over workgroups
    rel = (r - t0[..., None]) * 0.01  # 100 MHz ticks -> us
    valid = r > 0
    lay = slice(2, L)  # skip the first layers (cold start)
    print(f"phase timestamps, {w.name} T=1: {K} steps x layers {lay.start}..{L - 1} x {nwg} workgroups "
          f"(us after the earliest workgroup started the layer)")
    print(f"{'slot':>4} {'phase':<38} {'p10':>7} {'median':>7} {'p90':>7} {'max':>7}")
    rows = []
    for p, name in enumerate(PHASES):
        v = rel[:, lay, :, p][valid[:, lay, :, p]]
        if v.size == 0:
            continue
        q = np.percentile(v, [10, 50, 90]).tolist() + [float(v.max())]
        rows.append((p, name, q))
        print(f"{p:>4} {name:<38} {q[0]:7.2f} {q[1]:7.2f} {q[2]:7.2f} {q[3]:7.2f}")
    # layer duration: next layer's earliest start - this layer's earliest start
    starts = r[:, :L, :, 0].min(axis=2) * 0.01
    dur = np.diff(starts, axis=1)[:, lay.start:]
    print(f"layer duration (earliest start to earliest start): median {np.median(dur):.2f} us, "
          f"p10 {np.percentile(dur, 10):.2f}, p90 {np.percentile(dur, 90):.2f}")
    return 0


def bench_gemv(K: int, W: int, rows_per_step: int) -> int:
    """Dense 8-bit projections of the 35B-A3B shape through moe_gemv: per step,
    for each of the 10 full-attention layers a fused Q/K/V call (4096 + 512 +
    512 rows x 2048) and an attention output call (2048 x 4096), then one
    lm_head call (32768 x 2048, the draft vocabulary the PureDrive card names),
    each layer with its own seeded weights (272 MB per step, beyond the
    256 MB memory-side cache), T token rows from seeded x."""
    import torch

    from quantized_moe_decode_softmax_amd import _lib as Lb

    T = rows_per_step
    H, QD, KD, V, n_att = 2048, 16 * 256, 2 * 256, 32768, 10
    stream = torch.cuda.current_stream().cuda_stream

    def mat(rows, cols, layer, tensor):
        b = torch.empty(Lb.moe_matrix_bytes(8, rows, cols), dtype=torch.uint8, device="cuda")
        Lb.moe_generate_matrix(8, rows, cols, 0, layer, tensor, b.data_ptr(), stream)
        return b

    layers = [dict(q=mat(QD, H, l, 6), k=mat(KD, H, l, 7), v=mat(KD, H, l, 8), o=mat(H, QD, l, 9))
              for l in range(n_att)]
    lm = mat(V, H, 0, 10)
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    xo = torch.empty((T, QD), dtype=torch.bfloat16, device="cuda")
    Lb.moe_generate_rows(1000, T, H, x.data_ptr(), stream)
    Lb.moe_generate_rows(1001, T, QD, xo.data_ptr(), stream)
    yq = torch.empty((T, QD), dtype=torch.float32, device="cuda")
    yk = torch.empty((T, KD), dtype=torch.float32, device="cuda")
    yv = torch.empty((T, KD), dtype=torch.float32, device="cuda")
    yo = torch.empty((T, H), dtype=torch.float32, device="cuda")
    yl = torch.empty((T, V), dtype=torch.float32, device="cuda")
    alg = {"qkv": (QD + 2 * KD) * _matrix_alg_bytes(8, 1, H), "o_proj": _matrix_alg_bytes(8, H, QD),
           "lm_head": _matrix_alg_bytes(8, V, H)}
    ev = {k: [] for k in alg}

    def step(timed):
        for L in layers:
            e0 = torch.cuda.Event(enable_timing=True) if timed else None
            e1 = torch.cuda.Event(enable_timing=True) if timed else None
            e2 = torch.cuda.Event(enable_timing=True) if timed else None
            if timed:
                e0.record()
            Lb.moe_gemv(8, H, T, x.data_ptr(), [(L["q"].data_ptr(), QD, yq.data_ptr()),
                                                 (L["k"].data_ptr(), KD, yk.data_ptr()),
                                                 (L["v"].data_ptr(), KD, yv.data_ptr())], stream)
            if timed:
                e1.record()
            Lb.moe_gemv(8, QD, T, xo.data_ptr(), [(L["o"].data_ptr(), H, yo.data_ptr())], stream)
            if timed:
                e2.record()
                ev["qkv"].append((e0, e1))
                ev["o_proj"].append((e1, e2))
        e3 = torch.cuda.Event(enable_timing=True) if timed else None
        e4 = torch.cuda.Event(enable_timing=True) if timed else None
        if timed:
            e3.record()
        Lb.moe_gemv(8, H, T, x.data_ptr(), [(lm.data_ptr(), V, yl.data_ptr())], stream)
        if timed:
            e4.record()
            ev["lm_head"].append((e3, e4))

    for _ in range(W):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) / 1e3 for k, v in ev.items()}
    step_bytes = n_att * (alg["qkv"] + alg["o_proj"]) + alg["lm_head"]
    gbps = {k: alg[k] / per[k] / 1e9 for k in alg}
    res = {
        "metric": "dense 8-bit projection GEMV GB/s (fused Q/K/V, attention output, lm_head) vs 8 TB/s",
        "value": round(step_bytes * K / wall / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": (f"35B-A3B dense projections, T={T}: 10 x (fused QKV 5120x2048 + o-proj 2048x4096) "
                                f"+ lm_head 32768x2048, 8-bit group 64, seeded weights per layer"),
                   "T": T, "bytes_per_step": step_bytes},
        "per_call_us": {k: round(v * 1e6, 2) for k, v in per.items()},
        "per_call_GBps": {k: round(v, 1) for k, v in gbps.items()},
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel (lm_head call)", "achieved": round(gbps["lm_head"], 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps["lm_head"] / HBM_PEAK_GBPS, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_attn(K: int, W: int, T: int, ctx: int) -> int:
    """GQA decode attention of the 35B-A3B shape through moe_gqa_decode: 16
    query heads, 2 KV heads, head dim 256, bf16 K/V cache of `ctx` positions
    per layer (about 2 KB per position and layer, the card's ~20 KB per token
    over 10 attention layers); per step one call for each of the 10 layers
    (own caches), T verify rows at the end of the context."""
    import torch

    from quantized_moe_decode_softmax_amd import _lib as Lb

    n_q, n_kv, d, n_att = 16, 2, 256, 10
    stream = torch.cuda.current_stream().cuda_stream
    shape = Lb.moe_attn_shape_t(n_q, n_kv, d, ctx)
    caches = []
    for l in range(n_att):
        k = torch.empty((n_kv, ctx, d), dtype=torch.bfloat16, device="cuda")
        v = torch.empty((n_kv, ctx, d), dtype=torch.bfloat16, device="cuda")
        Lb.moe_generate_rows(2000 + 2 * l, n_kv * ctx, d, k.data_ptr(), stream)
        Lb.moe_generate_rows(2001 + 2 * l, n_kv * ctx, d, v.data_ptr(), stream)
        caches.append((k, v))
    q = torch.empty((T, n_q, d), dtype=torch.bfloat16, device="cuda")
    Lb.moe_generate_rows(77, T * n_q, d, q.data_ptr(), stream)
    o = torch.empty((T, n_q, d), dtype=torch.float32, device="cuda")
    wsb = Lb.moe_gqa_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    p0 = ctx - T
    kv_bytes = n_kv * ctx * d * 2 * 2  # K and V of every visible position, read once per call
    ev = []

    def step(timed):
        for k, v in caches:
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            Lb.moe_gqa_decode(shape, T, p0, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), ws.data_ptr(),
                              wsb, stream)
            if timed:
                e1.record()
                ev.append((e0, e1))

    for _ in range(W):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    res = {
        "metric": "GQA decode attention: KV-cache GB/s vs 8 TB/s",
        "value": round(kv_bytes / per / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic",
        "config": {"workload": (f"35B-A3B attention shape: 16 q / 2 KV heads, head dim 256, bf16 KV cache of {ctx} "
                                f"positions per layer, 10 layers, T={T} verify rows"), "T": T, "context": ctx,
                   "kv_bytes_per_call": kv_bytes},
        "per_call_us": round(per * 1e6, 2),
        "roofline": {"bound": "hbm", "kernel": "attn_partial_kernel + attn_combine_kernel (one call)",
                     "achieved": round(kv_bytes / per / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(kv_bytes / per / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_gdn(K: int, W: int, T: int) -> int:
    """Gated DeltaNet decode steps through moe_gdn_step: 30 layers (the card's
    30 GDN layers of the 35B-A3B model), each with its own fp32 state of 32
    value heads x 128 x 128 (16 key heads; a reading, the pages give no GDN
    shape), T tokens per call; the state is read and written once per call."""
    import torch

    from quantized_moe_decode_softmax_amd import _lib as Lb

    n_k, n_v, dk, dv, n_gdn = 16, 32, 128, 128, 30
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    states = [0.1 * torch.randn((n_v, dv, dk), generator=g, device="cuda") for _ in range(n_gdn)]
    q = torch.nn.functional.normalize(torch.randn((T, n_k, dk), generator=g, device="cuda"), dim=-1)
    k = torch.nn.functional.normalize(torch.randn((T, n_k, dk), generator=g, device="cuda"), dim=-1)
    v = torch.randn((T, n_v, dv), generator=g, device="cuda")
    al = 0.5 + 0.5 * torch.rand((T, n_v), generator=g, device="cuda")
    be = torch.rand((T, n_v), generator=g, device="cuda")
    o = torch.empty((T, n_v, dv), device="cuda")
    shape = Lb.moe_gdn_shape_t(n_k, n_v, dk, dv)
    state_bytes = n_v * dv * dk * 4
    ev = []

    def step(timed):
        for st in states:
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            Lb.moe_gdn_step(shape, T, st.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), al.data_ptr(),
                            be.data_ptr(), o.data_ptr(), stream)
            if timed:
                e1.record()
                ev.append((e0, e1))

    for _ in range(W):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    traffic = 2 * state_bytes  # read once, written once
    res = {
        "metric": "Gated DeltaNet decode step: state GB/s vs 8 TB/s", "value": round(traffic / per / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": (f"30 GDN layers, 16 key / 32 value heads of 128 x 128, fp32 state, T={T}"), "T": T,
                   "state_bytes_per_call": state_bytes},
        "per_call_us": round(per * 1e6, 2),
        "roofline": {"bound": "hbm", "kernel": "gdn_kernel (one call)", "achieved": round(traffic / per / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(traffic / per / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="a3b")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time per measured mode")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--rows", type=int, default=0, help="token rows per step (default: the workload's T)")
    ap.add_argument("--phase-trace", action="store_true", help="per-phase timestamps (phase-trace build)")
    ap.add_argument("--op", choices=["moe", "gemv", "attn", "gdn"], default="moe",
                    help="moe: the MoE stack (default); gemv: the dense projections of the 35B-A3B shape; "
                         "attn: GQA decode attention of the 35B-A3B shape")
    ap.add_argument("--ctx", type=int, default=131072, help="--op attn: context positions per layer")
    ap.add_argument("--api", choices=["stack", "pointers"], default="stack",
                    help="stack: moe_stack_init once + moe_stack_decode per step (layer pointers in the workspace); "
                         "pointers: moe_decode_stack with the host array of layer pointers per step")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this "
              "path is a design note, not a measured configuration", file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.op == "gemv":
        return bench_gemv(min(args.steps, 200), args.warmup, args.rows or 1)
    if args.op == "gdn":
        return bench_gdn(min(args.steps, 200), args.warmup, args.rows or 1)
    if args.op == "attn":
        return bench_attn(min(args.steps, 100), args.warmup, args.rows or 1, args.ctx)
    if args.phase_trace:
        from quantized_moe_decode_softmax_amd import WORKLOADS as _W

        return phase_trace(_W[args.workload], min(args.steps, 50), min(args.warmup, 10))

    import torch

    from quantized_moe_decode_softmax_amd import WORKLOADS
    from quantized_moe_decode_softmax_amd.runtime import DeviceStack

    w = WORKLOADS[args.workload]
    if args.rows:
        import dataclasses

        w = dataclasses.replace(w, T=args.rows)
    T, L, K, W = w.T, w.n_layers, args.steps, args.warmup
    ds = DeviceStack.from_workload(w)
    xs = [ds.rows(1000 + s, T) for s in range(W + K)]
    ids = torch.empty((K, L, T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((K, L, T, w.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, w.hidden), dtype=torch.bfloat16, device="cuda")
    from quantized_moe_decode_softmax_amd import _lib as Lb

    stream = torch.cuda.current_stream().cuda_stream
    st = ds.state()  # moe_stack_init: the descriptor table of the 40 layers in the workspace, once
    ptrs = [b.data_ptr() for b in ds.layers]

    def step(x, idp, wp):
        if args.api == "stack":
            Lb.moe_stack_decode(st, T, x.data_ptr(), out.data_ptr(), idp, wp, None, stream)
        else:
            Lb.moe_decode_stack(ds.shape, ptrs, T, x.data_ptr(), out.data_ptr(), idp, wp, None, ds.ws.data_ptr(),
                                ds.ws_bytes, stream)

    for s in range(W):
        step(xs[s], ids[0].data_ptr(), wts[0].data_ptr())
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
    t0 = time.perf_counter()
    for s in range(K):
        ev[2 * s].record()
        step(xs[W + s], ids[s].data_ptr(), wts[s].data_ptr())
        ev[2 * s + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = np.array([ev[2 * s].elapsed_time(ev[2 * s + 1]) for s in range(K)])
    launch_s = float(np.mean(call_ms)) / 1e3
    st = ds.status(T)
    if st != 0:
        print(f"stack kernel status {st}: a cross-workgroup wait timed out", file=sys.stderr)
        return 1
    ids_h = ids.cpu().numpy()
    tb = touched_bytes(w, ids_h)
    # unique routed experts per layer and step (the union over the T rows)
    units = np.array([len(np.unique(ids_h[s, l])) for s in range(K) for l in range(L)])
    tok_s = T * K / wall
    gbps = tb / (wall * 1e9)
    kernel_gbps = tb / K / launch_s / 1e9
    tr = TRAFFIC.get(args.workload) if T == WORKLOADS[args.workload].T else None
    traffic = traffic_detail = None
    if tr is not None and tr["src_hash"] == kernel_source_hash():
        traffic = tr["fetch_bytes"] + tr["write_bytes"]
        traffic_detail = {"fetch_bytes": tr["fetch_bytes"], "write_bytes": tr["write_bytes"],
                          "vs_touched_bytes": round(traffic / (tb / K), 3)}
    res = {
        "metric": "MoE-stack decode tokens/s + achieved HBM GB/s on touched expert bytes vs 8 TB/s",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: {L}-layer MoE stack, H {w.hidden}, {w.n_experts} experts of I {w.inter}, "
                         f"top-{w.top_k} + shared (I {w.shared_inter}), {w.expert_bits}-bit routed / "
                         f"{w.shared_bits}-bit shared / "
                         f"{'bf16' if w.router_bits == 16 else str(w.router_bits) + '-bit'} router, group 64, "
                         f"T={T}, seeded weights resident in HBM, fresh x per step"),
            "T": T,
            "layers": L,
            "touched_bytes_per_step": tb // K,
        },
        "achieved_GBps": round(gbps, 1),
        "step_us": {"median": round(float(np.median(call_ms)) * 1e3, 1),
                    "p10": round(float(np.percentile(call_ms, 10)) * 1e3, 1),
                    "p90": round(float(np.percentile(call_ms, 90)) * 1e3, 1)},
        "unique_experts_per_layer": round(float(units.mean()), 2),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": f"{kernel_path(w)}, mean call {launch_s * 1e6:.1f} us",
            "achieved": round(kernel_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(kernel_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_detail": traffic_detail,
        },
    }
    if args.workload == "a3b" and not args.rows:
        res["config0_gpu"] = config0_gpu()
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
