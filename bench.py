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
* cpu_baseline: the fp64 oracle timed on this host on a bounded sample.

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
KERNEL_SOURCES = ["stack1.hip", "gemv.h", "device_common.h"]  # the stack kernel's device code

# HBM traffic of one stack-kernel launch, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over
# `bench.py --steps 5 --warmup 2 --no-cpu`, each scaled by bytes/counter of a
# 256 MiB device copy measured the same way. Keyed by workload; valid only
# for the kernel sources whose hash is stored with it.
TRAFFIC = {
    "a3b": {"src_hash": "af6e4a3aa94bd18a", "fetch_bytes": 996_328_853, "write_bytes": 55_063_808},
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
        return (f"per-layer kernels: route_mfma, down_mfma, select, expert, down per layer ({w.n_layers} "
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


def cpu_baseline(w, budget_s: float = 15.0):
    """The oracle as it stands: token rows through the layer stack, in order, until the budget is spent."""
    import oracle
    from oracle.gen import GeneratedLayer, MoEShape, gen_x

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    sh = MoEShape(hidden=w.hidden, n_experts=w.n_experts, inter=w.inter, top_k=w.top_k,
                  shared_inter=w.shared_inter, router_bits=w.router_bits, expert_bits=w.expert_bits,
                  shared_bits=w.shared_bits, eps=w.rms_eps)
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        n = 0  # layer passes done
        tokens = 0
        while time.perf_counter() - t0 < budget_s:
            h = gen_x(1000 + tokens, 1, w.hidden)
            for layer in range(w.n_layers):
                r = oracle.layer_forward(GeneratedLayer(sh, 0, layer), h)
                h = oracle.bf16_round(r["y"])
                n += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            tokens += 1
        dt = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    per_token = dt / n * w.n_layers
    return {
        "value": 1.0 / per_token,
        "unit": "tok/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{n} layer passes ({tokens} token(s), x seeds from 1000, through the {w.n_layers}-layer "
                   f"stack in order) in {dt:.1f} s, fp64 numpy incl. regenerating the selected experts, BLAS "
                   f"limited to 1 thread; scaled to {w.n_layers} layers per token"),
        "host_cpus": os.cpu_count(),
    }


PHASES = ["layer start", "h staged", "phase A computed", "all logits seen", "top-k done",
          "routed loads issued", "routed pairs computed (wave 0)", "routed pairs computed (wave 7)",
          "activations published", "first down inputs in LDS", "down rows done", "combine done",
          "shared down inputs fetched (wave 7)"]


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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="a3b")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--rows", type=int, default=0, help="token rows per step (default: the workload's T)")
    ap.add_argument("--phase-trace", action="store_true", help="per-phase timestamps (phase-trace build)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this "
              "path is a design note, not a measured configuration", file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe(args.copy_probe)
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

    def step(x, idp, wp):
        Lb.moe_stack_decode(st, T, x.data_ptr(), out.data_ptr(), idp, wp, None, stream)

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
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
