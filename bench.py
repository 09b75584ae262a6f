#!/usr/bin/env python3
"""Throughput of causal packed attention fwd+bwd on one MI355X, as one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is one pass of the whole hot path over one batch of resident synthetic input: the
forward call (work list + fused forward) and the backward call (work list + D = rowsum(dO∘O)
+ dK/dV + dQ). Inputs are generated on the host from a fixed seed and uploaded before the
timed region. ``value`` is causal TFLOP/s with the FLOP convention 3.5 × 4·d·hq·Σ L(L+1)/2.

``roofline`` describes the dominant kernel (largest share of the step): its algorithmic FLOPs
per launch divided by its mean launch time, both measured here with HIP events recorded by
the library around that kernel on the bench stream during the timed steps. Algorithmic FLOPs
per kernel follow the same convention: forward = 2 GEMM units (S, PV); dK/dV = 4 units
(S, dP, dV, dK); dQ = 1 unit (dQ; its S/dP recompute is not counted); one unit = 2·d·hq·Σ
L(L+1)/2. ``traffic`` comes from committed rocprofv3 counter summaries (profiles/), and is
null when the kernel source changed since they were taken.

``cpu_baseline`` times the float64 oracle (naive two-pass attention with an explicit mask)
on a bounded sample of the same workload on the host cores, and reports its causal FLOP rate.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp32": 157.3}   # MI355X dense MFMA / vector fp32
HBM_PEAK_GBS = 8000.0
METRIC = "causal fwd+bwd attention TFLOP/s and % of MFMA peak (bf16, MXFP8), 1 GPU"

KERNELS = {  # name -> (call, index in that call's event list, GEMM units counted)
    "attn_fwd_bf16_kernel": ("fwd", 0, 2.0),
    "bwd_pre_kernel": ("bwd", 0, 0.0),
    "attn_bwd_dkdv_kernel": ("bwd", 1, 4.0),
    "attn_bwd_dq_kernel": ("bwd", 2, 1.0),
}
KERNEL_SOURCES = {
    "attn_fwd_bf16_kernel": "attn_fwd.hip",
    "bwd_pre_kernel": "attn_bwd.hip",
    "attn_bwd_dkdv_kernel": "attn_bwd.hip",
    "attn_bwd_dq_kernel": "attn_bwd.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 5],
                    help="seeded workload number (3 = one 32K-token document, 32 q / 8 kv heads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    return ap.parse_args()


def source_hash(fname):
    with open(os.path.join(ROOT, "causal_flashattention_amd", "csrc", fname), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel, workload_name):
    """HBM bytes per launch from a committed counter summary, if it matches the current source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, sample_tokens):
    """Oracle fwd+bwd on one kv group (all its query heads) of the longest document's prefix."""
    import threadpoolctl
    from oracle import attention as ref
    cu = w.cu_seqlens
    L = np.diff(cu)
    n = int(np.argmax(L))
    s0 = int(cu[n])
    P = int(min(sample_tokens, L[n]))
    G = w.hq // w.hkv
    hs = list(range(G))
    q = _f64(w.q[s0:s0 + P][:, hs])
    k = _f64(w.k[s0:s0 + P][:, [0]])
    v = _f64(w.v[s0:s0 + P][:, [0]])
    do = _f64(w.do[s0:s0 + P][:, hs])
    scu = np.array([0, P])
    t0 = time.perf_counter()
    ref.attn_fwd(q, k, v, scu, w.scale)
    ref.attn_bwd(q, k, v, do, scu, w.scale)
    dt = time.perf_counter() - t0
    from causal_flashattention_amd import workloads as W
    fl = W.causal_flops_fwd_bwd(scu, G, w.d)
    threads = max([p["num_threads"] for p in threadpoolctl.threadpool_info() if p["user_api"] == "blas"] or [1])
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle fwd+bwd, 1 kv head with its {G} query heads, first {P} tokens of the "
                      f"longest document ({fl / 1e9:.1f} causal GFLOP in {dt:.1f} s)",
            "seconds": dt}


def _f64(a):
    from causal_flashattention_amd import workloads as W
    return W.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention path has no multi-GPU exchange in this "
              "library; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import causal_flashattention_amd as cfa
    from causal_flashattention_amd import workloads as W
    from causal_flashattention_amd import _lib

    w = W.make_workload(args.workload)
    dev = "cuda:0"

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = up(w.q), up(w.k), up(w.v), up(w.do)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    cu_h = torch.from_numpy(w.cu_seqlens)
    T, hq, hkv, d = w.total_tokens, w.hq, w.hkv, w.d
    o = torch.empty_like(q)
    lse = torch.empty((hq, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_f = torch.empty(cfa.workspace_bytes(0, T, w.n_docs, hq, hkv, d, cfa.CFA_BF16), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(cfa.workspace_bytes(1, T, w.n_docs, hq, hkv, d, cfa.CFA_BF16), dtype=torch.uint8, device=dev)
    L = _lib.lib()
    import ctypes

    def step():
        cfa.attn_fwd(q, k, v, cu, scale=w.scale, cu_seqlens_host=cu_h, out=o, lse=lse, workspace=ws_f)
        cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=w.scale, cu_seqlens_host=cu_h, dq=dq, dk=dk, dv=dv,
                     workspace=ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel events, recorded by the library around each main kernel of each timed step
    K = args.steps
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for name in KERNELS}
    for name in ev:
        for a, b in ev[name]:
            a.record(); b.record()          # create the underlying HIP events
    torch.cuda.synchronize()

    def handles(call, i):
        names = [n for n, (c, _, _) in KERNELS.items() if c == call]
        names.sort(key=lambda n: KERNELS[n][1])
        arr = (ctypes.c_void_p * (2 * len(names)))()
        for j, n in enumerate(names):
            a, b = ev[n][i]
            arr[2 * j] = a.cuda_event
            arr[2 * j + 1] = b.cuda_event
        return arr, len(names)

    fwd_h = [handles("fwd", i) for i in range(K)]
    bwd_h = [handles("bwd", i) for i in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        _lib.check(L.cfa_set_kernel_events(fwd_h[i][0], fwd_h[i][1]))
        cfa.attn_fwd(q, k, v, cu, scale=w.scale, cu_seqlens_host=cu_h, out=o, lse=lse, workspace=ws_f)
        _lib.check(L.cfa_set_kernel_events(bwd_h[i][0], bwd_h[i][1]))
        cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=w.scale, cu_seqlens_host=cu_h, dq=dq, dk=dk, dv=dv,
                     workspace=ws_b)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _lib.check(L.cfa_set_kernel_events(None, 0))

    elapsed = t1 - t0
    ms_per_step = elapsed / K * 1e3
    flops = w.flops_fwd_bwd()
    value = flops / (elapsed / K) / 1e12
    unit_flops = w.flops_fwd() / 2.0          # one GEMM unit over the causal pairs
    kern = {}
    for name, (_, _, units) in KERNELS.items():
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[name]]))
        kern[name] = {"ms": ms, "units": units}
    dom = max(kern, key=lambda n: kern[n]["ms"])
    dom_flops = kern[dom]["units"] * unit_flops
    achieved = dom_flops / (kern[dom]["ms"] * 1e-3) / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
            "frac": achieved / PEAK_TFLOPS["bf16"], "traffic": traffic_for(dom, w.name),
            "algorithmic_flop_per_launch": dom_flops, "mean_launch_ms": kern[dom]["ms"]}
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "pct_of_peak": 100.0 * value / PEAK_TFLOPS["bf16"],
        "config": {"workload": w.name, "total_tokens": T, "n_docs": w.n_docs, "hq": hq, "hkv": hkv, "d": d,
                   "causal": True, "seed": w.info["seed"], "causal_tflop_per_step": flops / 1e12},
        "kernels_ms": {n: round(kern[n]["ms"], 4) for n in kern},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
