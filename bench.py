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
(S, dP, dV, dK); dQ = 1 unit (dQ; its S/dP recompute is not counted); with CFA_DQ_MODE=fused the
bf16 backward at d = 128 runs dK, dV and dQ in one pass, 5 units; one unit = 2·d·hq·Σ L(L+1)/2. ``traffic`` comes from committed rocprofv3 counter summaries (profiles/), and is
null when the kernel source changed since they were taken.

``cpu_baseline`` times the float64 oracle (naive two-pass attention with an explicit mask)
on a bounded sample of the same workload on the host cores, and reports its causal FLOP rate.

The same line carries the MX paths on the 65K-token packed workload: ``mxfp8`` (E4M3 operands),
``mxfp4`` and ``mxfp6`` (E2M1 / E2M3 score product, the rest as mxfp8), each with its own
``roofline``. Their ``pct_of_peak`` and roofline ``peak`` are the dense MFMA peak of the path's
format (fp8 5.0 PFLOP/s; fp4 / fp6 10.1) although the dS products and diagonal tiles run in
bf16; the blended peak of the counted units' formats (n / Σ 1/peak) is ``mixed_peak``.
``--mx6-e3m2-workload 4`` adds ``mxfp6_e3m2`` (E3M2 score product), off by default.

    python bench.py --decode      # decoding over a packed KV cache: GB/s against HBM peak
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

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp6": 10100.0, "fp4": 10100.0, "fp32": 157.3}   # MI355X dense MFMA / vector fp32
# Counted GEMM units per MX kernel and the format each runs in ("qk": the score product, E4M3 on
# the MXFP8 path and E2M1 on the MXFP4/FP8 path). A mixed kernel's peak is the rate at which its
# counted units would run if each ran at its format's peak: n / Σ 1/peak.
# dK = dSᵀQ and dQ = dS·K run as bf16 products on the MX paths (bf16 dS and bf16 Q / K rows)
MX_UNIT_FORMATS = {"attn_fwd_mx_kernel": ["qk", "fp8"], "attn_bwd_dkdv_mx_kernel": ["qk", "fp8", "fp8", "bf16"],
                   "attn_bwd_dq_mx_kernel": ["bf16"]}
# the whole fwd+bwd step under the 3.5× convention: S twice (fwd, bwd recompute), PV, dP, dV, dK, dQ
MX_STEP_FORMATS = ["qk", "qk", "fp8", "fp8", "fp8", "bf16", "bf16"]


def mixed_peak(formats, qk_fmt):
    return len(formats) / sum(1.0 / PEAK_TFLOPS[qk_fmt if f == "qk" else f] for f in formats)
HBM_PEAK_GBS = 8000.0
METRIC = "causal fwd+bwd attention TFLOP/s and % of MFMA peak (bf16, MXFP8), 1 GPU"

# name -> (call, index in that call's event list, GEMM units counted); see cfa_set_kernel_events
KERNELS_BF16 = {
    "attn_fwd_bf16_kernel": ("fwd", 0, 2.0),
    "bwd_pre_kernel": ("bwd", 0, 0.0),
    "attn_bwd_dkdv_kernel": ("bwd", 1, 4.0),
    "attn_bwd_dq_kernel": ("bwd", 2, 1.0),
}
# d = 128 bf16 backward with dQ summed inside the dK/dV pass (CFA_DQ_MODE=fused; the default is
# the separate dQ pass above): S, dP, dV, dK and dQ, 5 units
KERNELS_BF16_FUSED = {
    "attn_fwd_bf16_kernel": ("fwd", 0, 2.0),
    "bwd_pre_kernel": ("bwd", 0, 0.0),
    "attn_bwd_dkdv_dq_kernel": ("bwd", 1, 5.0),
}
# MX: one operand pass per direction -- mx_prep_fwd_kernel writes K_d, V_d and V_t from one read of
# K and V (the MX forward kernel quantises Q from the rows it reads); mx_prep_bwd_kernel writes D,
# dO_d and dO_t from one read of O and dO
KERNELS_MX = {
    "attn_fwd_mx_kernel": ("fwd", 0, 2.0),
    "mx_prep_fwd_kernel": ("fwd", 1, 0.0),
    "mx_prep_bwd_kernel": ("bwd", 0, 0.0),
    "attn_bwd_dkdv_mx_kernel": ("bwd", 1, 4.0),
    "attn_bwd_dq_mx_kernel": ("bwd", 2, 1.0),
}
KERNEL_SOURCES = {
    "attn_fwd_bf16_kernel": "attn_fwd.hip",
    "bwd_pre_kernel": "attn_bwd.hip",
    "attn_bwd_dkdv_kernel": "attn_bwd.hip",
    "attn_bwd_dq_kernel": "attn_bwd.hip",
    "attn_bwd_dkdv_dq_kernel": "attn_bwd.hip",
    "attn_fwd_mx_kernel": "attn_fwd_mx.hip",
    "attn_bwd_dkdv_mx_kernel": "attn_bwd_mx.hip",
    "attn_bwd_dq_mx_kernel": "attn_bwd_mx.hip",
    "mx_prep_fwd_kernel": "mx_quantize.hip",
    "mx_prep_bwd_kernel": "mx_quantize.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 5],
                    help="bf16 workload (3 = one 32K-token document, 32 q / 8 kv heads)")
    ap.add_argument("--mx-workload", type=int, default=4, choices=[0, 4, 5],
                    help="MXFP8 workload reported under 'mxfp8' (0 = skip)")
    ap.add_argument("--mx4-workload", type=int, default=4, choices=[0, 4, 5],
                    help="MXFP4/FP8 workload reported under 'mxfp4' (0 = skip)")
    ap.add_argument("--mx6-workload", type=int, default=4, choices=[0, 4, 5],
                    help="MXFP6/FP8 workload reported under 'mxfp6' (0 = skip)")
    ap.add_argument("--mx6-e3m2-workload", type=int, default=0, choices=[0, 4, 5],
                    help="MXFP6/FP8 with E3M2 score operands, reported under 'mxfp6_e3m2' (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--doc-order", default="drawn", choices=["drawn", "longest-last"],
                    help="pack each workload's documents as drawn, or sorted shortest first (the order "
                         "that is worst for handing out work by document index)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 3 times (to scale the "
                         "FETCH_SIZE/WRITE_SIZE counters against a kernel of known traffic) and exit")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768)
    ap.add_argument("--decode", action="store_true",
                    help="instead: time decoding over a packed KV cache (bf16 and MX caches; one JSON line)")
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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, sample_tokens):
    """Oracle fwd+bwd on one kv group (all its query heads) of the longest document's prefix.

    The oracle as it stands (``oracle.attention.attn_rows``: every quantity of a query row from
    its own softmax row, with partial dK/dV sums) split into (query head, query range) units of
    equal causal work, run on a thread pool with one BLAS thread per worker, so that ``cores``
    is the number of threads that actually ran (NumPy releases the GIL in array operations)."""
    import concurrent.futures as cf

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
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, 16))
    n_ranges = max(1, (2 * workers + G - 1) // G)
    b = [0] + [int(P * math.sqrt(i / n_ranges)) for i in range(1, n_ranges)] + [P]
    tasks = [(h, np.arange(b[i], b[i + 1])) for h in range(G) for i in range(n_ranges) if b[i + 1] > b[i]]
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(1), cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda t: ref.attn_rows(q[:, [t[0]]], k, v, do[:, [t[0]]], t[1], w.scale), tasks))
    dt = time.perf_counter() - t0
    from causal_flashattention_amd import workloads as W
    fl = W.causal_flops_fwd_bwd(np.array([0, P]), G, w.d)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"float64 oracle fwd+bwd (attn_rows), 1 kv head with its {G} query heads, first {P} tokens "
                      f"of the longest document, {len(tasks)} (head, query range) units on {workers} threads "
                      f"with 1 BLAS thread each ({fl / 1e9:.1f} causal GFLOP in {dt:.1f} s)",
            "seconds": dt, "cpu_model": _cpu_model(), "affinity_cores": affinity, "workers": workers,
            "blas_threads_per_worker": 1}


def _f64(a):
    from causal_flashattention_amd import workloads as W
    return W.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def operand_pass_rates(w, qk_fmt, kern):
    """Algorithmic HBM bytes of the two MX operand passes (every input read once, every copy
    written once, padding columns of the token-blocked copies included) over their event time."""
    T, hq, hkv, d = w.total_tokens, w.hq, w.hkv, w.d
    t_pad = 32 * ((T + 31) // 32) + 32 * w.n_docs
    code = {"fp8": 1.0, "fp4": 0.5, "fp6": 0.75}[qk_fmt]
    sc = 1.0 / 32
    fwd = (2 * T * (2 * hkv) * d                            # K, V read (bf16); Q is quantised by
           + T * hkv * d * (code + sc)                       # K_d (score format)   the forward kernel
           + T * hkv * d * (1 + sc)                          # V_d (E4M3)
           + hkv * d * t_pad * (1 + sc))                     # V_t (E4M3, padded columns)
    bwd = (2 * 2 * T * hq * d                                # O, dO read (bf16)
           + 4 * T * hq                                      # D written (fp32)
           + T * hq * d * (1 + sc)                           # dO_d
           + hq * d * t_pad * (1 + sc))                      # dO_t
    out = {}
    for name, nbytes in (("mx_prep_fwd_kernel", fwd), ("mx_prep_bwd_kernel", bwd)):
        ms = kern[name]["ms"]
        out[name] = {"algorithmic_bytes": nbytes, "ms": ms, "GB_per_s": nbytes / (ms * 1e-3) / 1e9,
                     "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def measure(w, mx, steps, warmup):
    """Warm up, then time `steps` fwd+bwd steps; per-kernel HIP events inside the timed region."""
    import ctypes
    import torch
    import causal_flashattention_amd as cfa
    from causal_flashattention_amd import _lib

    dev = "cuda:0"

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = up(w.q), up(w.k), up(w.v), up(w.do)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    cu_h = torch.from_numpy(w.cu_seqlens)
    T, hq, hkv, d = w.total_tokens, w.hq, w.hkv, w.d
    dt = {"mxfp4": cfa.CFA_MXFP4, "mxfp6": cfa.CFA_MXFP6, "mxfp6_e3m2": cfa.CFA_MXFP6_E3M2}.get(
        mx, cfa.CFA_MXFP8 if mx else cfa.CFA_BF16)
    qk_fmt = {"mxfp4": "fp4", "mxfp6": "fp6", "mxfp6_e3m2": "fp6"}.get(mx, "fp8")
    o = torch.empty_like(q)
    lse = torch.empty((hq, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_f = torch.empty(cfa.workspace_bytes(0, T, w.n_docs, hq, hkv, d, dt), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(cfa.workspace_bytes(1, T, w.n_docs, hq, hkv, d, dt), dtype=torch.uint8, device=dev)
    saved = torch.empty(max(cfa.saved_bytes(T, w.n_docs, hq, hkv, d, dt), 256), dtype=torch.uint8, device=dev) \
        if mx else None
    L = _lib.lib()
    fused = not mx and d == 128 and os.environ.get("CFA_DQ_MODE") == "fused"
    kernels = KERNELS_MX if mx else (KERNELS_BF16_FUSED if fused else KERNELS_BF16)

    def fwd():
        cfa.attn_fwd(q, k, v, cu, scale=w.scale, cu_seqlens_host=cu_h, out=o, lse=lse, workspace=ws_f, mx=mx,
                     saved=saved)

    def bwd():
        cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=w.scale, cu_seqlens_host=cu_h, dq=dq, dk=dk, dv=dv,
                     workspace=ws_b, mx=mx, saved=saved)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    K = steps
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for n in kernels}
    for n in ev:
        for a, b in ev[n]:
            a.record()
            b.record()          # creates the underlying HIP events
    torch.cuda.synchronize()

    def handles(call, i):
        names = sorted([n for n, (c, _, _) in kernels.items() if c == call], key=lambda n: kernels[n][1])
        arr = (ctypes.c_void_p * (2 * len(names)))()
        for n in names:
            a, b = ev[n][i]
            arr[2 * kernels[n][1]] = a.cuda_event
            arr[2 * kernels[n][1] + 1] = b.cuda_event
        return arr, len(names)

    fwd_h = [handles("fwd", i) for i in range(K)]
    bwd_h = [handles("bwd", i) for i in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        _lib.check(L.cfa_set_kernel_events(fwd_h[i][0], fwd_h[i][1]))
        fwd()
        _lib.check(L.cfa_set_kernel_events(bwd_h[i][0], bwd_h[i][1]))
        bwd()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _lib.check(L.cfa_set_kernel_events(None, 0))

    elapsed = t1 - t0
    flops = w.flops_fwd_bwd()
    value = flops / (elapsed / K) / 1e12
    unit_flops = w.flops_fwd() / 2.0
    kern = {n: {"ms": float(np.mean([a.elapsed_time(b) for a, b in ev[n]])), "units": u}
            for n, (_, _, u) in kernels.items()}
    # per-step spread from the same events: first forward kernel's start to the last backward
    # kernel's end (the forward's plan launch, ~13 us, precedes the span)
    first = "mx_prep_fwd_kernel" if mx else "attn_fwd_bf16_kernel"      # launch order, not event slot
    last = "attn_bwd_dq_mx_kernel" if mx else ("attn_bwd_dkdv_dq_kernel" if fused else "attn_bwd_dq_kernel")
    spans = [ev[first][i][0].elapsed_time(ev[last][i][1]) for i in range(K)]
    dom = max(kern, key=lambda n: kern[n]["ms"])
    dom_flops = kern[dom]["units"] * unit_flops
    # MX legs: % of the dense MFMA peak of the path's own format (MXFP8: fp8; MXFP4/6: the
    # score product's fp4/fp6), whatever some products run in; the blended peak of the counted
    # units' formats is reported beside it
    peak = PEAK_TFLOPS[qk_fmt] if mx else PEAK_TFLOPS["bf16"]
    dom_peak = PEAK_TFLOPS[qk_fmt] if mx else PEAK_TFLOPS["bf16"]
    achieved = dom_flops / (kern[dom]["ms"] * 1e-3) / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": dom_peak, "unit": "TFLOP/s",
            "frac": achieved / dom_peak,
            "traffic": traffic_for(dom, w.name.replace("mxfp8", mx) if mx in ("mxfp4", "mxfp6", "mxfp6_e3m2") else w.name),
            "algorithmic_flop_per_launch": dom_flops, "mean_launch_ms": kern[dom]["ms"]}
    if mx:
        roof["mixed_peak"] = mixed_peak(MX_UNIT_FORMATS[dom], qk_fmt)
    res = {"value": value, "ms_per_step": elapsed / K * 1e3,
           "step_ms_events": {"median": float(np.median(spans)), "min": float(np.min(spans)),
                              "max": float(np.max(spans))},
           "pct_of_peak": 100.0 * value / peak, "peak": peak,
           **({"pct_of_fp8_peak": 100.0 * value / PEAK_TFLOPS["fp8"],
               "pct_of_mixed_peak": 100.0 * value / mixed_peak(MX_STEP_FORMATS, qk_fmt),
               "mixed_peak": mixed_peak(MX_STEP_FORMATS, qk_fmt)} if mx else {}),
           "config": {"workload": w.name, "total_tokens": T, "n_docs": w.n_docs, "hq": hq, "hkv": hkv, "d": d,
                      "causal": True, "seed": w.info["seed"], "causal_tflop_per_step": flops / 1e12,
                      **({"doc_order": w.info["doc_order"]} if "doc_order" in w.info else {}),
                      **({"schedule": "naive"} if os.environ.get("CFA_SCHED") == "naive" else {})},
           "kernels_ms": {n: round(kern[n]["ms"], 4) for n in kern}, "roofline": roof}
    if mx:
        res["operand_passes"] = operand_pass_rates(w, qk_fmt, kern)
    del q, k, v, do, o, lse, dq, dk, dv, ws_f, ws_b, saved
    torch.cuda.empty_cache()
    return res


def measure_decode(w, steps, warmup):
    """Time attn_decode on resident inputs: wall clock over `steps` calls, and per-kernel HIP
    events (0 = chunk partials, 1 = merge). Algorithmic bytes = the cache read once (K and V
    codes + scales, or bf16) + Q read + O written."""
    import ctypes
    import torch
    import causal_flashattention_amd as cfa
    from causal_flashattention_amd import _lib

    dev = "cuda:0"

    def bf(a):
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)

    q = bf(w.q)
    if w.kv == "mxfp8":
        k, v = torch.from_numpy(w.k).to(dev), torch.from_numpy(w.v).to(dev)
        ks, vs = torch.from_numpy(w.k_scales).to(dev), torch.from_numpy(w.v_scales).to(dev)
    else:
        k, v, ks, vs = bf(w.k), bf(w.v), None, None
    cu = torch.from_numpy(w.cu_seqlens_k.astype(np.int32)).to(dev)
    cu_h = torch.from_numpy(w.cu_seqlens_k.astype(np.int32))
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.n_seqs), dtype=torch.float32, device=dev)
    kvd = cfa.CFA_MXFP8 if w.kv == "mxfp8" else cfa.CFA_BF16
    ws = torch.empty(_lib.lib().cfa_decode_workspace_bytes(w.n_seqs, w.total_k, w.hq, w.hkv, w.d, kvd),
                     dtype=torch.uint8, device=dev)
    L = _lib.lib()

    def call():
        cfa.attn_decode(q, k, v, cu, k_scales=ks, v_scales=vs, scale=w.scale, cu_seqlens_k_host=cu_h, out=o,
                        lse=lse, workspace=ws)

    for _ in range(warmup):
        call()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in ev:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    arrs = []
    for e in ev:
        a = (ctypes.c_void_p * 4)()
        for j in range(4):
            a[j] = e[j].cuda_event
        arrs.append(a)
    t0 = time.perf_counter()
    for i in range(steps):
        _lib.check(L.cfa_set_kernel_events(arrs[i], 2))
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _lib.check(L.cfa_set_kernel_events(None, 0))
    main_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    comb_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    step_s = (t1 - t0) / steps
    nbytes = w.kv_bytes() + 2 * 2.0 * w.n_seqs * w.hq * w.d
    achieved = nbytes / (main_ms * 1e-3) / 1e9
    return {"kv": w.kv, "value": nbytes / step_s / 1e9, "unit": "GB/s (algorithmic bytes / wall time per call)",
            "ms_per_call": step_s * 1e3, "tokens_per_s": w.n_seqs / step_s,
            "kernels_ms": {"attn_decode_kernel": round(main_ms, 4), "attn_decode_combine_kernel": round(comb_ms, 4)},
            "roofline": {"kernel": "attn_decode_kernel", "bound": "hbm", "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "algorithmic_bytes_per_launch": nbytes, "mean_launch_ms": main_ms}}


def main_decode(args):
    from causal_flashattention_amd import workloads as W

    cases = {"decode_batch64": (W.decode_batch_lengths(seed=7, n_seqs=64), 32, 8),
             "decode_one_32k": ([32768], 32, 8)}
    out = {"metric": "decode over a packed KV cache, GB/s of cache read (1 GPU)", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "data": "synthetic", "results": []}
    for name, (lengths, hq, hkv) in cases.items():
        for kv in ("bf16", "mxfp8"):
            w = W.make_decode(seed=11, lengths=lengths, hq=hq, hkv=hkv, kv=kv)
            r = measure_decode(w, args.steps, args.warmup)
            r["config"] = {"workload": name, "n_seqs": w.n_seqs, "total_k": w.total_k, "hq": hq, "hkv": hkv,
                           "d": w.d, "seed": 11}
            out["results"].append(r)
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention path has no multi-GPU exchange in this "
              "library; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        import torch
        a = torch.empty(args.copy_calibration // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        for i in range(3):
            b.copy_(a)
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
        nb = a.numel() * 2
        # the device copy's own rate (read + write bytes over its time): the practical ceiling of a
        # pass that reads and writes comparable amounts, next to the 8 TB/s datasheet figure
        print(json.dumps({"copy_calibration_bytes": nb, "copy_ms": ms,
                          "copy_GB_per_s": 2 * nb / (min(ms[1:]) * 1e-3) / 1e9}))
        return
    if args.decode:
        main_decode(args)
        return
    from causal_flashattention_amd import workloads as W

    def load(k):
        wk = W.make_workload(k)
        return W.longest_last(wk) if args.doc_order == "longest-last" else wk

    w = load(args.workload)
    head = measure(w, False, args.steps, args.warmup)
    out = {
        "metric": METRIC, "value": head["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "pct_of_peak": head["pct_of_peak"],
        "config": head["config"], "kernels_ms": head["kernels_ms"], "roofline": head["roofline"],
        "step_ms_events": head["step_ms_events"],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens)
    del w
    if args.mx_workload:
        wm = load(args.mx_workload)
        mres = measure(wm, True, args.steps, args.warmup)
        mres["dtype"] = "mxfp8 (E4M3 + E8M0 per 32; the dS products dK = dS^T Q and dQ = dS K and the diagonal tiles in bf16)"
        mres["unit"] = "TFLOP/s"
        out["mxfp8"] = mres
    if args.mx4_workload:
        wm = load(args.mx4_workload)
        mres = measure(wm, "mxfp4", args.steps, args.warmup)
        mres["dtype"] = "mxfp4/fp8 (QK^T on E2M1 + E8M0 per 32, the rest as mxfp8)"
        mres["unit"] = "TFLOP/s"
        mres["peak_note"] = "pct_of_peak against fp4 10.1 PFLOP/s; mixed_peak = n / sum(1/peak) over the counted GEMM units"
        out["mxfp4"] = mres
    if args.mx6_workload:
        wm = load(args.mx6_workload)
        mres = measure(wm, "mxfp6", args.steps, args.warmup)
        mres["dtype"] = "mxfp6/fp8 (QK^T on E2M3 + E8M0 per 32, the rest as mxfp8)"
        mres["unit"] = "TFLOP/s"
        mres["peak_note"] = "pct_of_peak against fp6 10.1 PFLOP/s; mixed_peak = n / sum(1/peak) over the counted GEMM units"
        out["mxfp6"] = mres
    if args.mx6_e3m2_workload:
        wm = load(args.mx6_e3m2_workload)
        mres = measure(wm, "mxfp6_e3m2", args.steps, args.warmup)
        mres["dtype"] = "mxfp6/fp8 (QK^T on E3M2 + E8M0 per 32, the rest as mxfp8)"
        mres["unit"] = "TFLOP/s"
        mres["peak_note"] = "pct_of_peak against fp6 10.1 PFLOP/s; mixed_peak = n / sum(1/peak) over the counted GEMM units"
        out["mxfp6_e3m2"] = mres
    print(json.dumps(out))


if __name__ == "__main__":
    main()
