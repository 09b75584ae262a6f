"""Helpers for the GPU parity tests: upload seeded workloads, download outputs as float64."""
import sys

import numpy as np
import torch

from causal_flashattention_amd import workloads as W

DEV = "cuda:0"


def announce(*parts):
    """Name the case on stdout before touching the GPU (a fault then still names it)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def to_dev(a):
    """numpy uint16 bf16 bits / float32 -> torch tensor on the GPU with the same bits."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV)


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(w):
    d = {name: to_dev(getattr(w, name)) for name in ("q", "k", "v")}
    if w.do is not None:
        d["do"] = to_dev(w.do)
    d["cu"] = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(DEV)
    d["cu_host"] = torch.from_numpy(w.cu_seqlens.astype(np.int32))
    return d


def rel_l2(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def head_group(w, g):
    """Query heads of kv head g."""
    G = w.hq // w.hkv
    return list(range(g * G, (g + 1) * G))


def key_block_threaded(q, k, v, do, k0, k1, scale, n_ranges=8, workers=16):
    """Oracle dK, dV of keys k0..k1-1 of one document (doc-local float64 arrays, one kv head)
    summed over every query: ``oracle.attention.attn_key_block`` per query head and per query
    range (ranges of equal causal work), run on a thread pool (NumPy releases the GIL in its
    array operations) and added up."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    from oracle import attention as ref
    L, hq = q.shape[0], q.shape[1]
    b = [0] + [int(L * np.sqrt(i / n_ranges)) for i in range(1, n_ranges)] + [L]
    tasks = [(h, (b[i], b[i + 1])) for h in range(hq) for i in range(n_ranges) if b[i + 1] > b[i]]
    with threadpool_limits(1), cf.ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda t: ref.attn_key_block(q[:, [t[0]]], k, v, do[:, [t[0]]], k0, k1, scale,
                                                         row_block=64, q_range=t[1]), tasks))
    return sum(p[0] for p in parts), sum(p[1] for p in parts)


def mx_rows_threaded(q, k, v, do, scale, workers=16):
    """``oracle.mx_attention.attn_mx_rows`` over every row of one document, one call per head
    (hq = hkv here) on a thread pool: o, lse, dq, dk, dv with heads stacked in order."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    from oracle import mx_attention as mxa
    L, H = q.shape[0], q.shape[1]
    rows = np.arange(L)
    with threadpool_limits(1), cf.ThreadPoolExecutor(min(workers, H)) as ex:
        parts = list(ex.map(lambda h: mxa.attn_mx_rows(q[:, [h]], k[:, [h]], v[:, [h]], do[:, [h]], rows, scale),
                            range(H)))
    o = np.concatenate([p[0] for p in parts], axis=1)
    lse = np.concatenate([p[1] for p in parts], axis=0)
    dq, dk, dv = (np.concatenate([p[i] for p in parts], axis=1) for i in (2, 3, 4))
    return o, lse, dq, dk, dv
