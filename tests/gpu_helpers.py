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
