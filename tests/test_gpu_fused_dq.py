"""The bf16 backward at d = 128 with dQ summed inside the dK/dV pass, in key-tile order
(CFA_DQ_MODE=fused; the default runs dQ as a separate pass).

Checked against the float64 oracle beside the default mode, for bit-identical reruns, for
document isolation, and for a clear wait flag (no bounded wait gave up)."""
import os

import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import attention as ref

from gpu_helpers import DEV, announce, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu


class env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update(self.kv)

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _run(w, causal=True, fused=True):
    with env(CFA_DQ_MODE="fused" if fused else "separate"):
        return _run_now(w, causal)


def _run_now(w, causal):
    q, k, v, do = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.do)
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(DEV)
    o, lse, _ = cfa.attn_fwd(q, k, v, cu, scale=w.scale, causal=causal)
    ws = torch.empty(cfa.workspace_bytes(1, w.total_tokens, w.n_docs, w.hq, w.hkv, w.d, cfa.CFA_BF16),
                     dtype=torch.uint8, device=DEV)
    g = cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=w.scale, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    return [t.clone() for t in g], cfa.device_error(ws)


CASES = [
    ([1, 5, 64, 127, 129, 300, 1000], 4, 2, True),
    ([2100, 33, 700], 8, 8, True),
    ([700, 1, 260], 4, 1, True),          # MQA: the head split (4 workgroups per key tile)
    ([100, 257, 640], 2, 1, False),       # not causal: every key tile adds into every block
]


@pytest.mark.parametrize("lengths,hq,hkv,causal", CASES)
def test_fused_dq_matches_oracle_and_separate_mode(lengths, hq, hkv, causal):
    w = W.make_random(seed=500 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, causal=causal)
    announce("fused dQ", lengths, hq, hkv, causal)
    fused, flag = _run(w, causal)
    assert flag == 0
    sep, _ = _run(w, causal, fused=False)
    want = ref.attn_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal)
    errs = [(rel_l2(to_f64(a), r), rel_l2(to_f64(b), r)) for a, b, r in zip(fused, sep, want)]
    print("rel-L2 dq dk dv (fused, separate)", errs)
    assert all(ea <= 1e-2 and eb <= 1e-2 for ea, eb in errs)
    again, _ = _run(w, causal)
    for a, b in zip(fused, again):
        assert torch.equal(a, b)


def test_fused_dq_isolation_and_causality():
    lengths = [300, 129, 1, 64, 700]
    w = W.make_random(seed=521, lengths=lengths, hq=4, hkv=2)
    announce("fused dQ invariants", lengths)
    r1, _ = _run(w)
    cu = w.cu_seqlens
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=128, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1],
                         do=w.do[s0:s1])
        ra, _ = _run(sub)
        for a, b in zip(ra, r1):
            assert torch.equal(a, b[s0:s1])
