"""More than 1024 packed documents (the work-list builder then runs several chunks of its
1024-thread scans), bf16 and MXFP8, forward and backward, every row checked on the GPU.

2600 documents of 0-48 tokens with a few of 300-1300 among them (several length buckets, ties,
empty documents), 4 query / 2 kv heads (bf16) and one head (MXFP8, whose oracle is slower), d = 128. The oracle runs
over the whole packed batch (documents are independent). A schedule bug (a wrong item prefix,
a document placed twice or not at all) leaves tiles uncomputed or computed twice, which these
full comparisons see; the index-order schedule must give bit-identical results.
Tolerances as in the other parity tests: bf16 O within 1e-2·max(1, |O|) (short documents leave
|O| near single V entries, up to ~4, where bf16 itself rounds by up to 0.008), LSE 1e-3, gradients
1e-2 rel-L2; MXFP8 3e-2 rel-L2 on O and the gradients."""
import os

import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import attention as ref
from oracle import mx_attention as mxa
from gpu_helpers import announce, rel_l2, to_f64, upload

pytestmark = pytest.mark.gpu


def _lengths(seed=21, n=2600):
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = [int(x) for x in rng.integers(0, 49, size=n)]
    for i, L in zip(rng.choice(n, size=6, replace=False), (300, 300, 512, 700, 1000, 1300)):
        lengths[int(i)] = L
    return lengths


def _run(w, dev, mx):
    o, lse, saved = cfa.attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu"], scale=w.scale,
                                 cu_seqlens_host=dev["cu_host"], mx=mx)
    g = cfa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dev["cu"], scale=w.scale,
                     cu_seqlens_host=dev["cu_host"], mx=mx, saved=saved)
    torch.cuda.synchronize()
    return [o, lse, *g]


@pytest.mark.parametrize("mx", [False, "mxfp8"])
def test_many_documents(mx):
    lengths = _lengths()
    assert len(lengths) > 1024 and 0 in lengths
    hq, hkv = (1, 1) if mx else (4, 2)
    w = W.make_random(seed=22, lengths=lengths, hq=hq, hkv=hkv)
    announce("many documents", mx or "bf16", len(lengths), w.total_tokens)
    dev = upload(w)
    a = _run(w, dev, mx)
    o, lse, dq, dk, dv = (to_f64(t) for t in a)
    q, k, v, do = (w.f64(n) for n in ("q", "k", "v", "do"))
    if mx:
        ro, rl = mxa.attn_mx_fwd(q, k, v, w.cu_seqlens, w.scale)
        rdq, rdk, rdv = mxa.attn_mx_bwd(q, k, v, do, w.cu_seqlens, w.scale)[:3]
        assert rel_l2(o, ro) <= 3e-2
        tol = 3e-2
    else:
        ro, rl = ref.attn_fwd(q, k, v, w.cu_seqlens, w.scale)
        rdq, rdk, rdv = ref.attn_bwd(q, k, v, do, w.cu_seqlens, w.scale)[:3]
        assert np.max(np.abs(o - ro) / np.maximum(1.0, np.abs(ro))) <= 1e-2
        tol = 1e-2
    assert np.max(np.abs(lse - rl)) <= 1e-3
    assert rel_l2(dq, rdq) <= tol
    assert rel_l2(dk, rdk) <= tol
    assert rel_l2(dv, rdv) <= tol
    # the index-order schedule computes every tile the same way
    old = os.environ.get("CFA_SCHED")
    os.environ["CFA_SCHED"] = "naive"
    try:
        b = _run(w, dev, mx)
    finally:
        if old is None:
            del os.environ["CFA_SCHED"]
        else:
            os.environ["CFA_SCHED"] = old
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
