"""attn_bwd_noalloc (scratch in the library's fixed per-GPU array) against attn_bwd (caller
workspace): the same kernels, so the gradients must be bit-identical. Two calls in a row, the
second on a smaller input, so the array's leftovers from the first call cannot leak into the
second."""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W

from gpu_helpers import announce, to_dev, DEV

pytestmark = pytest.mark.gpu

CASES = [  # (lengths, hq, hkv, mx): bf16 with the GQA head split, then smaller inputs
    ([900, 1, 2100, 64], 8, 2, False),
    ([300, 129, 5], 4, 4, False),
    ([700, 33], 4, 2, "mxfp8"),
    ([130, 2], 2, 2, "mxfp8"),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("pair", [(0, 1), (2, 3)])
def test_noalloc_backward_equals_workspace_backward(pair):
    for i in pair:
        lengths, hq, hkv, mx = CASES[i]
        announce("attn_bwd_noalloc", lengths, hq, hkv, mx)
        w = W.make_random(seed=300 + i, lengths=lengths, hq=hq, hkv=hkv)
        q, k, v, do = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.do)
        cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(DEV)
        o, lse, saved = cfa.attn_fwd(q, k, v, cu, scale=w.scale, mx=mx)
        want = cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=w.scale, mx=mx, saved=saved)
        got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        cfa.attn_bwd_noalloc(q, k, v, o, lse, do, cu, dq=got[0], dk=got[1], dv=got[2], scale=w.scale, mx=mx,
                             saved=saved)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(_bits(a), _bits(b)), (lengths, mx)
