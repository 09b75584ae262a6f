"""Oracle regression fixtures and the seeded workload generator (CPU only)."""
import os
import sys

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

from oracle import attention, mx  # noqa: E402
from causal_flashattention_amd import workloads as W  # noqa: E402
import make_golden  # noqa: E402


def test_tiny_attention_fixture():
    _, cu, q, k, v, do, sc = make_golden.tiny_inputs()
    o, lse = attention.attn_fwd(q, k, v, cu, sc)
    g = attention.attn_bwd(q, k, v, do, cu, sc)
    got = {"o": o, "lse": lse, "dq": g[0], "dk": g[1], "dv": g[2]}
    with open(os.path.join(HERE, "golden", "tiny_attention.txt")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            name, *vals = line.split()
            np.testing.assert_allclose(got[name].ravel(), np.array(vals, dtype=np.float64), rtol=0, atol=1e-13)


def test_e4m3_table_fixture():
    with open(os.path.join(HERE, "golden", "e4m3_table.txt")) as f:
        rows = [l.split() for l in f if not l.startswith("#")]
    codes = np.array([int(r[0]) for r in rows])
    vals = np.array([float(r[1]) for r in rows])
    np.testing.assert_array_equal(mx.e4m3_decode(codes), vals)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f64(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


@pytest.mark.parametrize("k", [1, 2, 3])
def test_workload_shapes_and_determinism(k):
    w = W.make_workload(k)
    assert w.cu_seqlens[0] == 0 and w.cu_seqlens[-1] == w.total_tokens
    assert w.q.shape == (w.total_tokens, w.hq, w.d) and w.k.shape == (w.total_tokens, w.hkv, w.d)
    w2 = W.make_workload(k)
    assert np.array_equal(w.q, w2.q) and np.array_equal(w.cu_seqlens, w2.cu_seqlens)
    L = np.diff(w.cu_seqlens)
    if k == 2:
        assert np.all(L[:-1] >= 64) and np.all(L <= 2048)
    if k == 1:
        assert w.q.dtype == np.float32 and w.d == 64 and w.scale == 0.125


def test_flop_count():
    cu = np.array([0, 3, 3, 7])
    # pairs: 3*4/2 + 4*5/2 = 16
    assert W.causal_flops_fwd(cu, 2, 8) == 4 * 8 * 2 * 16
    assert W.causal_flops_fwd_bwd(cu, 2, 8) == 3.5 * 4 * 8 * 2 * 16
    w3_pairs = 32768 * 32769 / 2
    assert W.causal_flops_fwd(np.array([0, 32768]), 32, 128) == 4 * 128 * 32 * w3_pairs


def test_longest_last_moves_whole_documents():
    w = W.make_random(3, [5, 17, 2, 9, 17], hq=2, hkv=1, d=64)
    r = W.longest_last(w)
    L = list(np.diff(r.cu_seqlens))
    assert L == [2, 5, 9, 17, 17] and r.info["doc_order"] == "longest_last"
    cu = w.cu_seqlens
    for new, old in enumerate([2, 0, 3, 1, 4]):          # stable: the first 17 stays before the second
        a, b = r.cu_seqlens[new], r.cu_seqlens[new + 1]
        for name in ("q", "k", "v", "do"):
            assert np.array_equal(getattr(r, name)[a:b], getattr(w, name)[cu[old]:cu[old + 1]])
    assert r.flops_fwd_bwd() == w.flops_fwd_bwd()
    with pytest.raises(ValueError):
        W.reorder_documents(w, [0, 0, 1, 2, 3])
