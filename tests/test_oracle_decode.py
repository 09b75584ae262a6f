"""Pins for the decoding oracle (one query per sequence over a packed KV cache), on the CPU.

* Reduction to the pinned attention oracle: the decode of a sequence equals the last row of a
  causal document whose last query is the decoding query (that row sees every key).
* Closed forms: q = 0 gives the mean of V and lse = ln L; one key gives o = V_0, lse = s_0;
  an empty sequence gives o = 0, lse = -inf; constant V rows pass through.
* The cache values are the exact MX decode: hand-computed elements.
"""
import math

import numpy as np

from causal_flashattention_amd import workloads as W
from oracle import attention as att
from oracle import decode as dec


def _vals(w):
    if w.kv == "mxfp8":
        return dec.dequantize_cache(w.k, w.k_scales), dec.dequantize_cache(w.v, w.v_scales)
    return W.bf16_bits_to_f64(w.k), W.bf16_bits_to_f64(w.v)


def test_equals_last_row_of_causal_attention():
    for kv in ("bf16", "mxfp8"):
        w = W.make_decode(seed=3, lengths=[1, 7, 40, 129], hq=4, hkv=2, d=64, kv=kv)
        k, v = _vals(w)
        q = W.bf16_bits_to_f64(w.q)
        o, lse = dec.decode_attention(q, k, v, w.cu_seqlens_k, w.scale)
        rng = np.random.default_rng(0)
        for b in range(w.n_seqs):
            s0, s1 = int(w.cu_seqlens_k[b]), int(w.cu_seqlens_k[b + 1])
            L = s1 - s0
            qq = rng.standard_normal((L, 4, 64))     # earlier queries: any values
            qq[-1] = q[b]
            oo, ll = att.attn_fwd(qq, k[s0:s1], v[s0:s1], np.array([0, L]), w.scale, causal=True)
            np.testing.assert_allclose(o[b], oo[-1], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[:, b], ll[:, -1], rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(4)
    cu = np.array([0, 0, 1, 6])                  # empty, one key, five keys
    k = rng.standard_normal((6, 1, 8))
    v = rng.standard_normal((6, 1, 8))
    q = rng.standard_normal((3, 2, 8))
    q[2, 0] = 0.0
    o, lse = dec.decode_attention(q, k, v, cu, 0.5)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[:, 0]))
    for h in range(2):
        np.testing.assert_array_equal(o[1, h], v[0, 0])
        assert lse[h, 1] == 0.5 * float(k[0, 0] @ q[1, h])
    np.testing.assert_allclose(o[2, 0], v[1:6, 0].mean(axis=0), rtol=1e-14, atol=1e-15)
    assert abs(lse[0, 2] - math.log(5)) < 1e-14
    vc = np.repeat(v[:1], 6, axis=0)             # constant V rows
    o2, _ = dec.decode_attention(q, k, vc, cu, 0.5)
    np.testing.assert_allclose(o2[2], np.broadcast_to(v[0, 0], (2, 8)), rtol=1e-14)


def test_cache_values_are_exact_mx_decode():
    codes = np.zeros((1, 1, 32), np.uint8)
    codes[0, 0, :4] = [0x38, 0xB9, 0x01, 0x7E]   # 1.0, -1.125, 2^-9 (smallest subnormal), 448
    scales = np.array([[[130]]], np.uint8)       # 2^3
    x = dec.dequantize_cache(codes, scales)
    np.testing.assert_array_equal(x[0, 0, :4], [8.0, -9.0, 2.0 ** -6, 3584.0])
    assert np.all(x[0, 0, 4:] == 0)
