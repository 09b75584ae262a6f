"""Decoding oracle: one new query token per sequence over a packed, quantised KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Flash Attention" (ai.ozdemir.be), sections "Tanım" and "Gerçek dünyadan örnek": local
inference engines keep the K/V cache in a quantised type (an 8-bit type at about half the
memory of f16, a 4-bit one at about a quarter) and need flash attention to read a quantised V
cache. The page names the cache types by their memory ratio only. The reading here: the cache
holds, per token and kv head, the E4M3 codes and E8M0 block scales of the MX quantiser along
the head dim (blocks of 32 channels of one token: ``oracle.mx.quantize_d``), 8.25 bits per
element, or plain bf16. A cached element's value is its exact decode, code × 2^(scale − 127).

For sequence ``b`` with cached keys ``K[cu_k[b]:cu_k[b+1]]`` (the current token's included)
and query head ``h`` (kv head ``h // (hq // hkv)``), the one query ``q[b, h]`` sees every
cached key -- the last row of a causal document ("GPT Kernel Programlama" §4: the last token
sees all earlier ones and itself):

    s_j = scale·q·K̂_j,   p = softmax(s),   o = Σ_j p_j·V̂_j,   lse = log Σ_j exp(s_j)

computed in float64 with the two-pass (max, then sum) softmax of §5. A sequence with no cached
token gives ``o = 0`` and ``lse = -inf`` (an empty sum).
"""

import numpy as np

from . import mx as _mx


def dequantize_cache(codes, scales):
    """Exact values of an MX cache: codes [T, h, d] (E4M3 bytes), scales [T, h, d/32] (E8M0)."""
    return _mx.dequantize_d(codes, scales)


def decode_attention(q, k, v, cu_seqlens_k, scale):
    """q [B, hq, d]; k, v [Tk, hkv, d] (values, e.g. from ``dequantize_cache``); returns
    o [B, hq, d] and lse [hq, B] in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    cu = np.asarray(cu_seqlens_k, np.int64)
    B, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0 and len(cu) == B + 1 and cu[0] == 0 and cu[-1] == k.shape[0]
    group = hq // hkv
    o = np.zeros((B, hq, d))
    lse = np.full((hq, B), -np.inf)
    for b in range(B):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        for h in range(hq):
            g = h // group
            s = scale * (k[s0:s1, g] @ q[b, h])
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            o[b, h] = (e / l) @ v[s0:s1, g]
            lse[h, b] = m + np.log(l)
    return o, lse
