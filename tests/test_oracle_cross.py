"""Pins for the cross-attention oracle (separate query and key documents), on the CPU.

* With identical query and key documents it is the self-attention oracle (bit for bit on the
  outputs that both compute the same way, to rounding otherwise).
* A one-query document is decoding: equal to the decoding oracle.
* torch's float64 CPU scaled_dot_product_attention with the explicit boolean mask (a library
  routine), for Lq < Lk and Lq > Lk (rows that see no key are compared separately: O = 0).
* Central differences of the forward for the gradient, with rows that see no key present.
"""
import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import decode as dec


def _case(lq, lk, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = rng.standard_normal((cq[-1], hq, d))
    k = rng.standard_normal((ck[-1], hkv, d))
    v = rng.standard_normal((ck[-1], hkv, d))
    do = rng.standard_normal((cq[-1], hq, d))
    return q, k, v, do, cq, ck


@pytest.mark.parametrize("causal", [True, False])
def test_equal_documents_reduce_to_self_attention(causal):
    L = [7, 1, 40]
    q, k, v, do, cq, ck = _case(L, L, 4, 2, 8, seed=1)
    o, lse, dq, dk, dv = att.attn_cross(q, k, v, do, cq, ck, 0.3, causal)
    o0, l0 = att.attn_fwd(q, k, v, cq, 0.3, causal)
    g0 = att.attn_bwd(q, k, v, do, cq, 0.3, causal)
    np.testing.assert_allclose(o, o0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, l0, rtol=1e-13, atol=1e-14)
    for a, b in zip((dq, dk, dv), g0):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_one_query_is_decoding():
    q, k, v, _, cq, ck = _case([1, 1, 1], [5, 0, 33], 4, 2, 8, seed=2)
    o, lse, *_ = att.attn_cross(q, k, v, None, cq, ck, 0.4, True)
    od, ld = dec.decode_attention(q, k, v, ck, 0.4)
    np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ld))
    fin = np.isfinite(ld)
    np.testing.assert_allclose(lse[fin], ld[fin], rtol=1e-13)


@pytest.mark.parametrize("lq,lk,causal", [([5, 20], [12, 9], True), ([5, 20], [12, 9], False), ([3], [3], True)])
def test_against_torch_sdpa_with_mask(lq, lk, causal):
    q, k, v, _, cq, ck = _case(lq, lk, 2, 1, 8, seed=3)
    o, lse, *_ = att.attn_cross(q, k, v, None, cq, ck, 0.35, causal)
    for n in range(len(lq)):
        Lq, Lk = lq[n], lk[n]
        allowed = ~np.isinf(att.cross_mask(Lq, Lk, causal))        # [Lq, Lk]
        seen = allowed.any(axis=1)
        tq = torch.from_numpy(q[cq[n]:cq[n + 1]]).permute(1, 0, 2)
        tk = torch.from_numpy(k[ck[n]:ck[n + 1]]).permute(1, 0, 2).expand(2, Lk, 8)
        tv = torch.from_numpy(v[ck[n]:ck[n + 1]]).permute(1, 0, 2).expand(2, Lk, 8)
        ref = torch.nn.functional.scaled_dot_product_attention(tq[:, seen], tk, tv,
                                                               attn_mask=torch.from_numpy(allowed[seen]), scale=0.35)
        np.testing.assert_allclose(o[cq[n]:cq[n + 1]][seen], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)
        assert np.all(o[cq[n]:cq[n + 1]][~seen] == 0) and np.all(np.isneginf(lse[:, cq[n]:cq[n + 1]][:, ~seen]))


def test_finite_differences_cross():
    q, k, v, do, cq, ck = _case([6, 2], [3, 4], 2, 1, 3, seed=4)    # doc 0: rows 0..2 see no key
    dlse = np.random.default_rng(5).standard_normal((2, 8))
    _, lse0, dq, dk, dv = att.attn_cross(q, k, v, do, cq, ck, 0.7, True, dlse=dlse)
    assert np.isneginf(lse0[0, 0]) and np.all(dq[:3] == 0)
    fin = np.isfinite(lse0)

    def loss(a):
        o, lse, *_ = att.attn_cross(a["q"], a["k"], a["v"], None, cq, ck, 0.7, True)
        return float(np.sum(o * do) + np.sum(np.where(fin, lse, 0.0) * dlse))

    base = {"q": q, "k": k, "v": v}
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        arr = base[name]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += 1e-6
            a2[idx] -= 1e-6
            num[idx] = (loss({**base, name: a1}) - loss({**base, name: a2})) / 2e-6
        assert np.linalg.norm(num - grad) <= 1e-6 * max(np.linalg.norm(grad), 1e-30), name
