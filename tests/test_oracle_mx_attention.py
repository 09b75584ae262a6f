"""Pins for the MX attention oracle.

* Quantisation-transparent inputs (integers in [-8, 8]) are exact in E4M3 under the block
  rule, so every quantised copy equals the bf16 tensor and the MX oracle must reduce to the
  plain attention oracle (itself pinned against closed forms, finite differences and torch).
* Causality under MX: perturbing token j leaves O and dQ of every earlier query bit-identical.
* Isolation: a packed run equals each document run alone.
* The diagonal-tile rule: moving a token-blocked copy away from the bf16 values changes only
  off-diagonal contributions.
* The dS products take the bf16 Q and K: on inputs whose d-blocked copies are exact but whose
  token-blocked Q/K copies are not, dQ and dK still equal the plain oracle's.
"""

import numpy as np

from oracle import attention as att
from oracle import mx
from oracle import mx_attention as mxa


def _int_case(lengths, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    mk = lambda h: rng.integers(-8, 9, size=(T, h, d)).astype(np.float64)
    return mk(hq), mk(hkv), mk(hkv), mk(hq), cu


def test_integer_inputs_are_exact_in_e4m3():
    q, k, v, do, cu = _int_case([40, 200], 2, 1, 64, seed=0)
    for x in (q, k, v, do):
        xd, xt = mxa.operand_copies(x, cu)
        assert np.array_equal(xd, x) and np.array_equal(xt, x)


def test_transparent_inputs_reduce_to_plain_oracle():
    lengths = [130, 7, 300]
    q, k, v, do, cu = _int_case(lengths, 4, 2, 64, seed=1)
    sc = 2.0 ** -10 * 8
    o, lse = mxa.attn_mx_fwd(q, k, v, cu, sc)
    o0, lse0 = att.attn_fwd(q, k, v, cu, sc)
    np.testing.assert_allclose(o, o0, rtol=0, atol=1e-12 * np.abs(o0).max())
    np.testing.assert_array_equal(lse, lse0)
    g = mxa.attn_mx_bwd(q, k, v, do, cu, sc)
    g0 = att.attn_bwd(q, k, v, do, cu, sc)
    for a, b in zip(g, g0):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * np.abs(b).max())
    dlse = np.random.default_rng(5).standard_normal((4, sum(lengths)))
    g = mxa.attn_mx_bwd(q, k, v, do, cu, sc, dlse=dlse)
    g1 = att.attn_bwd(q, k, v, do, cu, sc, dlse=dlse)
    for a, b in zip(g, g1):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * np.abs(b).max())
    for b, c in zip(g1[:2], g0[:2]):                              # dQ, dK move; dV does not
        assert np.abs(b - c).max() > 1e-3 * np.abs(c).max()
    assert np.array_equal(g1[2], g0[2])


def test_causality_bit_exact_under_mx():
    rng = np.random.default_rng(2)
    lengths = [300, 150]
    T = sum(lengths)
    cu = np.array([0, 300, 450])
    # bf16-valued random inputs (values with 8 significant bits) so quantisation is not exact
    mk = lambda h: np.round(rng.standard_normal((T, h, 64)) * 128) / 128
    q, k, v, do = mk(2), mk(1), mk(1), mk(2)
    sc = 0.125
    o, _ = mxa.attn_mx_fwd(q, k, v, cu, sc)
    dq, _, _ = mxa.attn_mx_bwd(q, k, v, do, cu, sc)
    for j in (5, 31, 32, 100, 127, 128, 200, 299, 300 + 40):
        q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
        for a in (q2, k2, v2, do2):
            a[j] = a[j] * 7.5 + 30.0          # a large change: moves the token's block scales
        o2, _ = mxa.attn_mx_fwd(q2, k2, v2, cu, sc)
        dq2, _, _ = mxa.attn_mx_bwd(q2, k2, v2, do2, cu, sc)
        assert np.array_equal(o2[:j], o[:j]), j
        assert np.array_equal(dq2[:j], dq[:j]), j


def test_leak_without_safeguard():
    """Control: with the diagonal tile shrunk to one token the token-block scale leaks."""
    rng = np.random.default_rng(3)
    cu = np.array([0, 64])
    mk = lambda h: np.round(rng.standard_normal((64, h, 32)) * 128) / 128
    q, k, v = mk(1), mk(1), mk(1)
    o, _ = mxa.attn_mx_fwd(q, k, v, cu, 0.2, tile=1)
    v2 = v.copy()
    v2[40] *= 300.0                              # raise the block max of tokens 32..63
    o2, _ = mxa.attn_mx_fwd(q, k, v2, cu, 0.2, tile=1)
    assert not np.array_equal(o2[32:40], o[32:40])   # earlier queries changed: a leak
    o3, _ = mxa.attn_mx_fwd(q, k, v2, cu, 0.2)       # with the 128-token diagonal tile: none
    o1, _ = mxa.attn_mx_fwd(q, k, v, cu, 0.2)
    assert np.array_equal(o3[:40], o1[:40])


def test_isolation_bit_exact_under_mx():
    rng = np.random.default_rng(4)
    lengths = [33, 200, 1, 64]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = cu[-1]
    mk = lambda h: np.round(rng.standard_normal((T, h, 64)) * 64) / 64
    q, k, v, do = mk(2), mk(1), mk(1), mk(2)
    o, lse = mxa.attn_mx_fwd(q, k, v, cu, 0.1)
    g = mxa.attn_mx_bwd(q, k, v, do, cu, 0.1)
    for n in range(len(lengths)):
        s0, s1 = cu[n], cu[n + 1]
        one = np.array([0, s1 - s0])
        o1, l1 = mxa.attn_mx_fwd(q[s0:s1], k[s0:s1], v[s0:s1], one, 0.1)
        g1 = mxa.attn_mx_bwd(q[s0:s1], k[s0:s1], v[s0:s1], do[s0:s1], one, 0.1)
        assert np.array_equal(o1, o[s0:s1]) and np.array_equal(l1, lse[:, s0:s1])
        for a, b in zip(g1, g):
            assert np.array_equal(a, b[s0:s1])


def test_operand_selection_by_tile():
    """O splits into a bf16 diagonal part and a token-blocked off-diagonal part."""
    rng = np.random.default_rng(5)
    L = 300
    cu = np.array([0, L])
    mk = lambda h: np.round(rng.standard_normal((L, h, 32)) * 128) / 128
    q, k, v = mk(1), mk(1), mk(1)
    sc = 0.2
    o, _ = mxa.attn_mx_fwd(q, k, v, cu, sc)
    qd, _ = mxa.operand_copies(q, cu)
    kd, _ = mxa.operand_copies(k, cu)
    _, vt = mxa.operand_copies(v, cu)
    for i in (0, 127, 128, 200, 299):
        s = sc * kd[:i + 1, 0] @ qd[i, 0]
        p = np.exp(s - s.max()); p /= p.sum()
        ref = np.zeros(32)
        for j in range(i + 1):
            ref += p[j] * (v[j, 0] if (i // 128 == j // 128) else vt[j, 0])
        np.testing.assert_allclose(o[i, 0], ref, atol=1e-12)
    assert not np.array_equal(vt, v)
    np.testing.assert_array_equal(mx.padded_offsets(cu), [0, 320])


def test_mx_rows_match_full_mx_oracle():
    rng = np.random.default_rng(6)
    L = 300
    cu = np.array([0, L])
    mk = lambda h: np.round(rng.standard_normal((L, h, 32)) * 128) / 128
    q, k, v, do = mk(2), mk(1), mk(1), mk(2)
    o, lse = mxa.attn_mx_fwd(q, k, v, cu, 0.2)
    dq, dk, dv = mxa.attn_mx_bwd(q, k, v, do, cu, 0.2)
    rows = np.array([0, 31, 128, 129, 299])
    ro, rl, rdq, _, _ = mxa.attn_mx_rows(q, k, v, do, rows, 0.2)
    np.testing.assert_allclose(ro, o[rows], atol=1e-12)
    np.testing.assert_allclose(rl, lse[:, rows], atol=1e-12)
    np.testing.assert_allclose(rdq, dq[rows], atol=1e-12)
    _, _, _, pdk, pdv = mxa.attn_mx_rows(q, k, v, do, np.arange(200, L), 0.2)
    np.testing.assert_allclose(pdk[200:], dk[200:], atol=1e-12)
    np.testing.assert_allclose(pdv[200:], dv[200:], atol=1e-12)


def test_ds_products_take_bf16_q_and_k():
    """Q, K: each token row is c·2^(8·(i % 3)) with |c| in {1, 1.25, ..., 3.5} (3 mantissa bits,
    largest element <= 1.75·2^k), so every d-block (one token) is exact in E4M3, while a token
    block spans a 2^16 range and rounds its small tokens. V, dO take values in {0, ±1, ±2, ±4},
    exact under either blocking. Every MX copy the forward, dP and dV use is then exact, and the
    MX oracle must equal the plain oracle in all three gradients."""
    rng = np.random.default_rng(11)
    lengths = [300, 90]
    T = sum(lengths)
    cu = np.array([0, 300, 390])
    mags = np.array([1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5])
    loc = np.concatenate([np.arange(n) for n in lengths])

    def big_range(h):
        x = rng.choice(mags, size=(T, h, 64)) * rng.choice([-1.0, 1.0], size=(T, h, 64))
        return x * (2.0 ** (8 * (loc % 3)))[:, None, None]

    def pow2(h):
        return rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0], size=(T, h, 64))
    q, k, v, do = big_range(2), big_range(1), pow2(1), pow2(2)
    for x in (q, k):
        xd, xt = mxa.operand_copies(x, cu)
        assert np.array_equal(xd, x) and not np.array_equal(xt, x)
    for x in (v, do):
        xd, xt = mxa.operand_copies(x, cu)
        assert np.array_equal(xd, x) and np.array_equal(xt, x)
    sc = 2.0 ** -36                       # scores of the largest rows O(1), the rest near 0
    g = mxa.attn_mx_bwd(q, k, v, do, cu, sc)
    g0 = att.attn_bwd(q, k, v, do, cu, sc)
    for a, b in zip(g, g0):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(b).max())
    assert np.abs(g0[1]).max() > 0 and np.abs(g0[0]).max() > 0
    rows = np.array([0, 2, 130, 299])
    _, _, rdq, _, _ = mxa.attn_mx_rows(q[:300], k[:300], v[:300], do[:300], rows, sc)
    np.testing.assert_allclose(rdq, g0[0][rows], rtol=0, atol=1e-12 * np.abs(g0[0]).max())
