"""Pins for the operand copy each MX backward product takes (``attn_mx_bwd`` and ``attn_mx_rows``).

FLAMIA page, "FLAMIA Mimarisi ve Temel Tasarım İlkeleri": quantised operands are reused across
orientations by token-block scaling, and targeted safeguards keep a shared scale from carrying
data across the causal boundary. The oracle's reading: dP = dO·Vᵀ contracts over the head dim
and takes the d-blocked copies ``dO_d``, ``V_d``; dV = Pᵀ·dO contracts over tokens and takes the
token-blocked ``dO_t`` on off-diagonal 128×128 tiles and the bf16 ``dO_b`` on diagonal tiles.

Each pin feeds inputs that are exact under one blocking and inexact under the other, so a
wrong copy moves the result by far more than rounding:

* dO exact in d-blocks (one token per block, 3 significant bits) but not in token blocks
  (token rows scaled by 2^0, 2^8, 2^16 in turn): dV must carry the token-blocked rounding on
  off-diagonal pairs only, and dQ, dK must not move.
* V exact in token blocks (one channel per block) but not in d-blocks (channels scaled by
  2^0, 2^8, 2^16 in turn): dQ, dK must carry the d-blocked rounding of V through dP, and dV
  must not move.
* Anti-causality of the key gradients: dK_j and dV_j depend on the queries and output
  gradients of tokens i >= j only (P_ij = 0 for i < j), so perturbing Q and dO of token i
  must leave dK and dV of every later key bit-identical. A token block that mixed dO of an
  earlier query into a diagonal pair would break this.

The expected values are built pair by pair from ``oracle.mx`` copies and the plain oracle's
probabilities, a separate formulation from the oracle's masked matrix products.
"""

import numpy as np

from oracle import attention as att
from oracle import mx
from oracle import mx_attention as mxa

MAGS = np.array([1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5])   # 3 significant bits
LENGTHS = [300, 90]
D = 64
SC = 2.0 ** -8


def _cu():
    return np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int64)


def _loc():
    return np.concatenate([np.arange(n) for n in LENGTHS])


def _ints(rng, h):
    """Integers in [-8, 8]: exact in E4M3 under either blocking."""
    return rng.integers(-8, 9, size=(sum(LENGTHS), h, D)).astype(np.float64)


def _pow2(rng, h):
    return rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0], size=(sum(LENGTHS), h, D))


def _token_scaled(rng, h):
    """Row i is c·2^(8·(i % 3)): exact per d-block, inexact per token block."""
    x = rng.choice(MAGS, size=(sum(LENGTHS), h, D)) * rng.choice([-1.0, 1.0], size=(sum(LENGTHS), h, D))
    return x * (2.0 ** (8 * (_loc() % 3)))[:, None, None]


def _channel_scaled(rng, h):
    """Channel c is m·2^(8·(c % 3)): exact per token block, inexact per d-block."""
    x = rng.choice(MAGS, size=(sum(LENGTHS), h, D)) * rng.choice([-1.0, 1.0], size=(sum(LENGTHS), h, D))
    return x * (2.0 ** (8 * (np.arange(D) % 3)))[None, None, :]


def _probs(q, k, s0, L, h, g):
    """Plain softmax probabilities of one document and head (Q, K exact in E4M3 here)."""
    p, _ = att._probabilities(q[s0:s0 + L, h], k[s0:s0 + L, g], SC, 0, True)
    return p


def _expected_grads(q, k, v, do, cu, v_dp, do_dp, do_off):
    """dQ, dK, dV pair by pair: dP from the copies v_dp / do_dp, dV from do_off on off-diagonal
    pairs and from the bf16 dO on diagonal pairs (tile 128); O and D from the plain oracle
    (its V copies are exact in every case used here)."""
    o, _ = att.attn_fwd(q, k, v, cu, SC)
    T, hq, _ = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for n in range(len(cu) - 1):
        s0, L = int(cu[n]), int(cu[n + 1] - cu[n])
        for h in range(hq):
            g = h // G
            p = _probs(q, k, s0, L, h, g)
            for i in range(L):
                Di = do[s0 + i, h] @ o[s0 + i, h]
                for j in range(i + 1):
                    pij = p[i, j]
                    dsij = pij * (do_dp[s0 + i, h] @ v_dp[s0 + j, g] - Di)
                    dq[s0 + i, h] += SC * dsij * k[s0 + j, g]
                    dk[s0 + j, g] += SC * dsij * q[s0 + i, h]
                    diag = (i // 128) == (j // 128)
                    dv[s0 + j, g] += pij * (do[s0 + i, h] if diag else do_off[s0 + i, h])
    return dq, dk, dv


def _close(a, b, tol=1e-11):
    np.testing.assert_allclose(a, b, rtol=0, atol=tol * max(1.0, np.abs(b).max()))


def _far(a, b):
    """Differs by far more than the 1e-11 match tolerance (a wrong copy moves the small-magnitude
    tokens only, about 1e-7 of the largest entry)."""
    return np.abs(a - b).max() > 1e-8 * np.abs(b).max()


def test_dv_takes_token_blocked_do_off_diagonal_and_bf16_do_on_diagonal():
    rng = np.random.default_rng(21)
    cu = _cu()
    q, k, v, do = _ints(rng, 2), _ints(rng, 1), _pow2(rng, 1), _token_scaled(rng, 2)
    do_d, do_t = mxa.operand_copies(do, cu)
    assert np.array_equal(do_d, do) and not np.array_equal(do_t, do)
    for x in (q, k, v):
        xd, xt = mxa.operand_copies(x, cu)
        assert np.array_equal(xd, x) and np.array_equal(xt, x)
    edq, edk, edv = _expected_grads(q, k, v, do, cu, v_dp=v, do_dp=do, do_off=do_t)
    dq, dk, dv = mxa.attn_mx_bwd(q, k, v, do, cu, SC)
    pq, pk, pv = att.attn_bwd(q, k, v, do, cu, SC)
    _close(dv, edv)
    _close(dq, edq)
    _close(dk, edk)
    np.testing.assert_allclose(dq, pq, rtol=0, atol=1e-11 * np.abs(pq).max())   # dP and D exact
    np.testing.assert_allclose(dk, pk, rtol=0, atol=1e-11 * np.abs(pk).max())
    # the copy matters: dO_d (= dO) everywhere, or dO_t everywhere, give other dV
    assert _far(dv, pv)
    alt = np.zeros_like(dv)
    for n in range(len(cu) - 1):
        s0, L = int(cu[n]), int(cu[n + 1] - cu[n])
        for h in range(2):
            p = _probs(q, k, s0, L, h, 0)
            alt[s0:s0 + L, 0] += p.T @ do_t[s0:s0 + L, h]
    assert _far(dv, alt)
    # the row sampler of long documents follows the same rule (first document alone)
    L = LENGTHS[0]
    one = np.array([0, L])
    rows = np.arange(L)
    _, _, rdq, rdk, rdv = mxa.attn_mx_rows(q[:L], k[:L], v[:L], do[:L], rows, SC)
    fdq, fdk, fdv = mxa.attn_mx_bwd(q[:L], k[:L], v[:L], do[:L], one, SC)
    _close(rdv, fdv)
    _close(rdq, fdq)
    _close(rdk, fdk)
    edq1, edk1, edv1 = _expected_grads(q[:L], k[:L], v[:L], do[:L], one, v_dp=v[:L], do_dp=do[:L],
                                       do_off=mxa.operand_copies(do[:L], one)[1])
    _close(rdv, edv1)


def test_dp_takes_d_blocked_v_and_do():
    rng = np.random.default_rng(22)
    cu = _cu()
    q, k, v, do = _ints(rng, 2), _ints(rng, 1), _channel_scaled(rng, 1), _pow2(rng, 2)
    v_d, v_t = mxa.operand_copies(v, cu)
    assert np.array_equal(v_t, v) and not np.array_equal(v_d, v)
    for x in (q, k, do):
        xd, xt = mxa.operand_copies(x, cu)
        assert np.array_equal(xd, x) and np.array_equal(xt, x)
    edq, edk, edv = _expected_grads(q, k, v, do, cu, v_dp=v_d, do_dp=do, do_off=do)
    dq, dk, dv = mxa.attn_mx_bwd(q, k, v, do, cu, SC)
    pq, pk, pv = att.attn_bwd(q, k, v, do, cu, SC)
    _close(dq, edq)
    _close(dk, edk)
    _close(dv, edv)
    np.testing.assert_allclose(dv, pv, rtol=0, atol=1e-11 * np.abs(pv).max())    # P and dO exact
    assert _far(dq, pq) and _far(dk, pk)          # bf16 V in dP would give the plain gradients
    # attn_mx_rows on the first document: the same dP operands
    L = LENGTHS[0]
    one = np.array([0, L])
    rows = np.array([0, 5, 127, 128, 200, 299])
    _, _, rdq, _, _ = mxa.attn_mx_rows(q[:L], k[:L], v[:L], do[:L], rows, SC)
    edq1, _, _ = _expected_grads(q[:L], k[:L], v[:L], do[:L], one, v_dp=mxa.operand_copies(v[:L], one)[0],
                                 do_dp=do[:L], do_off=do[:L])
    _close(rdq, edq1[rows])
    _, _, _, rdk, rdv = mxa.attn_mx_rows(q[:L], k[:L], v[:L], do[:L], np.arange(L), SC)
    fdq, fdk, fdv = mxa.attn_mx_bwd(q[:L], k[:L], v[:L], do[:L], one, SC)
    _close(rdk, fdk)
    _close(rdv, fdv)


def test_key_gradients_ignore_earlier_queries_under_mx():
    """Perturb Q and dO of token i: dK and dV of every key j > i of the document stay
    bit-identical (P_ij = 0 for i < j). dO of i shares its token block with later queries,
    which the diagonal rule keeps out of every pair it could reach."""
    rng = np.random.default_rng(23)
    cu = np.array([0, 300, 450])
    T = 450
    mk = lambda h: np.round(rng.standard_normal((T, h, 32)) * 128) / 128
    q, k, v, do = mk(2), mk(1), mk(1), mk(2)
    sc = 0.125
    _, dk, dv = mxa.attn_mx_bwd(q, k, v, do, cu, sc)
    _, _, _, rdk, rdv = mxa.attn_mx_rows(q[:300], k[:300], v[:300], do[:300], np.arange(300), sc)
    for i in (0, 31, 32, 100, 127, 128, 200, 298, 300 + 40):
        q2, do2 = q.copy(), do.copy()
        q2[i] = q2[i] * 7.5 + 30.0
        do2[i] = do2[i] * -5.0 + 11.0            # moves the token's d-block and token-block scales
        _, dk2, dv2 = mxa.attn_mx_bwd(q2, k, v, do2, cu, sc)
        end = 300 if i < 300 else 450
        assert np.array_equal(dk2[i + 1:end], dk[i + 1:end]), i
        assert np.array_equal(dv2[i + 1:end], dv[i + 1:end]), i
        assert not np.array_equal(dv2[:i + 1], dv[:i + 1]), i      # the perturbation is seen
        if i < 300:
            _, _, _, rdk2, rdv2 = mxa.attn_mx_rows(q2[:300], k[:300], v[:300], do2[:300], np.arange(300), sc)
            assert np.array_equal(rdk2[i + 1:], rdk[i + 1:]), i
            assert np.array_equal(rdv2[i + 1:], rdv[i + 1:]), i


def test_token_blocked_do_everywhere_would_leak_into_later_keys():
    """Control for the pin above: the same perturbation, with every pair's dV taking the
    token-blocked dO (no diagonal rule), moves dV of later keys in the token's 32-block."""
    rng = np.random.default_rng(24)
    L = 160
    cu = np.array([0, L])
    mk = lambda h: np.round(rng.standard_normal((L, h, 32)) * 128) / 128
    q, k, do = mk(1), mk(1), mk(1)

    def dv_all_token_blocked(do_):
        p = _probs_sc(q, k, L, 0.2)
        return p.T @ mxa.operand_copies(do_, cu)[1][:, 0]

    def _probs_sc(q_, k_, L_, sc):
        p, _ = att._probabilities(q_[:, 0], k_[:, 0], sc, 0, True)
        return p
    i = 40
    do2 = do.copy()
    do2[i] = do2[i] * -5.0 + 11.0
    a, b = dv_all_token_blocked(do), dv_all_token_blocked(do2)
    assert not np.array_equal(a[i + 1:64], b[i + 1:64])      # keys 41..63 share the block: a leak
    assert mx.padded_offsets(cu)[1] == 160
