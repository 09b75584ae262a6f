"""Pins for the float64 attention oracle (forward and gradient), all on the CPU.

Each pin comes from something other than the oracle itself: closed forms of the softmax
definition, finite differences, exact invariants of the gradient, a library routine
(torch's float64 CPU scaled_dot_product_attention and autograd), and brute-force loops.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att

RNG = np.random.default_rng(1234)


def _rand_case(lengths, hq, hkv, d, seed=0):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    do = rng.standard_normal((T, hq, d))
    return q, k, v, do, cu


# ---------------------------------------------------------------- closed forms (forward)

@pytest.mark.parametrize("which", ["q", "k"])
def test_zero_scores_give_prefix_mean(which):
    lengths = [7, 1, 40, 3]
    q, k, v, _, cu = _rand_case(lengths, 4, 2, 16, seed=1)
    if which == "q":
        q[:] = 0
    else:
        k[:] = 0
    o, lse = att.attn_fwd(q, k, v, cu, scale=0.3)
    for n in range(len(lengths)):
        s0, s1 = cu[n], cu[n + 1]
        for h in range(4):
            g = h // 2
            pref = np.cumsum(v[s0:s1, g], axis=0) / np.arange(1, s1 - s0 + 1)[:, None]
            np.testing.assert_allclose(o[s0:s1, h], pref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[h, s0:s1], np.log(np.arange(1, s1 - s0 + 1)), rtol=0, atol=1e-12)


def test_single_token_documents():
    lengths = [1, 1, 1]
    q, k, v, _, cu = _rand_case(lengths, 2, 1, 8, seed=2)
    o, lse = att.attn_fwd(q, k, v, cu, scale=0.5)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])
    np.testing.assert_array_equal(o[:, 1], v[:, 0])
    np.testing.assert_allclose(lse[0], 0.5 * np.sum(q[:, 0] * k[:, 0], axis=1), atol=1e-12)


def test_constant_values_pass_through():
    lengths = [9, 30]
    q, k, v, _, cu = _rand_case(lengths, 2, 2, 8, seed=3)
    c = np.linspace(-1, 1, 8)
    v[:] = c
    o, _ = att.attn_fwd(q, k, v, cu, scale=1.0)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-12)


def test_brute_force_loops_small():
    """Scalar triple loop over the definition, without matrices or masks."""
    lengths = [4, 6]
    q, k, v, _, cu = _rand_case(lengths, 2, 1, 3, seed=4)
    sc = 0.7
    o, lse = att.attn_fwd(q, k, v, cu, scale=sc)
    for n in range(2):
        s0 = cu[n]
        for h in range(2):
            for i in range(lengths[n]):
                sc_row = [sc * sum(q[s0 + i, h, r] * k[s0 + j, 0, r] for r in range(3)) for j in range(i + 1)]
                mx = max(sc_row)
                w = [math.exp(s - mx) for s in sc_row]
                tot = sum(w)
                for r in range(3):
                    ref = sum(w[j] * v[s0 + j, 0, r] for j in range(i + 1)) / tot
                    assert abs(o[s0 + i, h, r] - ref) < 1e-12
                assert abs(lse[h, s0 + i] - (mx + math.log(tot))) < 1e-12


# ---------------------------------------------------------------- library cross-check

def _torch_sdpa_per_doc(q, k, v, cu, scale, causal):
    hq, hkv = q.shape[1], k.shape[1]
    outs = []
    for n in range(len(cu) - 1):
        s0, s1 = cu[n], cu[n + 1]
        tq = torch.from_numpy(q[s0:s1]).permute(1, 0, 2)
        tk = torch.from_numpy(k[s0:s1]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        tv = torch.from_numpy(v[s0:s1]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        outs.append((tq, tk, tv))
    return outs


@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_sdpa_and_autograd(causal):
    lengths = [5, 33, 1, 70]
    hq, hkv, d = 4, 2, 16
    q, k, v, do, cu = _rand_case(lengths, hq, hkv, d, seed=5)
    sc = 1.0 / math.sqrt(d)
    o, lse = att.attn_fwd(q, k, v, cu, sc, causal=causal)
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, sc, causal=causal)
    for n in range(len(lengths)):
        s0, s1 = cu[n], cu[n + 1]
        tq = torch.from_numpy(q[s0:s1].copy()).permute(1, 0, 2).requires_grad_(True)
        tk = torch.from_numpy(k[s0:s1].copy()).permute(1, 0, 2).requires_grad_(True)
        tv = torch.from_numpy(v[s0:s1].copy()).permute(1, 0, 2).requires_grad_(True)
        ke = tk.repeat_interleave(hq // hkv, dim=0)
        ve = tv.repeat_interleave(hq // hkv, dim=0)
        to = torch.nn.functional.scaled_dot_product_attention(
            tq.unsqueeze(0), ke.unsqueeze(0), ve.unsqueeze(0), is_causal=causal, scale=sc)[0]
        np.testing.assert_allclose(o[s0:s1], to.permute(1, 0, 2).detach().numpy(), atol=1e-12)
        tdo = torch.from_numpy(do[s0:s1].copy()).permute(1, 0, 2)
        (to * tdo).sum().backward()
        np.testing.assert_allclose(dq[s0:s1], tq.grad.permute(1, 0, 2).numpy(), atol=1e-12)
        np.testing.assert_allclose(dk[s0:s1], tk.grad.permute(1, 0, 2).numpy(), atol=1e-12)
        np.testing.assert_allclose(dv[s0:s1], tv.grad.permute(1, 0, 2).numpy(), atol=1e-12)
        # LSE from the library's own softmax input
        s = torch.einsum("hid,hjd->hij", tq.detach(), ke.detach()) * sc
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(s1 - s0, s1 - s0, dtype=torch.bool), 1), float("-inf"))
        np.testing.assert_allclose(lse[:, s0:s1], torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


def test_online_softmax_matches_two_pass():
    """Fused-kernel claim: a blockwise running-max/running-sum pass gives the same result."""
    lengths = [300]
    q, k, v, _, cu = _rand_case(lengths, 1, 1, 32, seed=6)
    sc = 0.2
    o, lse = att.attn_fwd(q, k, v, cu, sc)
    L = 300
    acc = np.zeros((L, 32))
    m = np.full(L, -np.inf)
    l = np.zeros(L)
    for j0 in range(0, L, 64):  # key blocks
        j1 = min(L, j0 + 64)
        s = sc * q[:, 0] @ k[j0:j1, 0].T
        s[np.arange(j0, j1)[None, :] > np.arange(L)[:, None]] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.where(np.isfinite(m_new), np.exp(m - m_new), 0.0)
        p = np.exp(s - m_new[:, None])
        l = l * alpha + p.sum(axis=1)
        acc = acc * alpha[:, None] + p @ v[j0:j1, 0]
        m = m_new
    np.testing.assert_allclose(o[:, 0], acc / l[:, None], atol=1e-12)
    np.testing.assert_allclose(lse[0], m + np.log(l), atol=1e-12)


# ---------------------------------------------------------------- gradient pins

def test_finite_differences():
    lengths = [1, 3, 5]
    hq, hkv, d = 2, 1, 4
    q, k, v, do, cu = _rand_case(lengths, hq, hkv, d, seed=7)
    sc = 0.6
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, sc)
    eps = 1e-6

    def loss(q_, k_, v_):
        o, _ = att.attn_fwd(q_, k_, v_, cu, sc)
        return float(np.sum(o * do))

    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a1 = arr.copy(); a1[idx] += eps
            a2 = arr.copy(); a2[idx] -= eps
            args1 = {"q": q, "k": k, "v": v}; args1[name] = a1
            args2 = {"q": q, "k": k, "v": v}; args2[name] = a2
            num[idx] = (loss(args1["q"], args1["k"], args1["v"]) - loss(args2["q"], args2["k"], args2["v"])) / (2 * eps)
        rel = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        assert rel < 1e-6, (name, rel)


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences_with_lse_gradient(causal):
    """Loss Σ O·dO + Σ LSE·dLSE: the oracle backward with ``dlse`` against central differences."""
    lengths = [2, 4, 3]
    hq, hkv, d = 2, 1, 3
    q, k, v, do, cu = _rand_case(lengths, hq, hkv, d, seed=11)
    dlse = np.random.default_rng(12).standard_normal((hq, sum(lengths)))
    sc = 0.7
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, sc, causal=causal, dlse=dlse)
    eps = 1e-6

    def loss(args):
        o, lse = att.attn_fwd(args["q"], args["k"], args["v"], cu, sc, causal=causal)
        return float(np.sum(o * do) + np.sum(lse * dlse))

    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1 = arr.copy(); a1[idx] += eps
            a2 = arr.copy(); a2[idx] -= eps
            base = {"q": q, "k": k, "v": v}
            num[idx] = (loss({**base, name: a1}) - loss({**base, name: a2})) / (2 * eps)
        rel = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        assert rel < 1e-6, (name, rel)


def test_lse_gradient_closed_form_single_tokens():
    """One-token documents: LSE = scale·q·k, so dQ = scale·dLSE·k, dK = scale·Σ_h dLSE·q, dV = 0."""
    lengths = [1, 1, 1, 1]
    q, k, v, _, cu = _rand_case(lengths, 2, 1, 5, seed=13)
    do = np.zeros_like(q)
    dlse = np.random.default_rng(14).standard_normal((2, 4))
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, 0.3, dlse=dlse)
    np.testing.assert_allclose(dq, 0.3 * dlse.T[:, :, None] * k, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dk[:, 0], 0.3 * np.einsum("th,thd->td", dlse.T, q), rtol=1e-13, atol=1e-15)
    assert not np.any(dv)


def test_gradient_closed_forms_q_zero():
    lengths = [6, 11]
    q, k, v, do, cu = _rand_case(lengths, 2, 2, 8, seed=8)
    q[:] = 0
    sc = 0.9
    o, _ = att.attn_fwd(q, k, v, cu, sc)
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, sc)
    assert np.all(dk == 0)
    for n in range(2):
        s0, s1 = cu[n], cu[n + 1]
        L = s1 - s0
        for h in range(2):
            for j in range(L):
                ref = sum(do[s0 + i, h] / (i + 1) for i in range(j, L))
                np.testing.assert_allclose(dv[s0 + j, h], ref, atol=1e-12)
            for i in range(L):
                ref = sc / (i + 1) * sum(np.dot(do[s0 + i, h], v[s0 + j, h] - o[s0 + i, h]) * k[s0 + j, h]
                                         for j in range(i + 1))
                np.testing.assert_allclose(dq[s0 + i, h], ref, atol=1e-12)


def test_gradient_closed_forms_k_zero_and_single_token():
    q, k, v, do, cu = _rand_case([5, 9], 2, 1, 8, seed=9)
    k[:] = 0
    dq, _, _ = att.attn_bwd(q, k, v, do, cu, 0.4)
    assert np.all(dq == 0)
    q, k, v, do, cu = _rand_case([1, 1, 1, 1], 2, 2, 8, seed=10)
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, 0.4)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)
    np.testing.assert_allclose(dv, do, atol=1e-12)


def test_gradient_invariants():
    lengths = [17, 64, 3]
    hq, hkv, d = 4, 2, 8
    q, k, v, do, cu = _rand_case(lengths, hq, hkv, d, seed=11)
    sc = 0.35
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, sc)
    for n in range(len(lengths)):
        s0, s1 = cu[n], cu[n + 1]
        for g in range(hkv):
            hs = [h for h in range(hq) if h // (hq // hkv) == g]
            # adding the same vector to every key of a document leaves the softmax unchanged
            np.testing.assert_allclose(dk[s0:s1, g].sum(axis=0), 0, atol=1e-10 * np.abs(dk).max())
            # adding a vector c to every value adds c to every output
            np.testing.assert_allclose(dv[s0:s1, g].sum(axis=0), sum(do[s0:s1, h].sum(axis=0) for h in hs),
                                       atol=1e-10 * np.abs(dv).max())
            # scores are bilinear in (Q, K): scaling Q by t and K by 1/t changes nothing
            lhs = sum(np.sum(q[s0:s1, h] * dq[s0:s1, h]) for h in hs)
            rhs = np.sum(k[s0:s1, g] * dk[s0:s1, g])
            assert abs(lhs - rhs) <= 1e-10 * (np.abs(q).max() * np.abs(dq).max() * (s1 - s0) * d * len(hs))


# ---------------------------------------------------------------- isolation and causality

def test_isolation_bit_exact():
    lengths = [13, 1, 700, 40]
    q, k, v, do, cu = _rand_case(lengths, 2, 1, 16, seed=12)
    o, lse = att.attn_fwd(q, k, v, cu, 0.25)
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, 0.25)
    for n in range(len(lengths)):
        s0, s1 = cu[n], cu[n + 1]
        one = np.array([0, s1 - s0])
        o1, l1 = att.attn_fwd(q[s0:s1], k[s0:s1], v[s0:s1], one, 0.25)
        g1 = att.attn_bwd(q[s0:s1], k[s0:s1], v[s0:s1], do[s0:s1], one, 0.25)
        assert np.array_equal(o1, o[s0:s1]) and np.array_equal(l1, lse[:, s0:s1])
        for a, b in zip(g1, (dq, dk, dv)):
            assert np.array_equal(a, b[s0:s1])


def test_causality_bit_exact():
    lengths = [50, 90]
    q, k, v, do, cu = _rand_case(lengths, 2, 2, 8, seed=13)
    o, _ = att.attn_fwd(q, k, v, cu, 0.3)
    dq, _, _ = att.attn_bwd(q, k, v, do, cu, 0.3)
    for j_local in (0, 17, 89):
        j = cu[1] + j_local
        q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
        for a in (q2, k2, v2, do2):
            a[j] += 3.0
        o2, _ = att.attn_fwd(q2, k2, v2, cu, 0.3)
        dq2, _, _ = att.attn_bwd(q2, k2, v2, do2, cu, 0.3)
        assert np.array_equal(o2[:j], o[:j])
        assert np.array_equal(dq2[:j], dq[:j])
        assert not np.array_equal(o2[j:cu[2]], o[j:cu[2]])


def test_mask_is_explicit_upper_triangle():
    m = att.causal_mask(4, 2, 7, True)
    for i in range(4):
        for j in range(7):
            assert m[i, j] == (-np.inf if j > i + 2 else 0.0)
    assert np.all(att.causal_mask(3, 0, 5, False) == 0)


def test_row_subset_matches_full_oracle():
    lengths = [150]
    q, k, v, do, cu = _rand_case(lengths, 4, 2, 8, seed=14)
    o, lse = att.attn_fwd(q, k, v, cu, 0.3)
    dq, dk, dv = att.attn_bwd(q, k, v, do, cu, 0.3)
    rows = np.array([0, 7, 64, 149])
    ro, rl, rdq, _, _ = att.attn_rows(q, k, v, do, rows, 0.3)
    np.testing.assert_allclose(ro, o[rows], atol=1e-12)
    np.testing.assert_allclose(rl, lse[:, rows], atol=1e-12)
    np.testing.assert_allclose(rdq, dq[rows], atol=1e-12)
    # rows 100.. cover every query that sees keys 100..149
    _, _, _, pdk, pdv = att.attn_rows(q, k, v, do, np.arange(100, 150), 0.3)
    np.testing.assert_allclose(pdk[100:], dk[100:], atol=1e-12)
    np.testing.assert_allclose(pdv[100:], dv[100:], atol=1e-12)
    _, _, _, fdk, fdv = att.attn_rows(q, k, v, do, np.arange(150), 0.3, causal=True)
    np.testing.assert_allclose(fdk, dk, atol=1e-12)


def test_key_block_gradients_equal_full_oracle():
    """attn_key_block (every query, a block of keys) against the full backward, causal and not,
    GQA, blocks at the start, in the middle, crossing row blocks and at the end."""
    rng = np.random.default_rng(77)
    L, hq, hkv, d = 700, 4, 2, 16
    q, k, v, do = (rng.standard_normal((L, h, d)) for h in (hq, hkv, hkv, hq))
    cu = np.array([0, L])
    for causal in (True, False):
        _, dk, dv = att.attn_bwd(q, k, v, do, cu, 0.3, causal)
        for k0, k1 in ((0, 128), (100, 101), (250, 520), (600, 700), (0, 700)):
            bk, bv = att.attn_key_block(q, k, v, do, k0, k1, 0.3, causal, row_block=96)
            np.testing.assert_allclose(bk, dk[k0:k1], rtol=0, atol=1e-12 * np.abs(dk).max())
            np.testing.assert_allclose(bv, dv[k0:k1], rtol=0, atol=1e-12 * np.abs(dv).max())


def test_key_block_query_ranges_add_up():
    rng = np.random.default_rng(78)
    L, d = 300, 8
    q, k, v, do = (rng.standard_normal((L, 2, d)) for _ in range(4))
    k, v = k[:, :1], v[:, :1]
    whole = att.attn_key_block(q, k, v, do, 40, 170, 0.5)
    parts = [att.attn_key_block(q, k, v, do, 40, 170, 0.5, q_range=r) for r in ((0, 90), (90, 91), (91, 300))]
    for i in range(2):
        np.testing.assert_allclose(sum(p[i] for p in parts), whole[i], rtol=0, atol=1e-12 * np.abs(whole[i]).max())
