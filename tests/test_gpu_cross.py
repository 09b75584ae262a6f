"""GPU parity of cross-attention (separate packed query and key documents, bf16), through the C ABI.

Oracle: ``oracle.attention.attn_cross`` (pinned on the CPU against self-attention, decoding,
torch SDPA with the explicit mask and central differences). Tolerances as for self-attention:
O max-abs <= 1e-2, LSE <= 1e-3 (rows that see no key: O = 0 and LSE = -inf exactly), gradients
rel-L2 <= 1e-2. Bit-identity: with identical query and key documents the cross-attention calls
equal attn_fwd / attn_bwd; reruns; each document alone against the packed batch.
"""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import attention as ref
from gpu_helpers import DEV, announce, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _case(lq, lk, hq, hkv, d, seed):
    """Seeded bf16 inputs: q, dO [Tq, hq, d]; k, v [Tk, hkv, d]."""
    rng = np.random.default_rng(seed)
    Tq, Tk = sum(lq), sum(lk)
    bf = lambda shape: W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    return dict(q=bf((Tq, hq, d)), k=bf((Tk, hkv, d)), v=bf((Tk, hkv, d)), do=bf((Tq, hq, d)),
                cq=W.cu_from_lengths(lq), ck=W.cu_from_lengths(lk))


def _run(c, causal, scale):
    dev = {n: to_dev(c[n]) for n in ("q", "k", "v", "do")}
    cq, ck = torch.from_numpy(c["cq"]).to(DEV), torch.from_numpy(c["ck"]).to(DEV)
    o, lse = cfa.attn_fwd_cross(dev["q"], dev["k"], dev["v"], cq, ck, scale=scale, causal=causal,
                                cu_seqlens_q_host=c["cq"], cu_seqlens_k_host=c["ck"])
    dq, dk, dv = cfa.attn_bwd_cross(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], cq, ck, scale=scale,
                                    causal=causal, cu_seqlens_q_host=c["cq"], cu_seqlens_k_host=c["ck"])
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


CASES = [
    ([5, 20, 1, 300], [12, 9, 40, 128], 4, 2, 128, True),     # Lq < Lk, Lq > Lk (rows with no key)
    ([64, 0, 129], [64, 33, 0], 2, 1, 128, True),               # an empty query and an empty key document
    ([200, 31], [700, 31], 8, 2, 128, False),
    ([77, 130], [300, 64], 4, 4, 64, True),
    ([40, 257], [100, 128], 4, 2, 256, True),
    ([513], [1024], 16, 1, 128, True),                           # MQA (head split)
]


@pytest.mark.parametrize("lq,lk,hq,hkv,d,causal", CASES)
def test_cross_attention(lq, lk, hq, hkv, d, causal):
    c = _case(lq, lk, hq, hkv, d, seed=1000 + sum(lq) + d)
    scale = 1.0 / np.sqrt(d)
    announce("cross", lq, lk, hq, hkv, d, causal)
    o, lse, dq, dk, dv = _run(c, causal, scale)
    f = W.bf16_bits_to_f64
    ro, rl, rdq, rdk, rdv = ref.attn_cross(f(c["q"]), f(c["k"]), f(c["v"]), f(c["do"]), c["cq"], c["ck"], scale,
                                           causal)
    o, lse = to_f64(o), lse.detach().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o - ro)) <= 1e-2
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin) and np.all(np.isneginf(lse[~fin]))
    assert np.max(np.abs(lse[fin] - rl[fin]), initial=0.0) <= 1e-3
    errs = [rel_l2(to_f64(a), b) for a, b in zip((dq, dk, dv), (rdq, rdk, rdv)) if np.any(b)]
    print("rel-L2", errs)
    assert max(errs) <= 1e-2
    unseen_rows = ~fin.any(axis=0)
    assert np.all(to_f64(dq)[unseen_rows] == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_equal_documents_match_self_attention_bit_exact(d):
    lengths = [300, 1, 129, 64]
    c = _case(lengths, lengths, 4, 2, d, seed=1100 + d)
    scale = 1.0 / np.sqrt(d)
    announce("cross == self", d)
    r = _run(c, True, scale)
    dev = {n: to_dev(c[n]) for n in ("q", "k", "v", "do")}
    cu = torch.from_numpy(c["cq"]).to(DEV)
    o, lse, _ = cfa.attn_fwd(dev["q"], dev["k"], dev["v"], cu, scale=scale, cu_seqlens_host=c["cq"])
    g = cfa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], cu, scale=scale, cu_seqlens_host=c["cq"])
    torch.cuda.synchronize()
    for a, b in zip(r, (o, lse) + tuple(g)):
        assert torch.equal(a, b)


def test_cross_isolation_and_determinism():
    lq, lk = [5, 300, 0, 77], [40, 200, 9, 77]
    c = _case(lq, lk, 4, 2, 128, seed=1200)
    scale = 0.088
    announce("cross invariants")
    r1 = _run(c, True, scale)
    r2 = _run(c, True, scale)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    for n in range(len(lq)):
        q0, q1, k0, k1 = c["cq"][n], c["cq"][n + 1], c["ck"][n], c["ck"][n + 1]
        sub = dict(q=c["q"][q0:q1], k=c["k"][k0:k1], v=c["v"][k0:k1], do=c["do"][q0:q1],
                   cq=np.array([0, q1 - q0], np.int32), ck=np.array([0, k1 - k0], np.int32))
        ra = _run(sub, True, scale)
        assert torch.equal(ra[0], r1[0][q0:q1]) and torch.equal(ra[1], r1[1][:, q0:q1])
        assert torch.equal(ra[2], r1[2][q0:q1])
        assert torch.equal(ra[3], r1[3][k0:k1]) and torch.equal(ra[4], r1[4][k0:k1])
