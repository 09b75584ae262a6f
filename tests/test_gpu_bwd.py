"""GPU parity of the backward pass against the float64 oracle (through the C ABI).

Tolerance: dQ, dK, dV rel-L2 <= 1e-2 each (bf16 inputs and outputs, fp32 accumulation).
Bit-identity (GPU against itself): rerun determinism, causality of dQ, document isolation.
At the 32K-token GQA shape the oracle computes sampled rows one by one (``attn_rows``), late
keys completely, and the gradient invariants that hold at any size.
"""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import attention as ref
from gpu_helpers import announce, head_group, key_block_threaded, rel_l2, to_f64, upload

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-2


def _fwd_bwd(w, dev):
    o, lse, _ = cfa.attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu"], scale=w.scale, causal=w.causal,
                             cu_seqlens_host=dev["cu_host"])
    dq, dk, dv = cfa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dev["cu"], scale=w.scale,
                              causal=w.causal, cu_seqlens_host=dev["cu_host"])
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("lengths,hq,hkv,d,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, 128, True),
    ([513, 31, 200], 8, 2, 128, True),
    ([700, 1], 4, 1, 128, True),
    ([77, 256, 1000], 4, 4, 64, True),
    ([33, 2, 190], 6, 3, 128, True),
    ([100, 257], 2, 1, 128, False),
    ([513, 31, 200], 8, 2, 64, True),          # d = 64 with the GQA head split
    ([700, 1], 4, 1, 64, True),                 # d = 64 MQA
    ([100, 257], 2, 1, 64, False),
])
def test_bf16_grads_random_documents(lengths, hq, hkv, d, causal):
    w = W.make_random(seed=7 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, d=d, causal=causal)
    announce("bwd bf16 random", lengths, hq, hkv, d, causal)
    dev = upload(w)
    _, _, dq, dk, dv = _fwd_bwd(w, dev)
    rdq, rdk, rdv = ref.attn_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal)
    for got, want in ((dq, rdq), (dk, rdk), (dv, rdv)):
        assert rel_l2(to_f64(got), want) <= GRAD_TOL


def test_bf16_grads_packed_workload_2():
    w = W.make_workload(2)
    announce("bwd bf16 workload 2", w.n_docs)
    dev = upload(w)
    _, _, dq, dk, dv = _fwd_bwd(w, dev)
    dq, dk, dv = to_f64(dq), to_f64(dk), to_f64(dv)
    for g in (0, 9):
        hs = head_group(w, g)
        rdq, rdk, rdv = ref.attn_bwd(w.f64("q")[:, hs], w.f64("k")[:, [g]], w.f64("v")[:, [g]],
                                     w.f64("do")[:, hs], w.cu_seqlens, w.scale)
        assert rel_l2(dq[:, hs], rdq) <= GRAD_TOL
        assert rel_l2(dk[:, [g]], rdk) <= GRAD_TOL
        assert rel_l2(dv[:, [g]], rdv) <= GRAD_TOL


def test_bf16_grads_gqa_workload_3_sampled():
    w = W.make_workload(3)
    announce("bwd bf16 workload 3")
    dev = upload(w)
    _, _, dq, dk, dv = _fwd_bwd(w, dev)
    dq, dk, dv = to_f64(dq), to_f64(dk), to_f64(dv)
    g = 2
    hs = head_group(w, g)
    q, k, v, do = w.f64("q")[:, hs], w.f64("k")[:, [g]], w.f64("v")[:, [g]], w.f64("do")[:, hs]
    L = w.total_tokens
    rows = np.array([0, 1, 63, 64, 127, 128, 5000, 16383, 16384, 30000, 32767])
    _, _, rdq, _, _ = ref.attn_rows(q, k, v, do, rows, w.scale)
    assert rel_l2(dq[rows][:, hs], rdq) <= GRAD_TOL
    tail = np.arange(L - 300, L)
    _, _, _, pdk, pdv = ref.attn_rows(q, k, v, do, tail, w.scale)
    assert rel_l2(dk[L - 300:, [g]], pdk[L - 300:]) <= GRAD_TOL
    assert rel_l2(dv[L - 300:, [g]], pdv[L - 300:]) <= GRAD_TOL
    # key tile 0 complete: the keys every one of the 32768 queries of the four heads sees, which
    # the dK/dV pass accumulates over its longest query loop
    bk, bv = key_block_threaded(q, k, v, do, 0, 128, w.scale)
    print("rel-L2 dK, dV of keys 0..127", rel_l2(dk[:128, [g]], bk), rel_l2(dv[:128, [g]], bv))
    assert rel_l2(dk[:128, [g]], bk) <= GRAD_TOL
    assert rel_l2(dv[:128, [g]], bv) <= GRAD_TOL
    # invariants at full size, every kv head: Σ_j dK_j = 0; Σ_j dV_j = Σ_{h in group} Σ_i dO_i;
    # Σ_h <Q, dQ> = <K, dK>  (tolerances relative to the magnitudes involved)
    do_all = w.f64("do")
    for gg in range(w.hkv):
        hh = head_group(w, gg)
        # bound: four times the spread of independent bf16 output roundings (2^-9 relative)
        s_dk = dk[:, gg].sum(axis=0)
        assert np.linalg.norm(s_dk) <= 4 * 2.0 ** -8 * np.sqrt(L * w.d * np.mean(dk[:, gg] ** 2))
        s_dv = dv[:, gg].sum(axis=0)
        want = do_all[:, hh].sum(axis=(0, 1))
        assert np.linalg.norm(s_dv - want) <= 4 * 2.0 ** -8 * np.sqrt(L * w.d * np.mean(dv[:, gg] ** 2)) + \
            1e-3 * np.linalg.norm(want)
        # the sums cancel almost completely, so the bound is the same rounding spread of the terms
        tq = w.f64("q")[:, hh] * dq[:, hh]
        tk = w.f64("k")[:, gg] * dk[:, gg]
        assert abs(tq.sum() - tk.sum()) <= 4 * 2.0 ** -8 * (np.sqrt(np.sum(tq ** 2)) + np.sqrt(np.sum(tk ** 2)))


@pytest.mark.parametrize("d", [128, 64])
def test_bf16_bwd_determinism_isolation_causality(d):
    lengths = [300, 129, 1, 64, 700]
    w = W.make_random(seed=21, lengths=lengths, hq=4, hkv=2, d=d)
    announce("bwd bf16 invariants", lengths, d)
    dev = upload(w)
    r1 = _fwd_bwd(w, dev)
    r2 = _fwd_bwd(w, dev)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    cu = w.cu_seqlens
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=d, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1],
                         do=w.do[s0:s1])
        ra = _fwd_bwd(sub, upload(sub))
        for a, b in zip(ra[2:], r1[2:]):
            assert torch.equal(a, b[s0:s1])
    for jl in (0, 63, 64, 200, 699):
        j = int(cu[4]) + jl
        dev2 = {kk: vv.clone() for kk, vv in dev.items()}
        for name in ("q", "k", "v", "do"):
            dev2[name][j] = dev2[name][j] * 3 + 1
        r3 = _fwd_bwd(w, dev2)
        assert torch.equal(r3[2][:j], r1[2][:j])      # dQ of every earlier token
        assert torch.equal(r3[0][:j], r1[0][:j])      # and O


def test_gradient_sums_small_random():
    """Invariants of the gradient, checked on the GPU output itself."""
    lengths = [500, 37]
    w = W.make_random(seed=33, lengths=lengths, hq=4, hkv=1)
    announce("bwd bf16 gradient sums")
    dev = upload(w)
    _, _, dq, dk, dv = _fwd_bwd(w, dev)
    dk, dv = to_f64(dk), to_f64(dv)
    do = w.f64("do")
    for n in range(2):
        s0, s1 = w.cu_seqlens[n], w.cu_seqlens[n + 1]
        spread_k = 4 * 2.0 ** -8 * np.linalg.norm(dk[s0:s1, 0])   # rounding spread of the bf16 outputs
        spread_v = 4 * 2.0 ** -8 * np.linalg.norm(dv[s0:s1, 0])
        assert np.linalg.norm(dk[s0:s1, 0].sum(axis=0)) <= spread_k
        want = do[s0:s1].sum(axis=(0, 1))
        assert np.linalg.norm(dv[s0:s1, 0].sum(axis=0) - want) <= spread_v + 1e-3 * np.linalg.norm(want)
