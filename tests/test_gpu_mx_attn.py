"""GPU parity of the MXFP8 path against the MX oracle (the same quantisation, float64 arithmetic).

Tolerances: O, dQ, dK, dV rel-L2 <= 3e-2 against ``oracle.mx_attention``; LSE max-abs <= 1e-3
(the scores come from the identical E4M3 operands). Not modelled by the oracle, hence inside
the tolerance: the E4M3 encoding of P (fixed scale 2^-8) and of dS (MX scale along the
contraction) before the matrix-core products, and fp32 accumulation.
Bit-identity on the GPU: causality (perturbing token j leaves O and dQ of earlier tokens
unchanged, so no shared scale leaks a later token), document isolation, rerun determinism.
"""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import mx_attention as mxa
from gpu_helpers import announce, head_group, mx_rows_threaded, rel_l2, to_f64, upload

pytestmark = pytest.mark.gpu

MX_TOL = 3e-2
LSE_TOL = 1e-3


def _fwd(w, dev):
    o, lse, saved = cfa.attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu"], scale=w.scale, causal=w.causal,
                                 cu_seqlens_host=dev["cu_host"], mx=True)
    torch.cuda.synchronize()
    return o, lse, saved


@pytest.mark.parametrize("lengths,hq,hkv,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, True),
    ([513, 31, 200, 33], 4, 2, True),
    ([700, 1], 4, 1, True),
    ([100, 257], 2, 1, False),
])
def test_mx_forward_random_documents(lengths, hq, hkv, causal):
    w = W.make_random(seed=100 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, causal=causal)
    announce("mx fwd random", lengths, hq, hkv, causal)
    dev = upload(w)
    o, lse, _ = _fwd(w, dev)
    ro, rl = mxa.attn_mx_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale, causal)
    assert rel_l2(to_f64(o), ro) <= MX_TOL
    assert np.max(np.abs(to_f64(lse) - rl)) <= LSE_TOL


def test_mx_forward_workload_4_one_head():
    w = W.make_workload(4, with_grad=False)
    announce("mx fwd workload 4", w.n_docs)
    dev = upload(w)
    o, lse, _ = _fwd(w, dev)
    o, lse = to_f64(o), to_f64(lse)
    hh = 7
    ro, rl = mxa.attn_mx_fwd(w.f64("q")[:, [hh]], w.f64("k")[:, [hh]], w.f64("v")[:, [hh]], w.cu_seqlens, w.scale)
    assert rel_l2(o[:, [hh]], ro) <= MX_TOL
    assert np.max(np.abs(lse[[hh]] - rl)) <= LSE_TOL


def test_mx_forward_causality_isolation_determinism():
    lengths = [300, 129, 1, 64, 700]
    w = W.make_random(seed=44, lengths=lengths, hq=4, hkv=2)
    announce("mx fwd invariants", lengths)
    dev = upload(w)
    o1, l1, _ = _fwd(w, dev)
    o2, l2, _ = _fwd(w, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cu = w.cu_seqlens
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=128, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1])
        oa, la, _ = _fwd(sub, upload(sub))
        assert torch.equal(oa, o1[s0:s1]) and torch.equal(la, l1[:, s0:s1])
    for jl in (0, 31, 32, 100, 127, 128, 200, 699):
        j = int(cu[4]) + jl
        dev2 = {kk: vv.clone() for kk, vv in dev.items()}
        for name in ("q", "k", "v"):
            dev2[name][j] = dev2[name][j] * 7.5 + 30.0     # large: moves the token's block scales
        o3, l3, _ = _fwd(w, dev2)
        assert torch.equal(o3[:j], o1[:j]) and torch.equal(l3[:, :j], l1[:, :j]), jl


def _fwd_bwd(w, dev):
    o, lse, saved = _fwd(w, dev)
    dq, dk, dv = cfa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dev["cu"], scale=w.scale,
                              causal=w.causal, cu_seqlens_host=dev["cu_host"], mx=True, saved=saved)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("lengths,hq,hkv,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, True),
    ([513, 31, 200, 33], 4, 2, True),
    ([700, 1], 4, 1, True),
    ([100, 257], 2, 1, False),
])
def test_mx_backward_random_documents(lengths, hq, hkv, causal):
    w = W.make_random(seed=200 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, causal=causal)
    announce("mx bwd random", lengths, hq, hkv, causal)
    dev = upload(w)
    _, _, dq, dk, dv = _fwd_bwd(w, dev)
    ref = mxa.attn_mx_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal)
    errs = [rel_l2(to_f64(a), b) for a, b in zip((dq, dk, dv), ref)]
    print("rel-L2 dq dk dv", errs)
    assert max(errs) <= MX_TOL


def test_mx_backward_workload_4_sampled():
    """The longest document of the 65536-token packed workload, two heads, complete: dQ of every
    query and dK, dV of every key against the MX oracle (row by row, one thread per head)."""
    w = W.make_workload(4)
    announce("mx bwd workload 4", w.n_docs)
    dev = upload(w)
    _, _, dq, dk, dv = _fwd_bwd(w, dev)
    L_all = np.diff(w.cu_seqlens)
    n = int(np.argmax(L_all))
    s0, L = int(w.cu_seqlens[n]), int(L_all[n])
    heads = [3, 17]
    sl = slice(s0, s0 + L)
    q, k, v, do = (W.bf16_bits_to_f64(getattr(w, x)[sl][:, heads]) for x in ("q", "k", "v", "do"))
    _, _, rdq, rdk, rdv = mx_rows_threaded(q, k, v, do, w.scale)
    e_dq = rel_l2(to_f64(dq[sl][:, heads]), rdq)
    e_dk = rel_l2(to_f64(dk[sl][:, heads]), rdk)
    e_dv = rel_l2(to_f64(dv[sl][:, heads]), rdv)
    e_dk0 = rel_l2(to_f64(dk[sl][:128, heads]), rdk[:128])       # key tile 0: every query of the document
    e_dv0 = rel_l2(to_f64(dv[sl][:128, heads]), rdv[:128])
    print("rel-L2 dq dk dv (document of", L, "tokens, 2 heads)", e_dq, e_dk, e_dv, "key tile 0", e_dk0, e_dv0)
    assert max(e_dq, e_dk, e_dv, e_dk0, e_dv0) <= MX_TOL


def test_mx_backward_causality_isolation_determinism():
    lengths = [300, 129, 1, 64, 700]
    w = W.make_random(seed=45, lengths=lengths, hq=4, hkv=2)
    announce("mx bwd invariants", lengths)
    dev = upload(w)
    r1 = _fwd_bwd(w, dev)
    r2 = _fwd_bwd(w, dev)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    cu = w.cu_seqlens
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=128, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1],
                         do=w.do[s0:s1])
        ra = _fwd_bwd(sub, upload(sub))
        for a, b in zip(ra[2:], r1[2:]):
            assert torch.equal(a, b[s0:s1])
    for jl in (0, 31, 32, 100, 127, 128, 200, 699):
        j = int(cu[4]) + jl
        dev2 = {kk: vv.clone() for kk, vv in dev.items()}
        for name in ("q", "k", "v", "do"):
            dev2[name][j] = dev2[name][j] * 7.5 + 30.0
        r3 = _fwd_bwd(w, dev2)
        assert torch.equal(r3[0][:j], r1[0][:j]), jl
        assert torch.equal(r3[2][:j], r1[2][:j]), jl
