"""GPU parity of the MXFP6/FP8 paths (E2M3 or E3M2 score product, the rest MXFP8) against the MX
oracle with ``qk="e2m3"`` / ``qk="e3m2"``, through the C ABI; every test runs for both formats.

Tolerances as for MXFP8: O (and dQ, dK, dV) rel-L2 <= 3e-2; LSE max-abs <= 1e-3 (the scores come
from identical 6-bit operands and scales on both sides). Bit-identity on the GPU: causality,
document isolation and reruns.
"""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import mx_attention as mxa
from gpu_helpers import announce, rel_l2, to_f64, upload

pytestmark = pytest.mark.gpu

MX_TOL = 3e-2
LSE_TOL = 1e-3
PATH = {"e2m3": "mxfp6", "e3m2": "mxfp6_e3m2"}


@pytest.fixture(params=["e2m3", "e3m2"])
def fmt(request):
    return request.param


def _fwd(w, dev, fmt):
    o, lse, saved = cfa.attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu"], scale=w.scale, causal=w.causal,
                                 cu_seqlens_host=dev["cu_host"], mx=PATH[fmt])
    torch.cuda.synchronize()
    return o, lse, saved


@pytest.mark.parametrize("lengths,hq,hkv,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, True),
    ([513, 31, 200, 33], 4, 2, True),
    ([700, 1], 4, 1, True),
    ([100, 257], 2, 1, False),
])
def test_fp6_forward_random_documents(lengths, hq, hkv, causal, fmt):
    w = W.make_random(seed=1800 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, causal=causal)
    announce(PATH[fmt] + " fwd random", lengths, hq, hkv, causal)
    o, lse, _ = _fwd(w, upload(w), fmt)
    ro, rl = mxa.attn_mx_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale, causal, qk=fmt)
    r8, _ = mxa.attn_mx_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale, causal)
    err = rel_l2(to_f64(o), ro)
    print("rel-L2 o", err, "fp6 vs fp8 oracle", rel_l2(ro, r8))
    assert err <= MX_TOL
    assert np.max(np.abs(to_f64(lse) - rl)) <= LSE_TOL


def test_fp6_forward_causality_isolation_determinism(fmt):
    lengths = [300, 129, 1, 64, 700]
    w = W.make_random(seed=1844, lengths=lengths, hq=4, hkv=2)
    announce(PATH[fmt] + " fwd invariants", lengths)
    dev = upload(w)
    o1, l1, _ = _fwd(w, dev, fmt)
    o2, l2, _ = _fwd(w, dev, fmt)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cu = w.cu_seqlens
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=128, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1])
        oa, la, _ = _fwd(sub, upload(sub), fmt)
        assert torch.equal(oa, o1[s0:s1]) and torch.equal(la, l1[:, s0:s1])
    for jl in (0, 31, 32, 100, 127, 128, 200, 699):
        j = int(cu[4]) + jl
        dev2 = {kk: vv.clone() for kk, vv in dev.items()}
        for name in ("q", "k", "v"):
            dev2[name][j] = dev2[name][j] * 7.5 + 30.0
        o3, l3, _ = _fwd(w, dev2, fmt)
        assert torch.equal(o3[:j], o1[:j]) and torch.equal(l3[:, :j], l1[:, :j]), jl


def test_fp6_forward_workload_4_one_head(fmt):
    w = W.make_workload(4, with_grad=False)
    announce(PATH[fmt] + " fwd workload 4", w.n_docs)
    o, lse, _ = _fwd(w, upload(w), fmt)
    o, lse = to_f64(o), to_f64(lse)
    hh = 5
    ro, rl = mxa.attn_mx_fwd(w.f64("q")[:, [hh]], w.f64("k")[:, [hh]], w.f64("v")[:, [hh]], w.cu_seqlens, w.scale,
                             qk=fmt)
    assert rel_l2(o[:, [hh]], ro) <= MX_TOL
    assert np.max(np.abs(lse[[hh]] - rl)) <= LSE_TOL


def _fwd_bwd(w, dev, fmt):
    o, lse, saved = _fwd(w, dev, fmt)
    dq, dk, dv = cfa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dev["cu"], scale=w.scale,
                              causal=w.causal, cu_seqlens_host=dev["cu_host"], mx=PATH[fmt], saved=saved)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("lengths,hq,hkv,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, True),
    ([513, 31, 200, 33], 4, 2, True),
    ([700, 1], 4, 1, True),
    ([100, 257], 2, 1, False),
])
def test_fp6_backward_random_documents(lengths, hq, hkv, causal, fmt):
    w = W.make_random(seed=1900 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, causal=causal)
    announce(PATH[fmt] + " bwd random", lengths, hq, hkv, causal)
    _, _, dq, dk, dv = _fwd_bwd(w, upload(w), fmt)
    ref = mxa.attn_mx_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal, qk=fmt)
    errs = [rel_l2(to_f64(a), b) for a, b in zip((dq, dk, dv), ref)]
    print("rel-L2 dq dk dv", errs)
    assert max(errs) <= MX_TOL


def test_fp6_backward_causality_isolation_determinism(fmt):
    lengths = [300, 129, 1, 64, 700]
    w = W.make_random(seed=1944, lengths=lengths, hq=4, hkv=2)
    announce(PATH[fmt] + " bwd invariants", lengths)
    dev = upload(w)
    r1 = _fwd_bwd(w, dev, fmt)
    r2 = _fwd_bwd(w, dev, fmt)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    cu = w.cu_seqlens
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=128, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1],
                         do=w.do[s0:s1])
        ra = _fwd_bwd(sub, upload(sub), fmt)
        for a, b in zip(ra[2:], r1[2:]):
            assert torch.equal(a, b[s0:s1])
    for jl in (0, 31, 32, 127, 128, 699):
        j = int(cu[4]) + jl
        dev2 = {kk: vv.clone() for kk, vv in dev.items()}
        for name in ("q", "k", "v", "do"):
            dev2[name][j] = dev2[name][j] * 7.5 + 30.0
        r3 = _fwd_bwd(w, dev2, fmt)
        assert torch.equal(r3[2][:j], r1[2][:j]), jl


def test_fp6_backward_workload_4_sampled(fmt):
    w = W.make_workload(4)
    announce(PATH[fmt] + " bwd workload 4", w.n_docs)
    dev = upload(w)
    _, _, dq, dk, dv = _fwd_bwd(w, dev, fmt)
    L_all = np.diff(w.cu_seqlens)
    n = int(np.argmax(L_all))
    s0, L = int(w.cu_seqlens[n]), int(L_all[n])
    hh = 11
    sl = slice(s0, s0 + L)
    q, k, v, do = (W.bf16_bits_to_f64(getattr(w, x)[sl][:, [hh]]) for x in ("q", "k", "v", "do"))
    rows = np.unique(np.array([0, 1, 127, 128, 255, 256, L // 2, L - 129, L - 1]))
    _, _, rdq, _, _ = mxa.attn_mx_rows(q, k, v, do, rows, w.scale, qk=fmt)
    e_dq = rel_l2(to_f64(dq[sl][rows][:, [hh]]), rdq)
    # keys in the last 200 rows see only queries among those rows: their dK, dV are complete
    tail = np.arange(L - 200, L)
    _, _, _, pdk, pdv = mxa.attn_mx_rows(q, k, v, do, tail, w.scale, qk=fmt)
    e_dk = rel_l2(to_f64(dk[sl][L - 200:, [hh]]), pdk[L - 200:])
    e_dv = rel_l2(to_f64(dv[sl][L - 200:, [hh]]), pdv[L - 200:])
    print("rel-L2 dq dk dv (sampled)", e_dq, e_dk, e_dv)
    assert max(e_dq, e_dk, e_dv) <= MX_TOL
