"""GPU parity of the forward pass against the float64 oracle (through the C ABI).

Tolerances: bf16 O max-abs <= 1e-2, LSE max-abs <= 1e-3; fp32 O and LSE max-abs <= 1e-5.
Bit-identity (GPU against itself): rerun determinism, causality, document isolation.
"""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import attention as ref
from gpu_helpers import announce, head_group, to_f64, upload, DEV

pytestmark = pytest.mark.gpu

BF16_O_TOL = 1e-2
LSE_TOL = 1e-3


def _fwd(w, dev, **kw):
    o, lse, _ = cfa.attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu"], scale=w.scale, causal=w.causal,
                             cu_seqlens_host=dev["cu_host"], **kw)
    torch.cuda.synchronize()
    return o, lse


def _oracle_heads(w, g):
    hs = head_group(w, g)
    q = w.f64("q")[:, hs]
    k = w.f64("k")[:, [g]]
    v = w.f64("v")[:, [g]]
    o, lse = ref.attn_fwd(q, k, v, w.cu_seqlens, w.scale, w.causal)
    return hs, o, lse


def test_fp32_single_document():
    w = W.make_workload(1)
    announce("fwd fp32 workload 1", w.total_tokens)
    dev = upload(w)
    o, lse = _fwd(w, dev)
    ro, rl = ref.attn_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale)
    assert np.max(np.abs(to_f64(o) - ro)) <= 1e-5
    assert np.max(np.abs(to_f64(lse) - rl)) <= 1e-5


@pytest.mark.parametrize("lengths,hq,hkv,d,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, 128, True),
    ([77, 256, 33, 1], 4, 2, 64, True),
    ([100, 257], 2, 1, 128, False),
])
def test_fp32_random_documents(lengths, hq, hkv, d, causal):
    """The fp32 path beyond workload 1: packed ragged documents, GQA, d = 64 and 128, non-causal."""
    w = W.make_random(seed=700 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, d=d, dtype="f32", causal=causal)
    announce("fwd fp32 random", lengths, hq, hkv, d, causal)
    o, lse = _fwd(w, upload(w))
    assert o.dtype == torch.float32
    ro, rl = ref.attn_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale, causal)
    assert np.max(np.abs(to_f64(o) - ro)) <= 1e-5
    assert np.max(np.abs(to_f64(lse) - rl)) <= 1e-5


@pytest.mark.parametrize("lengths,hq,hkv,d", [
    ([1, 5, 64, 127, 129, 300], 2, 2, 128),
    ([513, 31, 200], 8, 2, 128),
    ([700, 1], 4, 1, 128),
    ([77, 256, 1000], 4, 4, 64),
    ([33, 2, 190], 6, 3, 128),
])
def test_bf16_random_documents(lengths, hq, hkv, d):
    w = W.make_random(seed=sum(lengths) + hq, lengths=lengths, hq=hq, hkv=hkv, d=d)
    announce("fwd bf16 random", lengths, hq, hkv, d)
    dev = upload(w)
    o, lse = _fwd(w, dev)
    ro, rl = ref.attn_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale)
    assert np.max(np.abs(to_f64(o) - ro)) <= BF16_O_TOL
    assert np.max(np.abs(to_f64(lse) - rl)) <= LSE_TOL


def test_bf16_non_causal():
    w = W.make_random(seed=3, lengths=[100, 257], hq=2, hkv=1, causal=False)
    announce("fwd bf16 non-causal")
    dev = upload(w)
    o, lse = _fwd(w, dev)
    ro, rl = ref.attn_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale, causal=False)
    assert np.max(np.abs(to_f64(o) - ro)) <= BF16_O_TOL
    assert np.max(np.abs(to_f64(lse) - rl)) <= LSE_TOL


def test_bf16_packed_workload_2():
    w = W.make_workload(2)
    announce("fwd bf16 workload 2", w.n_docs)
    dev = upload(w)
    o, lse = _fwd(w, dev)
    o, lse = to_f64(o), to_f64(lse)
    for g in (0, 11):
        hs, ro, rl = _oracle_heads(w, g)
        assert np.max(np.abs(o[:, hs] - ro)) <= BF16_O_TOL
        assert np.max(np.abs(lse[hs] - rl)) <= LSE_TOL


def test_bf16_gqa_workload_3_sampled_rows():
    """Full 32K-token GQA shape; one kv group, sampled query rows computed by the oracle alone."""
    w = W.make_workload(3, with_grad=False)
    announce("fwd bf16 workload 3")
    dev = upload(w)
    o, lse = _fwd(w, dev)
    o, lse = to_f64(o), to_f64(lse)
    g = 5
    hs = head_group(w, g)
    rows = np.array([0, 1, 127, 128, 4095, 16383, 16384, 32766, 32767])
    q = w.f64("q")
    k = w.f64("k")[:, g]
    v = w.f64("v")[:, g]
    for i in rows:
        for h in hs:
            s = w.scale * (k[:i + 1] @ q[i, h])
            m = s.max()
            p = np.exp(s - m)
            ro = p @ v[:i + 1] / p.sum()
            assert np.max(np.abs(o[i, h] - ro)) <= BF16_O_TOL
            assert abs(lse[h, i] - (m + np.log(p.sum()))) <= LSE_TOL


def test_bf16_determinism_isolation_causality():
    lengths = [300, 129, 1, 64, 700]
    w = W.make_random(seed=11, lengths=lengths, hq=4, hkv=2)
    announce("fwd bf16 invariants", lengths)
    dev = upload(w)
    o1, l1 = _fwd(w, dev)
    o2, l2 = _fwd(w, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cu = w.cu_seqlens
    # isolation: each document alone
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=128, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1])
        d1 = upload(sub)
        oa, la = _fwd(sub, d1)
        assert torch.equal(oa, o1[s0:s1]) and torch.equal(la, l1[:, s0:s1])
    # causality: perturb token j of document 4 in q, k, v
    for jl in (0, 63, 64, 200, 699):
        j = int(cu[4]) + jl
        dev2 = {kk: vv.clone() for kk, vv in dev.items()}
        for name in ("q", "k", "v"):
            dev2[name][j] = dev2[name][j] * 3 + 1
        o3, l3 = _fwd(w, dev2)
        assert torch.equal(o3[:j], o1[:j]) and torch.equal(l3[:, :j], l1[:, :j])


def test_empty_documents_and_zero_tokens():
    w = W.make_random(seed=5, lengths=[0, 40, 0, 0, 90, 0], hq=2, hkv=2)
    announce("fwd bf16 empty docs")
    dev = upload(w)
    o, lse = _fwd(w, dev)
    ro, rl = ref.attn_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale)
    assert np.max(np.abs(to_f64(o) - ro)) <= BF16_O_TOL
    z = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    cu = torch.zeros(2, dtype=torch.int32, device=DEV)
    o, lse, _ = cfa.attn_fwd(z, z, z, cu)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 128)
