"""GPU parity of the extensions beyond the causal GQA base case, through the C ABI.

* A gradient flowing into the forward's LSE (``dlse``): bf16 and MXFP8 against the oracles'
  ``dlse`` term (pinned on the CPU by central differences of the forward).
* Multi-query attention (one kv head for every query head) and head dim 256, both of which
  FlashAttention-2 added ("FlashAttention (HU)", "Evolúció és további fejlesztések",
  FlashAttention-2 (2023)).

Tolerances as for the base case: bf16 O max-abs <= 1e-2 and gradients rel-L2 <= 1e-2; MXFP8
rel-L2 <= 3e-2 against the MX oracle.
"""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import attention as ref
from oracle import mx_attention as mxa
from gpu_helpers import DEV, announce, rel_l2, to_f64, upload

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-2
O_TOL = 1e-2
LSE_TOL = 1e-3
MX_TOL = 3e-2


def _dlse(w, seed):
    """Seeded upstream gradient of LSE, [hq, T] float32 (the same bits on both sides)."""
    return np.random.default_rng(seed).standard_normal((w.hq, w.total_tokens)).astype(np.float32)


def _run(w, dev, mx, dlse=None):
    o, lse, saved = cfa.attn_fwd(dev["q"], dev["k"], dev["v"], dev["cu"], scale=w.scale, causal=w.causal,
                                 cu_seqlens_host=dev["cu_host"], mx=mx)
    dl = torch.from_numpy(dlse).to(DEV) if dlse is not None else None
    dq, dk, dv = cfa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dev["cu"], scale=w.scale,
                              causal=w.causal, cu_seqlens_host=dev["cu_host"], mx=mx, saved=saved, dlse=dl)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("lengths,hq,hkv,d,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, 128, True),
    ([513, 31, 200], 8, 2, 128, True),
    ([77, 256, 400], 4, 4, 64, True),
    ([100, 257], 2, 1, 128, False),
])
def test_bf16_lse_gradient(lengths, hq, hkv, d, causal):
    w = W.make_random(seed=300 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, d=d, causal=causal)
    dlse = _dlse(w, seed=301 + sum(lengths))
    announce("bwd bf16 dlse", lengths, hq, hkv, d, causal)
    dev = upload(w)
    _, _, dq, dk, dv = _run(w, dev, False, dlse)
    want = ref.attn_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal,
                        dlse=dlse.astype(np.float64))
    base = ref.attn_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal)
    for got, wnt, b in zip((dq, dk), want[:2], base[:2]):
        assert rel_l2(to_f64(got), wnt) <= GRAD_TOL
        assert rel_l2(b, wnt) > 3 * GRAD_TOL           # the dLSE term is large enough to be seen
    assert rel_l2(to_f64(dv), want[2]) <= GRAD_TOL


def test_bf16_lse_gradient_zero_is_no_gradient():
    """dlse = 0 gives bit-identical outputs to dlse = NULL."""
    w = W.make_random(seed=310, lengths=[300, 45, 129], hq=4, hkv=2)
    announce("bwd bf16 dlse zero")
    dev = upload(w)
    r0 = _run(w, dev, False)
    r1 = _run(w, dev, False, np.zeros((w.hq, w.total_tokens), np.float32))
    for a, b in zip(r0, r1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("lengths,hq,hkv,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, True),
    ([100, 257], 2, 1, False),
])
def test_mx_lse_gradient(lengths, hq, hkv, causal):
    w = W.make_random(seed=320 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, causal=causal)
    dlse = _dlse(w, seed=321 + sum(lengths))
    announce("bwd mx dlse", lengths, hq, hkv, causal)
    dev = upload(w)
    _, _, dq, dk, dv = _run(w, dev, True, dlse)
    want = mxa.attn_mx_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal,
                           dlse=dlse.astype(np.float64))
    errs = [rel_l2(to_f64(a), b) for a, b in zip((dq, dk, dv), want)]
    print("rel-L2 dq dk dv", errs)
    assert max(errs) <= MX_TOL


@pytest.mark.parametrize("mx", [False, True])
def test_mqa_one_kv_head(mx):
    """hq = 16 query heads on a single kv head."""
    lengths = [700, 129, 1, 300]
    w = W.make_random(seed=330, lengths=lengths, hq=16, hkv=1, causal=True)
    announce("mqa fwd+bwd", lengths, "mx" if mx else "bf16")
    dev = upload(w)
    o, lse, dq, dk, dv = _run(w, dev, mx)
    if mx:
        ro, rl = mxa.attn_mx_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale)
        assert rel_l2(to_f64(o), ro) <= MX_TOL
        g = mxa.attn_mx_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale)
        errs = [rel_l2(to_f64(a), b) for a, b in zip((dq, dk, dv), g)]
        assert max(errs) <= MX_TOL, errs
    else:
        ro, rl = ref.attn_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale)
        assert np.max(np.abs(to_f64(o) - ro)) <= O_TOL
        g = ref.attn_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale)
        for a, b in zip((dq, dk, dv), g):
            assert rel_l2(to_f64(a), b) <= GRAD_TOL


@pytest.mark.parametrize("lengths,hq,hkv,causal", [
    ([1, 5, 64, 127, 129, 300], 2, 2, True),
    ([513, 31, 200], 8, 2, True),
    ([700, 1], 4, 1, True),
    ([100, 257], 2, 1, False),
])
def test_head_dim_256(lengths, hq, hkv, causal):
    w = W.make_random(seed=340 + sum(lengths), lengths=lengths, hq=hq, hkv=hkv, d=256, causal=causal)
    announce("d=256 fwd+bwd", lengths, hq, hkv, causal)
    dev = upload(w)
    o, lse, dq, dk, dv = _run(w, dev, False)
    ro, rl = ref.attn_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale, causal)
    assert np.max(np.abs(to_f64(o) - ro)) <= O_TOL
    assert np.max(np.abs(to_f64(lse) - rl)) <= LSE_TOL
    g = ref.attn_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale, causal)
    errs = [rel_l2(to_f64(a), b) for a, b in zip((dq, dk, dv), g)]
    print("rel-L2 dq dk dv", errs)
    assert max(errs) <= GRAD_TOL


def test_head_dim_256_determinism_isolation_causality():
    lengths = [300, 129, 1, 64, 200]
    w = W.make_random(seed=350, lengths=lengths, hq=4, hkv=2, d=256)
    announce("d=256 invariants", lengths)
    dev = upload(w)
    r1 = _run(w, dev, False)
    r2 = _run(w, dev, False)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    cu = w.cu_seqlens
    for n in range(len(lengths)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sub = W.Workload(name="doc", total_tokens=s1 - s0, hq=4, hkv=2, d=256, dtype="bf16", scale=w.scale,
                         cu_seqlens=np.array([0, s1 - s0], np.int32), q=w.q[s0:s1], k=w.k[s0:s1], v=w.v[s0:s1],
                         do=w.do[s0:s1])
        ra = _run(sub, upload(sub), False)
        assert torch.equal(ra[0], r1[0][s0:s1]) and torch.equal(ra[1], r1[1][:, s0:s1])
        for a, b in zip(ra[2:], r1[2:]):
            assert torch.equal(a, b[s0:s1])
    for jl in (0, 63, 64, 150, 199):
        j = int(cu[4]) + jl
        dev2 = {kk: vv.clone() for kk, vv in dev.items()}
        for name in ("q", "k", "v", "do"):
            dev2[name][j] = dev2[name][j] * 3.0 + 1.0
        r3 = _run(w, dev2, False)
        assert torch.equal(r3[0][:j], r1[0][:j]), jl       # O of earlier queries
        assert torch.equal(r3[2][:j], r1[2][:j]), jl       # dQ of earlier queries


@pytest.mark.parametrize("mx,qk", [("mxfp4", "e2m1"), ("mxfp6", "e2m3"), ("mxfp6_e3m2", "e3m2")])
def test_narrow_mx_mqa_with_lse_gradient(mx, qk):
    """The narrow score formats on MQA (16 query heads, one kv head) with a dlse input, against
    the MX oracle with the same score format."""
    lengths = [700, 129, 1, 300]
    w = W.make_random(seed=340, lengths=lengths, hq=16, hkv=1, causal=True)
    dlse = _dlse(w, seed=341)
    announce("mqa narrow mx fwd+bwd dlse", lengths, mx)
    dev = upload(w)
    o, lse, dq, dk, dv = _run(w, dev, mx, dlse)
    ro, rl = mxa.attn_mx_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.cu_seqlens, w.scale, qk=qk)
    assert rel_l2(to_f64(o), ro) <= MX_TOL
    assert np.max(np.abs(to_f64(lse) - rl)) <= LSE_TOL
    g = mxa.attn_mx_bwd(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do"), w.cu_seqlens, w.scale,
                        dlse=dlse.astype(np.float64), qk=qk)
    errs = [rel_l2(to_f64(a), b) for a, b in zip((dq, dk, dv), g)]
    print("rel-L2 dq dk dv", errs)
    assert max(errs) <= MX_TOL, errs
