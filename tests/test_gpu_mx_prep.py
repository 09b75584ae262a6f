"""The MX forward's one operand pass: the d-blocked copies it leaves in `saved` (Q_d and K_d in
the score format, V_d in E4M3) are byte-identical to the reference quantiser's, on ragged packed
documents with an empty one, GQA heads and special values (zero and ±0 tokens, huge and tiny
magnitudes, outlier channels, NaN/Inf blocks). The token-blocked copies share their encoder with
mx_quantize axis 2, whose bytes test_gpu_mx_quantize checks; the backward pass's D and dO copies
are checked through the MX backward parity tests."""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import mx
from gpu_helpers import announce, to_dev, DEV

pytestmark = pytest.mark.gpu

FORMATS = {"mxfp8": (cfa.CFA_MXFP8, None), "mxfp4": (cfa.CFA_MXFP4, "fp4"),
           "mxfp6": (cfa.CFA_MXFP6, "e2m3"), "mxfp6_e3m2": (cfa.CFA_MXFP6_E3M2, "e3m2")}


def _a256(x):
    return (x + 255) // 256 * 256


def _tensor(T, h, seed, specials):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h, 128)).astype(np.float32)
    x *= np.exp(rng.uniform(-20, 20, size=(T, h, 1))).astype(np.float32)
    x[:, :, 7] *= 20.0
    if specials:
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 60), replace=False)
        sp = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-39, 3e38, -3e38, 448.0, 464.0], dtype=np.float32)
        flat[idx] = sp[rng.integers(0, len(sp), size=len(idx))]
    if T > 3:
        x[1] = 0.0
        x[3] = -0.0
    return W.f32_to_bf16_bits(x)


def _score_copy(x64, fmt):
    if fmt is None:
        return mx.quantize_d(x64)
    if fmt == "fp4":
        c, s = mx.quantize_d_fp4(x64)
        return mx.pack_fp4(c), s
    c, s = mx.quantize_d_fp6(x64, fmt)
    return mx.pack_fp6(c), s


def _sections(saved, sizes):
    """Split `saved` at 256-byte aligned section starts, in order."""
    out, off = [], 0
    for n in sizes:
        out.append(saved[off:off + n])
        off = _a256(off + n)
    return out


@pytest.mark.parametrize("specials", [False, True])
@pytest.mark.parametrize("name", list(FORMATS))
def test_forward_pass_saved_copies_bit_exact(name, specials):
    dt, fmt = FORMATS[name]
    lengths = [1, 31, 32, 33, 0, 100, 7, 300, 129]
    T, hq, hkv = sum(lengths), 4, 2
    cu = W.cu_from_lengths(lengths)
    qb, kb, vb = (_tensor(T, h, s + 10 * specials, specials) for h, s in ((hq, 1), (hkv, 2), (hkv, 3)))
    announce("mx prep forward saved copies", name, specials, lengths)
    o, lse, saved = cfa.attn_fwd(to_dev(qb), to_dev(kb), to_dev(vb), torch.from_numpy(cu).to(DEV), mx=name,
                                 cu_seqlens_host=cu)
    torch.cuda.synchronize()
    sv = saved.cpu().numpy()
    cb = {None: 128, "fp4": 64, "e2m3": 96, "e3m2": 96}[fmt]
    sec = _sections(sv, [T * hq * cb, T * hq * 4, T * hkv * cb, T * hkv * 4, T * hkv * 128, T * hkv * 4])
    assert _a256(T * hkv * 128) + _a256(T * hkv * 4) + _a256(T * hq * cb) + _a256(T * hq * 4) \
        + _a256(T * hkv * cb) + _a256(T * hkv * 4) == cfa.saved_bytes(T, len(lengths), hq, hkv, 128, dt)
    for (codes, scales), x in ((sec[0:2], qb), (sec[2:4], kb)):
        rc, rs = _score_copy(W.bf16_bits_to_f64(x), fmt)
        assert np.array_equal(codes, rc.reshape(-1))
        assert np.array_equal(scales, rs.reshape(-1))
    rc, rs = mx.quantize_d(W.bf16_bits_to_f64(vb))
    assert np.array_equal(sec[4], rc.reshape(-1))
    assert np.array_equal(sec[5], rs.reshape(-1))


@pytest.mark.parametrize("name", list(FORMATS))
def test_backward_without_saved_requantises_bit_identically(name):
    """attn_bwd with saved = NULL quantises Q, K and V again into its workspace: the gradients
    equal those of the call that reuses the forward's buffer, bit for bit (also through the
    no-allocation entry point)."""
    dt, _ = FORMATS[name]
    lengths = [33, 0, 300, 129, 64]
    T, hq, hkv = sum(lengths), 4, 2
    cu = W.cu_from_lengths(lengths)
    w = W.make_random(seed=41, lengths=lengths, hq=hq, hkv=hkv)
    q, k, v, do = (to_dev(a) for a in (w.q, w.k, w.v, w.do))
    cu_d = torch.from_numpy(cu).to(DEV)
    announce("mx backward without saved", name, lengths)
    o, lse, saved = cfa.attn_fwd(q, k, v, cu_d, scale=w.scale, mx=name)
    ref = cfa.attn_bwd(q, k, v, o, lse, do, cu_d, scale=w.scale, mx=name, saved=saved)
    got = cfa.attn_bwd(q, k, v, o, lse, do, cu_d, scale=w.scale, mx=name)
    na = [torch.empty_like(t) for t in (q, k, v)]
    cfa.attn_bwd_noalloc(q, k, v, o, lse, do, cu_d, dq=na[0], dk=na[1], dv=na[2], scale=w.scale, mx=name)
    torch.cuda.synchronize()
    for a, b, c in zip(ref, got, na):
        assert torch.equal(a, b) and torch.equal(a, c)
