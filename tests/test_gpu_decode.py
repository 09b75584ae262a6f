"""GPU parity of decoding over a packed KV cache (bf16 or MX-quantised), through the C ABI.

Oracle: ``oracle.decode`` on the exact cache values (pinned on the CPU against the causal
attention oracle's last row and closed forms). Tolerance, from the arithmetic: the cache values
(E4M3 × 2^e, or bf16) and Q are exact in bf16; P is rounded to bf16 (2^-9 relative) before the
value product and O to bf16 on output (2^-9), fp32 elsewhere, so
max |o - o_ref| <= 1e-2 · max(1, max |o_ref|) and |lse - lse_ref| <= 1e-3 · max(1, |lse_ref|).
Bit-identity on the GPU: reruns, and each sequence alone against the packed batch.
"""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import decode as dec
from gpu_helpers import DEV, announce, to_f64

pytestmark = pytest.mark.gpu


def _up_bf16(a):
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def _upload(w):
    d = {"q": _up_bf16(w.q), "cu": torch.from_numpy(w.cu_seqlens_k.astype(np.int32)).to(DEV),
         "cu_host": torch.from_numpy(w.cu_seqlens_k.astype(np.int32))}
    if w.kv == "mxfp8":
        for n in ("k", "v", "k_scales", "v_scales"):
            d[n] = torch.from_numpy(getattr(w, n).copy()).to(DEV)
    else:
        d["k"], d["v"] = _up_bf16(w.k), _up_bf16(w.v)
        d["k_scales"] = d["v_scales"] = None
    return d


def _run(w, dev):
    o, lse = cfa.attn_decode(dev["q"], dev["k"], dev["v"], dev["cu"], k_scales=dev["k_scales"],
                             v_scales=dev["v_scales"], scale=w.scale, cu_seqlens_k_host=dev["cu_host"])
    torch.cuda.synchronize()
    return o, lse


def _ref(w, seqs=None):
    if w.kv == "mxfp8":
        k, v = dec.dequantize_cache(w.k, w.k_scales), dec.dequantize_cache(w.v, w.v_scales)
    else:
        k, v = W.bf16_bits_to_f64(w.k), W.bf16_bits_to_f64(w.v)
    q = W.bf16_bits_to_f64(w.q)
    cu = w.cu_seqlens_k
    if seqs is None:
        return dec.decode_attention(q, k, v, cu, w.scale)
    outs = []
    for b in seqs:
        s0, s1 = int(cu[b]), int(cu[b + 1])
        outs.append(dec.decode_attention(q[b:b + 1], k[s0:s1], v[s0:s1], np.array([0, s1 - s0]), w.scale))
    return outs


def _check(o, lse, ro, rl):
    o = to_f64(o)
    lse = lse.detach().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o - ro)) <= 1e-2 * max(1.0, np.max(np.abs(ro)))
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin) and np.all(lse[~fin] == -np.inf)
    assert np.all(np.abs(lse[fin] - rl[fin]) <= 1e-3 * np.maximum(1.0, np.abs(rl[fin])))


LENGTHS = [0, 1, 31, 32, 33, 64, 255, 256, 257, 700, 3000]


@pytest.mark.parametrize("kv", ["bf16", "mxfp8"])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 4, 128), (32, 1, 128), (40, 1, 128), (8, 2, 64)])
def test_decode_random(kv, hq, hkv, d):
    w = W.make_decode(seed=500 + hq + d, lengths=LENGTHS, hq=hq, hkv=hkv, d=d, kv=kv)
    announce("decode", kv, hq, hkv, d)
    o, lse = _run(w, _upload(w))
    ro, rl = _ref(w)
    _check(o, lse, ro, rl)


@pytest.mark.parametrize("kv", ["bf16", "mxfp8"])
def test_decode_determinism_and_isolation(kv):
    w = W.make_decode(seed=600, lengths=[300, 0, 1, 1000, 257], hq=8, hkv=2, kv=kv)
    announce("decode invariants", kv)
    dev = _upload(w)
    o1, l1 = _run(w, dev)
    o2, l2 = _run(w, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cu = w.cu_seqlens_k
    for b in range(w.n_seqs):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        sub = W.DecodeWorkload(name="one", hq=8, hkv=2, d=128, kv=kv, scale=w.scale,
                               cu_seqlens_k=np.array([0, s1 - s0], np.int32), q=w.q[b:b + 1], k=w.k[s0:s1],
                               v=w.v[s0:s1], k_scales=None if w.k_scales is None else w.k_scales[s0:s1],
                               v_scales=None if w.v_scales is None else w.v_scales[s0:s1])
        oa, la = _run(sub, _upload(sub))
        assert torch.equal(oa[0], o1[b]) and torch.equal(la[:, 0], l1[:, b]), b


@pytest.mark.parametrize("kv", ["bf16", "mxfp8"])
def test_decode_serving_batch_sampled(kv):
    """64 sequences of 512..32768 cached tokens (hq = 32, hkv = 8); sampled sequences checked."""
    lengths = W.decode_batch_lengths(seed=7, n_seqs=64)
    w = W.make_decode(seed=700, lengths=lengths, hq=32, hkv=8, kv=kv)
    announce("decode batch", kv, sum(lengths))
    o, lse = _run(w, _upload(w))
    seqs = [0, 1, int(np.argmax(lengths)), 63]
    for b, (ro, rl) in zip(seqs, _ref(w, seqs)):
        _check(o[b:b + 1], lse[:, b:b + 1], ro, rl)
