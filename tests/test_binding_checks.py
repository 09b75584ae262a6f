"""Argument checks of the Python binding (CPU): the library sees only pointers and sizes, so the
binding checks shapes, dtypes and buffer sizes before anything reaches a kernel. Every call here
uses CPU tensors: a call whose metadata is valid gets as far as the device check."""
import pytest
import torch

import causal_flashattention_amd as cfa

BF = torch.bfloat16
GPU_MSG = "must live on the GPU"


def _qkv(T=64, hq=4, hkv=2, d=128, dtype=BF):
    return (torch.zeros(T, hq, d, dtype=dtype), torch.zeros(T, hkv, d, dtype=dtype),
            torch.zeros(T, hkv, d, dtype=dtype), torch.tensor([0, 40, 64], dtype=torch.int32))


def test_fwd_metadata():
    q, k, v, cu = _qkv()
    with pytest.raises(ValueError, match=GPU_MSG):
        cfa.attn_fwd(q, k, v, cu)
    with pytest.raises(ValueError, match="does not match q"):
        cfa.attn_fwd(q, k[:60], v[:60], cu)                 # self-attention: same token count
    with pytest.raises(ValueError, match="does not match q"):
        cfa.attn_fwd(q, k[:, :, :64].contiguous(), v[:, :, :64].contiguous(), cu)
    with pytest.raises(ValueError, match="v: shape"):
        cfa.attn_fwd(q, k, v[:, :1].contiguous(), cu)
    with pytest.raises(TypeError, match="dtype"):
        cfa.attn_fwd(q, k.float(), v.float(), cu)
    with pytest.raises(ValueError, match="int32"):
        cfa.attn_fwd(q, k, v, cu.long())
    with pytest.raises(ValueError, match="out: shape"):
        cfa.attn_fwd(q, k, v, cu, out=torch.zeros(64, 4, 64, dtype=BF))
    with pytest.raises(TypeError, match="lse: dtype"):
        cfa.attn_fwd(q, k, v, cu, lse=torch.zeros(4, 64, dtype=BF))
    with pytest.raises(ValueError, match="saved holds"):
        cfa.attn_fwd(q, k, v, cu, mx="mxfp6_e3m2", saved=torch.zeros(100, dtype=torch.uint8))


def test_bwd_metadata():
    q, k, v, cu = _qkv()
    o, do, lse = torch.zeros_like(q), torch.zeros_like(q), torch.zeros(4, 64)
    with pytest.raises(ValueError, match=GPU_MSG):
        cfa.attn_bwd(q, k, v, o, lse, do, cu)
    with pytest.raises(ValueError, match="dout: shape"):
        cfa.attn_bwd(q, k, v, o, lse, do[:32], cu)
    with pytest.raises(ValueError, match="dk: shape"):
        cfa.attn_bwd(q, k, v, o, lse, do, cu, dk=torch.zeros_like(q))
    with pytest.raises(ValueError, match="dlse: shape"):
        cfa.attn_bwd(q, k, v, o, lse, do, cu, dlse=torch.zeros(4, 63))
    with pytest.raises(ValueError, match="saved holds"):
        cfa.attn_bwd(q, k, v, o, lse, do, cu, mx="mxfp4", saved=torch.zeros(8, dtype=torch.uint8))


def test_cross_and_decode_metadata():
    q = torch.zeros(30, 4, 64, dtype=BF)
    k = torch.zeros(50, 2, 64, dtype=BF)
    cq, ck = torch.tensor([0, 10, 30], dtype=torch.int32), torch.tensor([0, 20, 50], dtype=torch.int32)
    with pytest.raises(ValueError, match=GPU_MSG):
        cfa.attn_fwd_cross(q, k, k.clone(), cq, ck)
    with pytest.raises(ValueError, match="same number of documents"):
        cfa.attn_fwd_cross(q, k, k.clone(), cq, ck[:2])
    with pytest.raises(ValueError, match="lse: shape"):
        cfa.attn_bwd_cross(q, k, k.clone(), q.clone(), torch.zeros(4, 50), q.clone(), cq, ck)
    qd = torch.zeros(2, 4, 128, dtype=BF)
    codes = torch.zeros(50, 2, 128, dtype=torch.uint8)
    sc = torch.zeros(50, 2, 4, dtype=torch.uint8)
    with pytest.raises(ValueError, match=GPU_MSG):
        cfa.attn_decode(qd, codes, codes.clone(), ck, k_scales=sc, v_scales=sc.clone())
    with pytest.raises(ValueError, match="k_scales: shape"):
        cfa.attn_decode(qd, codes, codes.clone(), ck, k_scales=sc[:, :1].contiguous(), v_scales=sc.clone())
    with pytest.raises(ValueError, match="3 entries for 3 sequences"):
        cfa.attn_decode(torch.zeros(3, 4, 128, dtype=BF), codes, codes.clone(), ck, k_scales=sc, v_scales=sc)


def test_quantiser_metadata():
    x = torch.zeros(64, 2, 128, dtype=BF)
    for fn, width in ((cfa.mx_quantize_fp4, 64), (cfa.mx_quantize_fp6, 96), (cfa.mx_quantize_fp6_e3m2, 96)):
        with pytest.raises(ValueError, match=GPU_MSG):
            fn(x)
        with pytest.raises(ValueError, match="codes: shape"):
            fn(x, codes=torch.zeros(64, 2, width + 1, dtype=torch.uint8))
        with pytest.raises(TypeError, match="bf16"):
            fn(x.float())
    cu = torch.tensor([0, 64], dtype=torch.int32)
    with pytest.raises(ValueError, match=GPU_MSG):
        cfa.mx_quantize(x, cu, 1)
    with pytest.raises(ValueError, match="codes: shape"):
        cfa.mx_quantize(x, cu, 1, t_pad=96, codes=torch.zeros(2, 128, 64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales: shape"):
        cfa.mx_quantize(x, cu, 0, scales=torch.zeros(64, 2, 3, dtype=torch.uint8))
