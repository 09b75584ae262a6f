"""Causal packed flash attention for AMD MI355X (gfx950).

Thin Python binding of the C ABI in ``include/cfa.h`` (``libcfa.so`` in this directory).
PyTorch provides device memory and the current HIP stream; every step of the computation runs
in the library's HIP kernels. There is no CPU or PyTorch fallback: a missing library or a
failing call raises.

    o, lse, saved = attn_fwd(q, k, v, cu_seqlens)          # q [T, hq, d], k/v [T, hkv, d]
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, cu_seqlens, saved=saved)
    codes, scales = mx_quantize(x, cu_seqlens, axis=0)     # MXFP8 E4M3 + E8M0, blocks of 32
    o, lse = attn_decode(q1, k_cache, v_cache, cu_seqlens_k)  # one query per sequence, KV cache
"""
import ctypes
import math

import torch

from . import _lib
from ._lib import CFA_BF16, CFA_F32, CFA_MXFP4, CFA_MXFP6, CFA_MXFP6_E3M2, CFA_MXFP8, CfaError

__all__ = ["attn_fwd", "attn_bwd", "attn_bwd_noalloc", "device_error", "attn_fwd_cross", "attn_bwd_cross", "attn_decode", "mx_quantize", "mx_quantize_fp4", "mx_quantize_fp6", "mx_quantize_fp6_e3m2", "workspace_bytes", "saved_bytes", "CfaError",
           "CFA_F32", "CFA_BF16", "CFA_MXFP8", "CFA_MXFP4", "CFA_MXFP6", "CFA_MXFP6_E3M2", "library_path"]


def library_path():
    return _lib.LIB_PATH


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _host_cu(cu_seqlens, cu_seqlens_host):
    if cu_seqlens_host is None:
        return None
    h = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    assert h.device.type == "cpu"
    return h


def _dtype_code(x, mx):
    """mx: False (bf16 / fp32 by x.dtype), True or "mxfp8" (MXFP8), "mxfp4" (MXFP4/FP8),
    "mxfp6" (MXFP6/FP8, E2M3 score operands), "mxfp6_e3m2" (MXFP6/FP8, E3M2 score operands)."""
    if mx:
        if x.dtype != torch.bfloat16:
            raise TypeError("the MX paths take bf16 inputs")
        if mx == "mxfp4":
            return CFA_MXFP4
        if mx == "mxfp6":
            return CFA_MXFP6
        if mx == "mxfp6_e3m2":
            return CFA_MXFP6_E3M2
        if mx is True or mx == "mxfp8":
            return CFA_MXFP8
        raise ValueError(f"unknown MX path {mx!r}")
    if x.dtype == torch.bfloat16:
        return CFA_BF16
    if x.dtype == torch.float32:
        return CFA_F32
    raise TypeError(f"unsupported dtype {x.dtype}")


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, shape, dtype, name):
    """Metadata check of an optional tensor argument (the library sees only pointers and sizes)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _check_qkv(q, k, v, same_tokens):
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q, k, v must be [tokens, heads, head_dim]")
    _expect(v, k.shape, k.dtype, "v")
    if k.dtype != q.dtype:
        raise TypeError(f"k: dtype {k.dtype}, q: {q.dtype}")
    if k.shape[2] != q.shape[2] or (same_tokens and k.shape[0] != q.shape[0]):
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)}")


def _check_cu(cu, name="cu_seqlens"):
    if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2:
        raise ValueError(f"{name} must be int32 [n_docs + 1]")


def _nbytes(t):
    return t.numel() * t.element_size()


def _at_least(t, n, name):
    if t is not None and _nbytes(t) < n:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, needs {n}")


def device_error(workspace):
    """The validation flag the last call left in ``workspace`` (synchronises the current stream):
    0 for a well-formed device cu_seqlens, else bit 0 = cu[0] != 0, bit 1 = a decreasing entry,
    bit 2 = cu[n_docs] != total_tokens (every document was then treated as empty)."""
    _check_dev(workspace)
    flag = ctypes.c_int(-1)
    _lib.check(_lib.lib().cfa_device_error(_ptr(workspace), _stream(), ctypes.byref(flag)))
    return flag.value


def workspace_bytes(pass_, total_tokens, n_docs, hq, hkv, d, dtype):
    return _lib.lib().cfa_workspace_bytes(pass_, total_tokens, n_docs, hq, hkv, d, dtype)


def saved_bytes(total_tokens, n_docs, hq, hkv, d, dtype):
    return _lib.lib().cfa_saved_bytes(total_tokens, n_docs, hq, hkv, d, dtype)


def attn_fwd(q, k, v, cu_seqlens, *, scale=None, causal=True, cu_seqlens_host=None, max_seqlen=0,
             mx=False, out=None, lse=None, saved=None, workspace=None):
    """Forward pass. Returns (o, lse, saved); ``saved`` is None unless ``mx``."""
    L = _lib.lib()
    _check_qkv(q, k, v, True)
    _check_cu(cu_seqlens)
    T, hq, d = q.shape
    hkv = k.shape[1]
    n_docs = cu_seqlens.numel() - 1
    dt = _dtype_code(q, mx)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (hq, T), torch.float32, "lse")
    if mx:
        _at_least(saved, L.cfa_saved_bytes(T, n_docs, hq, hkv, d, dt), "saved")
    _check_dev(q, k, v, cu_seqlens, out, lse, saved, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, T), dtype=torch.float32, device=dev)
    if mx and saved is None:
        saved = torch.empty(L.cfa_saved_bytes(T, n_docs, hq, hkv, d, dt), dtype=torch.uint8, device=dev)
    if workspace is None:
        nb = L.cfa_workspace_bytes(0, T, n_docs, hq, hkv, d, dt)
        workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    hcu = _host_cu(cu_seqlens, cu_seqlens_host)
    _lib.check(L.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                          _ptr(hcu) if hcu is not None else None, n_docs, T, int(max_seqlen), hq, hkv, d,
                          scale, int(bool(causal)), dt, _ptr(saved) if mx else None, _ptr(workspace),
                          _nbytes(workspace), _stream()))
    return out, lse, saved


def attn_bwd(q, k, v, o, lse, dout, cu_seqlens, *, scale=None, causal=True, cu_seqlens_host=None,
             max_seqlen=0, mx=False, saved=None, dlse=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward pass. Returns (dq, dk, dv) with the layouts and dtype of (q, k, v).

    ``dlse`` (float32 ``[hq, T]``, optional) is the gradient flowing into the forward's lse.
    ``mx`` without ``saved``: the library quantises Q, K and V again (the forward's bytes) into a
    workspace that also holds ``saved_bytes(...)``.
    """
    L = _lib.lib()
    _check_qkv(q, k, v, True)
    _check_cu(cu_seqlens)
    T, hq, d = q.shape
    hkv = k.shape[1]
    n_docs = cu_seqlens.numel() - 1
    dt = _dtype_code(q, mx)
    for t, name in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _expect(t, q.shape, q.dtype, name)
    for t, name in ((dk, "dk"), (dv, "dv")):
        _expect(t, k.shape, k.dtype, name)
    _expect(lse, (hq, T), torch.float32, "lse")
    _expect(dlse, (hq, T), torch.float32, "dlse")
    if mx and saved is not None:
        _at_least(saved, L.cfa_saved_bytes(T, n_docs, hq, hkv, d, dt), "saved")
    _check_dev(q, k, v, o, lse, dout, cu_seqlens, saved, dlse, dq, dk, dv, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        nb = L.cfa_workspace_bytes(1, T, n_docs, hq, hkv, d, dt)
        if mx and saved is None:
            nb += L.cfa_saved_bytes(T, n_docs, hq, hkv, d, dt)
        workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device)
    hcu = _host_cu(cu_seqlens, cu_seqlens_host)
    _lib.check(L.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                          _ptr(dlse) if dlse is not None else None, _ptr(saved) if saved is not None else None, _ptr(dq), _ptr(dk), _ptr(dv),
                          _ptr(cu_seqlens), _ptr(hcu) if hcu is not None else None, n_docs, T,
                          int(max_seqlen), hq, hkv, d, scale, int(bool(causal)), dt, _ptr(workspace),
                          _nbytes(workspace), _stream()))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, cu_seqlens, *, dq, dk, dv, scale=None, causal=True,
                     cu_seqlens_host=None, max_seqlen=0, mx=False, saved=None, dlse=None):
    """``attn_bwd`` whose scratch is the library's fixed per-GPU array (no workspace, no
    allocation by the library). The caller passes the outputs ``dq, dk, dv``; calls that overlap
    on one GPU race (they share the array)."""
    L = _lib.lib()
    _check_qkv(q, k, v, True)
    _check_cu(cu_seqlens)
    T, hq, d = q.shape
    n_docs = cu_seqlens.numel() - 1
    dt = _dtype_code(q, mx)
    for t, name in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _expect(t, q.shape, q.dtype, name)
    for t, name in ((dk, "dk"), (dv, "dv")):
        _expect(t, k.shape, k.dtype, name)
    _expect(lse, (hq, T), torch.float32, "lse")
    _expect(dlse, (hq, T), torch.float32, "dlse")
    if mx and saved is not None:
        _at_least(saved, L.cfa_saved_bytes(T, n_docs, hq, k.shape[1], d, dt), "saved")
    _check_dev(q, k, v, o, lse, dout, cu_seqlens, saved, dlse, dq, dk, dv)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    hcu = _host_cu(cu_seqlens, cu_seqlens_host)
    _lib.check(L.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                  _ptr(dlse) if dlse is not None else None,
                                  _ptr(saved) if saved is not None else None, _ptr(dq), _ptr(dk), _ptr(dv),
                                  _ptr(cu_seqlens), _ptr(hcu) if hcu is not None else None, n_docs, T,
                                  int(max_seqlen), hq, k.shape[1], d, scale, int(bool(causal)), dt, _stream()))
    return dq, dk, dv


def attn_fwd_cross(q, k, v, cu_seqlens_q, cu_seqlens_k, *, scale=None, causal=True, cu_seqlens_q_host=None,
                   cu_seqlens_k_host=None, out=None, lse=None, workspace=None):
    """Cross-attention forward (bf16): query documents on their own key/value documents.
    ``q [Tq, hq, d]``, ``k, v [Tk, hkv, d]``. Returns (o, lse [hq, Tq])."""
    L = _lib.lib()
    _check_qkv(q, k, v, False)
    _check_cu(cu_seqlens_q, "cu_seqlens_q")
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must list the same number of documents")
    if q.dtype != torch.bfloat16:
        raise TypeError("cross-attention takes bf16 inputs")
    Tq, hq, d = q.shape
    Tk, hkv = k.shape[0], k.shape[1]
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (hq, Tq), torch.float32, "lse")
    _check_dev(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, workspace)
    n_docs = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((hq, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    if workspace is None:
        nb = L.cfa_cross_workspace_bytes(0, Tq, Tk, n_docs, hq, hkv, d)
        workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device)
    hq_cu, hk_cu = _host_cu(cu_seqlens_q, cu_seqlens_q_host), _host_cu(cu_seqlens_k, cu_seqlens_k_host)
    _lib.check(L.attn_fwd_cross(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                _ptr(cu_seqlens_k), _ptr(hq_cu) if hq_cu is not None else None,
                                _ptr(hk_cu) if hk_cu is not None else None, n_docs, Tq, Tk, hq, hkv, d, scale,
                                int(bool(causal)), _ptr(workspace), _nbytes(workspace), _stream()))
    return out, lse


def attn_bwd_cross(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, *, scale=None, causal=True,
                   cu_seqlens_q_host=None, cu_seqlens_k_host=None, dlse=None, dq=None, dk=None, dv=None,
                   workspace=None):
    """Cross-attention backward (bf16). Returns (dq, dk, dv)."""
    L = _lib.lib()
    _check_qkv(q, k, v, False)
    _check_cu(cu_seqlens_q, "cu_seqlens_q")
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must list the same number of documents")
    Tq, hq, d = q.shape
    Tk, hkv = k.shape[0], k.shape[1]
    for t, name in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _expect(t, q.shape, q.dtype, name)
    for t, name in ((dk, "dk"), (dv, "dv")):
        _expect(t, k.shape, k.dtype, name)
    _expect(lse, (hq, Tq), torch.float32, "lse")
    _expect(dlse, (hq, Tq), torch.float32, "dlse")
    _check_dev(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dlse, dq, dk, dv, workspace)
    n_docs = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        nb = L.cfa_cross_workspace_bytes(1, Tq, Tk, n_docs, hq, hkv, d)
        workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device)
    hq_cu, hk_cu = _host_cu(cu_seqlens_q, cu_seqlens_q_host), _host_cu(cu_seqlens_k, cu_seqlens_k_host)
    _lib.check(L.attn_bwd_cross(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                _ptr(dlse) if dlse is not None else None, _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(hq_cu) if hq_cu is not None else None,
                                _ptr(hk_cu) if hk_cu is not None else None, n_docs, Tq, Tk, hq, hkv, d, scale,
                                int(bool(causal)), _ptr(workspace), _nbytes(workspace), _stream()))
    return dq, dk, dv


def attn_decode(q, k_cache, v_cache, cu_seqlens_k, *, k_scales=None, v_scales=None, scale=None,
                cu_seqlens_k_host=None, out=None, lse=None, workspace=None):
    """One query token per sequence over a packed KV cache. ``q [B, hq, d]`` bf16; the cache
    ``[Tk, hkv, d]`` is bf16, or uint8 E4M3 codes with ``k_scales, v_scales [Tk, hkv, d/32]``
    uint8 E8M0 bytes. Returns (o [B, hq, d] bf16, lse [hq, B] float32)."""
    L = _lib.lib()
    if q.dim() != 3 or k_cache.dim() != 3:
        raise ValueError("q [n_seqs, hq, d] and the caches [total_k, hkv, d] must be 3-D")
    _expect(v_cache, k_cache.shape, k_cache.dtype, "v_cache")
    if k_cache.shape[2] != q.shape[2]:
        raise ValueError(f"cache {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    B, hq, d = q.shape
    Tk, hkv = k_cache.shape[0], k_cache.shape[1]
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError(f"cu_seqlens_k has {cu_seqlens_k.numel()} entries for {B} sequences")
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        _expect(t, (Tk, hkv, d // 32), torch.uint8, name)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (hq, B), torch.float32, "lse")
    _check_dev(q, k_cache, v_cache, cu_seqlens_k, k_scales, v_scales, out, lse, workspace)
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bf16")
    if k_cache.dtype == torch.uint8:
        kv = CFA_MXFP8
        if k_scales is None or v_scales is None:
            raise ValueError("an MXFP8 cache needs k_scales and v_scales")
    elif k_cache.dtype == torch.bfloat16:
        kv = CFA_BF16
    else:
        raise TypeError(f"unsupported cache dtype {k_cache.dtype}")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, B), dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = L.cfa_decode_workspace_bytes(B, Tk, hq, hkv, d, kv)
        workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device)
    hcu = _host_cu(cu_seqlens_k, cu_seqlens_k_host)
    _lib.check(L.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(out),
                             _ptr(lse), _ptr(cu_seqlens_k), _ptr(hcu) if hcu is not None else None, B, Tk, hq, hkv,
                             d, scale, kv, _ptr(workspace), _nbytes(workspace), _stream()))
    return out, lse


def mx_quantize_fp4(x, *, codes=None, scales=None):
    """MXFP4 (E2M1 + E8M0) quantisation of bf16 ``x [T, h, d]`` in blocks of 32 channels.
    Returns (codes [T, h, d/2] uint8, two per byte, scales [T, h, d/32] uint8)."""
    L = _lib.lib()
    if x.dtype != torch.bfloat16 or x.dim() != 3:
        raise TypeError("x must be bf16 [T, h, d]")
    T, h, d = x.shape
    _expect(codes, (T, h, d // 2), torch.uint8, "codes")
    _expect(scales, (T, h, d // 32), torch.uint8, "scales")
    _check_dev(x, codes, scales)
    codes = torch.empty((T, h, d // 2), dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = torch.empty((T, h, d // 32), dtype=torch.uint8, device=x.device) if scales is None else scales
    _lib.check(L.mx_quantize_fp4(_ptr(x), T, h, d, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def _quantize_fp6(fn, x, codes, scales):
    L = _lib.lib()
    if x.dtype != torch.bfloat16 or x.dim() != 3:
        raise TypeError("x must be bf16 [T, h, d]")
    T, h, d = x.shape
    _expect(codes, (T, h, 3 * d // 4), torch.uint8, "codes")
    _expect(scales, (T, h, d // 32), torch.uint8, "scales")
    _check_dev(x, codes, scales)
    codes = torch.empty((T, h, 3 * d // 4), dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = torch.empty((T, h, d // 32), dtype=torch.uint8, device=x.device) if scales is None else scales
    _lib.check(getattr(L, fn)(_ptr(x), T, h, d, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def mx_quantize_fp6(x, *, codes=None, scales=None):
    """MXFP6 (E2M3 + E8M0) quantisation of bf16 ``x [T, h, d]`` in blocks of 32 channels.
    Returns (codes [T, h, 3d/4] uint8 -- per block a 16-byte part, then per block an 8-byte
    part, see ``mx_quantize_fp6`` in include/cfa.h -- and scales [T, h, d/32] uint8)."""
    return _quantize_fp6("mx_quantize_fp6", x, codes, scales)


def mx_quantize_fp6_e3m2(x, *, codes=None, scales=None):
    """MXFP6 with E3M2 elements (top exponent 4, largest value 28); storage as ``mx_quantize_fp6``."""
    return _quantize_fp6("mx_quantize_fp6_e3m2", x, codes, scales)


def mx_quantize(x, cu_seqlens, axis, *, cu_seqlens_host=None, t_pad=None, codes=None, scales=None,
                workspace=None):
    """MX-quantise bf16 ``x [T, h, d]``. axis 0: blocks along d; axis 1: doc-local token blocks;
    axis 2: the same token blocks in the attention kernels' internal layout.

    Returns (codes uint8, scales uint8): [T, h, d] / [T, h, d/32] for axis 0,
    [h, d, t_pad] / [h, d, t_pad/32] for axis 1 and [h, d, t_pad] / [h, t_pad/32, d] for axis 2
    (t_pad defaults to the size bound).
    """
    L = _lib.lib()
    if x.dtype != torch.bfloat16 or x.dim() != 3:
        raise TypeError("mx_quantize takes bf16 input [T, h, d]")
    _check_cu(cu_seqlens)
    T, h, d = x.shape
    n_docs = cu_seqlens.numel() - 1
    if axis == 0:
        _expect(codes, (T, h, d), torch.uint8, "codes")
        _expect(scales, (T, h, d // 32), torch.uint8, "scales")
    else:
        if t_pad is None:
            t_pad = L.mx_padded_tokens(T, n_docs)
        sshape = (h, t_pad // 32, d) if axis == 2 else (h, d, t_pad // 32)
        _expect(codes, (h, d, t_pad), torch.uint8, "codes")
        _expect(scales, sshape, torch.uint8, "scales")
    _check_dev(x, cu_seqlens, codes, scales, workspace)
    dev = x.device
    if axis == 0:
        t_pad = 0
        codes = torch.empty((T, h, d), dtype=torch.uint8, device=dev) if codes is None else codes
        scales = torch.empty((T, h, d // 32), dtype=torch.uint8, device=dev) if scales is None else scales
    else:
        codes = torch.zeros((h, d, t_pad), dtype=torch.uint8, device=dev) if codes is None else codes
        scales = torch.zeros(sshape, dtype=torch.uint8, device=dev) if scales is None else scales
        if workspace is None:
            workspace = torch.empty(max(L.mx_workspace_bytes(n_docs), 256), dtype=torch.uint8, device=dev)
    hcu = _host_cu(cu_seqlens, cu_seqlens_host)
    _lib.check(L.mx_quantize(_ptr(x), T, h, d, _ptr(cu_seqlens), _ptr(hcu) if hcu is not None else None,
                             n_docs, axis, _ptr(codes), _ptr(scales), int(t_pad),
                             _ptr(workspace) if workspace is not None else None,
                             _nbytes(workspace) if workspace is not None else 0, _stream()))
    return codes, scales
