"""GPU mx_quantize against the reference quantiser: codes and scale bytes bit-identical."""
import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W
from oracle import mx
from gpu_helpers import announce, to_dev, DEV

pytestmark = pytest.mark.gpu


def _special_tensor(T, h, d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h, d)).astype(np.float32)
    x *= np.exp(rng.uniform(-30, 30, size=(T, h, 1))).astype(np.float32)   # per-row magnitudes
    x[:, :, 5] *= 20.0                                                      # an outlier channel
    flat = x.reshape(-1)
    n = flat.size
    idx = rng.choice(n, size=min(n, 200), replace=False)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-39, -1e-39, 3e38, -3e38, 448.0, 464.0, 479.0],
                        dtype=np.float32)
    flat[idx] = specials[rng.integers(0, len(specials), size=len(idx))]
    x[1] = 0.0                     # an all-zero token
    x[2] = -0.0
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("lengths", [[1, 31, 32, 33, 0, 100, 7], [64], [300, 1, 1, 1]])
@pytest.mark.parametrize("d", [128, 64])
def test_mx_quantize_both_axes_bit_exact(lengths, d):
    h = 3
    T = sum(lengths)
    xb = _special_tensor(T, h, d, seed=len(lengths) + d)
    cu = W.cu_from_lengths(lengths)
    announce("mx_quantize", lengths, d)
    x = to_dev(xb)
    cud = torch.from_numpy(cu).to(DEV)
    x64 = W.bf16_bits_to_f64(xb)
    # along d
    c0, s0 = cfa.mx_quantize(x, cud, 0)
    rc, rs = mx.quantize_d(x64)
    torch.cuda.synchronize()
    assert np.array_equal(c0.cpu().numpy(), rc)
    assert np.array_equal(s0.cpu().numpy(), rs)
    # along doc-local tokens
    c1, s1 = cfa.mx_quantize(x, cud, 1, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    rc, rs = mx.quantize_t(x64, cu)
    tp = rc.shape[2]
    assert np.array_equal(c1.cpu().numpy()[:, :, :tp], rc)
    assert np.array_equal(s1.cpu().numpy()[:, :, :tp // 32], rs)


def test_mx_quantize_workload_4_sampled_heads():
    w = W.make_workload(4, with_grad=False)
    announce("mx_quantize workload 4", w.n_docs)
    cu = torch.from_numpy(w.cu_seqlens).to(DEV)
    for name in ("q", "v"):
        x = to_dev(getattr(w, name))
        c0, s0 = cfa.mx_quantize(x, cu, 0)
        c1, s1 = cfa.mx_quantize(x, cu, 1, cu_seqlens_host=w.cu_seqlens)
        torch.cuda.synchronize()
        for hh in (0, 31):
            x64 = W.bf16_bits_to_f64(getattr(w, name)[:, [hh]])
            rc, rs = mx.quantize_d(x64)
            assert np.array_equal(c0[:, hh:hh + 1].cpu().numpy(), rc)
            assert np.array_equal(s0[:, hh:hh + 1].cpu().numpy(), rs)
            rc, rs = mx.quantize_t(x64, w.cu_seqlens)
            tp = rc.shape[2]
            assert np.array_equal(c1[hh:hh + 1, :, :tp].cpu().numpy(), rc)
            assert np.array_equal(s1[hh:hh + 1, :, :tp // 32].cpu().numpy(), rs)
        del x, c0, s0, c1, s1


@pytest.mark.parametrize("d", [128, 64])
def test_mx_quantize_fp4_bit_exact(d):
    """E2M1 codes (packed) and scale bytes bit-identical to the reference, special values included;
    plus a tensor whose scaled elements sit exactly on E2M1 midpoints (ties to the even code)."""
    T, h = 97, 3
    xb = _special_tensor(T, h, d, seed=40 + d)
    rng = np.random.default_rng(41)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 4.0, -0.75, -5.0, 0.0], dtype=np.float32)
    xm = rng.choice(mids, size=(T, h, d)).astype(np.float32)
    xm[:, :, ::32] = 6.0                       # block max 6: e = 0, elements are the midpoints themselves
    for xin in (xb, W.f32_to_bf16_bits(xm)):
        announce("mx_quantize_fp4", d)
        c, s = cfa.mx_quantize_fp4(to_dev(xin))
        torch.cuda.synchronize()
        rc, rs = mx.quantize_d_fp4(W.bf16_bits_to_f64(xin))
        assert np.array_equal(c.cpu().numpy(), mx.pack_fp4(rc))
        assert np.array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("d", [128, 64])
def test_mx_quantize_fp6_bit_exact(d):
    """E2M3 codes (packed) and scale bytes bit-identical to the reference, special values included;
    plus a tensor whose scaled elements sit exactly on E2M3 midpoints (ties to the even code)."""
    T, h = 97, 3
    xb = _special_tensor(T, h, d, seed=50 + d)
    rng = np.random.default_rng(51)
    grid = np.concatenate([np.arange(16) / 8.0, 2.0 + np.arange(8) / 4.0, 4.0 + np.arange(8) / 2.0])
    mids = np.concatenate([(grid[:-1] + grid[1:]) / 2, -(grid[:-1] + grid[1:]) / 2, grid, [0.0]]).astype(np.float32)
    xm = rng.choice(mids, size=(T, h, d)).astype(np.float32)
    xm[:, :, ::32] = 7.5                       # block max 7.5: e = 0, elements are the midpoints themselves
    for xin in (xb, W.f32_to_bf16_bits(xm)):
        announce("mx_quantize_fp6", d)
        c, s = cfa.mx_quantize_fp6(to_dev(xin))
        torch.cuda.synchronize()
        rc, rs = mx.quantize_d_fp6(W.bf16_bits_to_f64(xin))
        assert np.array_equal(c.cpu().numpy(), mx.pack_fp6(rc))
        assert np.array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("d", [128, 64])
def test_mx_quantize_fp6_e3m2_bit_exact(d):
    """E3M2 codes (packed) and scale bytes bit-identical to the reference, special values included;
    plus a tensor whose scaled elements sit exactly on E3M2 midpoints (ties to the even code)."""
    T, h = 97, 3
    xb = _special_tensor(T, h, d, seed=60 + d)
    rng = np.random.default_rng(61)
    grid = np.concatenate([np.arange(4) / 16.0, [2.0 ** k * (1 + m / 4) for k in range(-2, 5) for m in range(4)]])
    mids = np.concatenate([(grid[:-1] + grid[1:]) / 2, -(grid[:-1] + grid[1:]) / 2, grid, [0.0]]).astype(np.float32)
    xm = rng.choice(mids, size=(T, h, d)).astype(np.float32)
    xm[:, :, ::32] = 28.0                      # block max 28: e = 0, elements are the midpoints themselves
    for xin in (xb, W.f32_to_bf16_bits(xm)):
        announce("mx_quantize_fp6_e3m2", d)
        c, s = cfa.mx_quantize_fp6_e3m2(to_dev(xin))
        torch.cuda.synchronize()
        rc, rs = mx.quantize_d_fp6(W.bf16_bits_to_f64(xin), "e3m2")
        assert np.array_equal(c.cpu().numpy(), mx.pack_fp6(rc))
        assert np.array_equal(s.cpu().numpy(), rs)


PIECES = np.array([0, 2, 4, 6, 1, 3, 5, 7])      # stored 4-token piece p holds logical piece PIECES[p]


@pytest.mark.parametrize("lengths", [[1, 31, 32, 33, 0, 100, 7], [300, 1, 1, 1], [4000, 129, 2]])
def test_mx_quantize_kernel_layout_bit_exact(lengths):
    """axis 2 (the token-blocked copies the attention kernels use, V in the forward and dO in the
    backward): after undoing the documented piece order and the block-major scale layout the
    bytes equal the reference quantiser's doc-local token blocks."""
    h, d = 3, 128
    T = sum(lengths)
    xb = _special_tensor(T, h, d, seed=90 + len(lengths))
    cu = W.cu_from_lengths(lengths)
    announce("mx_quantize kernel layout", lengths)
    c2, s2 = cfa.mx_quantize(to_dev(xb), torch.from_numpy(cu).to(DEV), 2, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    rc, rs = mx.quantize_t(W.bf16_bits_to_f64(xb), cu)
    tp = rc.shape[2]
    c2 = c2.cpu().numpy()[:, :, :tp].reshape(h, d, tp // 32, 8, 4)
    logical = np.empty_like(c2)
    logical[:, :, :, PIECES] = c2
    assert np.array_equal(logical.reshape(h, d, tp), rc)
    assert np.array_equal(np.transpose(s2.cpu().numpy()[:, :tp // 32], (0, 2, 1)), rs)
