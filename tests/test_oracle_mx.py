"""Pins for the reference MX quantiser (E4M3 elements, E8M0 scales, blocks of 32).

The pins come from the formats' definitions: known code values, an exhaustive independent
integer-only formulation over every bf16 bit pattern, round-trips, midpoints, saturation,
power-of-two block maxima, special blocks and the document-local token blocking.
"""

import numpy as np
import pytest

from oracle import mx


def _bf16_to_f64(bits):
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_known_e4m3_values():
    # facts of the E4M3 format: bias 7, 3 mantissa bits, max 448, min subnormal 2^-9
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x78: 256.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        assert mx.e4m3_decode(c) == v
    assert np.isnan(mx.e4m3_decode(0x7F)) and np.isnan(mx.e4m3_decode(0xFF))
    assert np.signbit(mx.e4m3_decode(0x80))
    assert mx.e8m0_decode(127) == 1.0 and mx.e8m0_decode(0) == 2.0 ** -127 and mx.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(mx.e8m0_decode(255))


def test_decode_is_monotone_and_encode_round_trips():
    codes = np.arange(256)
    vals = mx.e4m3_decode(codes)
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # strictly increasing positive codes
    finite = ~np.isnan(vals)
    enc = mx._e4m3_encode_scaled(vals[finite])
    assert np.array_equal(enc, codes[finite])


def test_midpoints_round_to_even_code():
    vals = mx.e4m3_decode(np.arange(0x7F))
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert mx._e4m3_encode_scaled(np.array([mid]))[0] == want
        assert mx._e4m3_encode_scaled(np.array([-mid]))[0] == want | 0x80
        # just above / below the midpoint
        assert mx._e4m3_encode_scaled(np.array([np.nextafter(mid, np.inf)]))[0] == c + 1
        assert mx._e4m3_encode_scaled(np.array([np.nextafter(mid, -np.inf)]))[0] == c


def _independent_one_element(bits):
    """Integer-only formulation of a one-element block of bf16 bits -> (code, scale byte).

    Written from the format definitions, separately from the oracle: the block scale makes
    the element's binary exponent 8 (values in [256, 512), E4M3 step 32) unless the shared
    exponent clamps at -127, which happens for bf16 exponent fields 0..7.
    """
    s = (bits >> 15) & 1
    E8 = (bits >> 7) & 0xFF
    m7 = bits & 0x7F
    if E8 == 0xFF:
        return 0x7F, 0xFF
    if E8 == 0 and m7 == 0:
        return s << 7, 0

    def rne_div(num, shift):  # round num / 2^shift to nearest, ties to even
        if shift <= 0:
            return num << -shift
        q, r = num >> shift, num & ((1 << shift) - 1)
        half = 1 << (shift - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
        return q

    if E8 >= 8:
        # y = 2·M with M = 128 + m7, saturate above 448, then step 32
        M = 128 + m7
        y = 2 * M
        if y > 448:
            return (s << 7) | 0x7E, E8 - 135 + 127
        q = rne_div(M, 4)                  # y/32 = M/16, in [8, 14]
        return (s << 7) | (15 << 3) | (q - 8), E8 - 135 + 127
    if E8 >= 1:
        # shared exponent clamped to -127: y = M·2^(E8-7), binary exponent E8
        M = 128 + m7
        q = rne_div(M, 4)
        e = E8
        if q == 16:
            q, e = 8, e + 1
        return (s << 7) | ((e + 7) << 3) | (q - 8), 0
    # bf16 subnormal: y = m7·2^-6
    p = m7.bit_length() - 1               # floor(log2 m7), 0..6
    q = rne_div(m7, p - 3)
    e = p - 6
    if q == 16:
        q, e = 8, e + 1
    return (s << 7) | ((e + 7) << 3) | (q - 8), 0


def test_every_bf16_pattern_as_one_element_block():
    bits = np.arange(65536, dtype=np.uint32)
    x = _bf16_to_f64(bits)
    codes, scales = mx.quantize_blocks(x[:, None])
    for b in range(65536):
        c, sb = _independent_one_element(b)
        assert codes[b, 0] == c and scales[b] == sb, (hex(b), codes[b, 0], scales[b], c, sb)


def test_block_scale_rule_and_saturation():
    rng = np.random.default_rng(0)
    for k in range(-20, 20):
        blk = rng.uniform(-1, 1, 32) * 2.0 ** k
        blk[5] = 2.0 ** k                  # amax exactly a power of two
        c, s = mx.quantize_blocks(blk[None, :])
        assert s[0] == k - 8 + 127 and c[0, 5] == 0x78
        blk[5] = 448 * 2.0 ** k            # amax = 448·2^k: element lands exactly on 448
        c, s = mx.quantize_blocks(blk[None, :])
        assert s[0] == k + 127 and c[0, 5] == 0x7E
        blk[5] = 300 * 2.0 ** k            # y = 300: nearest E4M3 values 288 and 320 -> 288
        c, s = mx.quantize_blocks(blk[None, :])
        assert s[0] == k + 127 and mx.e4m3_decode(c[0, 5]) == 288.0
        blk[5] = 479 * 2.0 ** k            # 479 has floor(log2) = 8: y = 479 > 448 saturates
        c, s = mx.quantize_blocks(blk[None, :])
        assert s[0] == k + 127 and c[0, 5] == 0x7E
        blk[5] = -479 * 2.0 ** k
        c, s = mx.quantize_blocks(blk[None, :])
        assert c[0, 5] == 0xFE


def test_special_blocks():
    c, s = mx.quantize_blocks(np.zeros((1, 32)))
    assert s[0] == 0 and np.all(c == 0)
    z = np.zeros((1, 32)); z[0, 3] = -0.0
    c, s = mx.quantize_blocks(z)
    assert c[0, 3] == 0x80 and s[0] == 0
    for bad in (np.nan, np.inf, -np.inf):
        b = np.ones((1, 32)); b[0, 7] = bad
        c, s = mx.quantize_blocks(b)
        assert s[0] == 0xFF and np.all(c == 0x7F)
    # a negative value too small for the block rounds to negative zero
    b = np.zeros((1, 32)); b[0, 0] = 1.0; b[0, 1] = -1e-9
    c, s = mx.quantize_blocks(b)
    assert c[0, 1] == 0x80


def test_dequantised_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 3, 128))
    codes, scales = mx.quantize_d(x)
    xd = mx.dequantize_d(codes, scales)
    amax = np.abs(x.reshape(64, 3, 4, 32)).max(axis=-1)
    e = np.floor(np.log2(amax)) - 8
    err = np.abs(xd - x).reshape(64, 3, 4, 32)
    # below 448·2^e: half an E4M3 ulp (relative 2^-4) or half the subnormal step; above: clipped
    big = np.abs(x).reshape(64, 3, 4, 32) > 448 * 2.0 ** e[..., None]
    bound = np.maximum(np.abs(x).reshape(64, 3, 4, 32) * 2.0 ** -4, 2.0 ** -10 * 2.0 ** e[..., None])
    assert np.all(err[~big] <= bound[~big] * (1 + 1e-12))
    assert np.all(np.abs(xd.reshape(64, 3, 4, 32)[big]) == (448 * 2.0 ** e[..., None] * np.ones_like(err))[big])


def test_token_blocks_are_document_local_and_padded():
    rng = np.random.default_rng(2)
    lengths = [5, 32, 33, 0, 70]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = cu[-1]
    x = rng.standard_normal((T, 2, 64))
    codes, scales = mx.quantize_t(x, cu)
    P = mx.padded_offsets(cu)
    assert list(P) == [0, 32, 64, 128, 128, 224]
    assert codes.shape == (2, 64, 224) and scales.shape == (2, 64, 7)
    for n in range(len(lengths)):
        s0, s1, p0 = cu[n], cu[n + 1], P[n]
        L = s1 - s0
        # each document alone gives the same bytes (isolation of token blocks)
        c1, s1b = mx.quantize_t(x[s0:s1], np.array([0, L]))
        assert np.array_equal(codes[:, :, p0:p0 + c1.shape[2]], c1)
        assert np.array_equal(scales[:, :, p0 // 32:p0 // 32 + s1b.shape[2]], s1b)
        # padding columns are zero
        assert np.all(codes[:, :, p0 + L:P[n + 1]] == 0)
        # the block values equal a direct one-block quantisation along tokens
        for b0 in range(0, L, 32):
            blk = x[s0 + b0:min(s1, s0 + b0 + 32)].transpose(1, 2, 0)
            cb, sb = mx.quantize_blocks(blk)
            assert np.array_equal(codes[:, :, p0 + b0:p0 + b0 + blk.shape[2]], cb)
            assert np.array_equal(scales[:, :, (p0 + b0) // 32], sb)
    back = mx.dequantize_t(codes, scales, cu)
    assert np.max(np.abs(back - x)) <= 0.125 * np.max(np.abs(x))  # clipping of the block max is at most 1/8


def test_d_blocks_follow_channels():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 2, 128))
    x[1, 1, 64:96] *= 1000.0
    codes, scales = mx.quantize_d(x)
    for t in range(3):
        for h in range(2):
            for c in range(4):
                cb, sb = mx.quantize_blocks(x[t, h, 32 * c:32 * c + 32][None, :])
                assert np.array_equal(codes[t, h, 32 * c:32 * c + 32], cb[0]) and scales[t, h, c] == sb[0]
    assert scales[1, 1, 2] > scales[1, 1, 1] + 8
