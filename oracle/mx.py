"""Reference MX (microscaling) quantiser: FP8 E4M3 (or FP4 E2M1, FP6 E2M3) elements with one E8M0 scale per 32.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FLAMIA page ("FLAMIA Mimarisi ve Temel Tasarım İlkeleri") names an MXFP8 attention path
with token-block scaling and document-local scales, but not the bit-level rules. The rules
below are the public definitions of the formats and the plainest MX scale rule:

* E4M3 ("FN" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals kept
  (step 2^-9 below 2^-6); largest finite 448; no infinities; NaN is S.1111.111.
* E8M0 scale byte b: the power of two 2^(b-127); b = 0xFF is NaN.
* Per block of 32 elements: amax = max |x|; shared exponent e = floor(log2 amax) - 8 (8 is the
  exponent of 448, the largest E4M3 power of two), clamped to [-127, 127]; e = -127 for an
  all-zero block; scale byte e + 127. Elements x·2^-e are saturated to ±448 and rounded to the
  nearest E4M3 value, ties to even mantissa; the sign of zero is kept. A block holding a NaN
  or an infinity gets scale byte 0xFF and NaN codes 0x7F.

Two blockings, both document-local when tokens are blocked:

* along d  (``quantize_d``): channels [32c, 32c+32) of one (token, head);
* along tokens (``quantize_t``): doc-local tokens [32b, 32b+32) of one (head, channel), the
  last block of a document holding only its real tokens. Blocks never span two documents.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest power of two not above 448
BLOCK = 32


def e4m3_decode(codes):
    """Value of each E4M3 byte (float64); 0x7F/0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.ldexp(1.0, (E - 7).astype(np.int64))
    val = sign * np.where(E == 0, sub, nrm)
    return np.where((E == 15) & (m == 7), np.nan, val)


def e8m0_decode(scale_bytes):
    """2^(b-127) for each E8M0 byte; 0xFF is NaN."""
    b = np.asarray(scale_bytes, dtype=np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - 127))


def _e4m3_encode_scaled(y):
    """Round already-scaled, finite values y (|y| <= 448) to E4M3 bytes, RNE, sign kept."""
    a = np.abs(y)
    neg = np.signbit(y)
    code = np.zeros(y.shape, dtype=np.int64)
    small = a < 2.0 ** -6
    # subnormal range: integer multiples of 2^-9; rint rounds halves to even.
    # A result of 8 is 2^-6, whose normal code 0x08 equals the integer 8.
    code = np.where(small, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    # normal range: exponent from the binary representation, 3 fraction bits
    _, ex = np.frexp(np.where(small, 1.0, a))      # a = f·2^ex, f in [0.5, 1)
    E = ex - 1                                       # floor(log2 a)
    mant = np.rint(np.ldexp(np.where(small, 1.0, a), 3 - E)).astype(np.int64)  # in [8, 16]
    carry = mant == 16
    E = np.where(carry, E + 1, E)
    mant = np.where(carry, 8, mant)
    ncode = ((E + 7) << 3) | (mant - 8)
    code = np.where(small, code, ncode)
    return code | np.where(neg, 0x80, 0)


def quantize_blocks(x):
    """Quantise rows of 32 (or fewer) values: x is [..., n] with n <= 32, one block per row.

    Returns (codes uint8 [..., n], scale bytes uint8 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.all(np.isfinite(x), axis=-1)
    xs = np.where(np.isfinite(x), x, 0.0)
    amax = np.max(np.abs(xs), axis=-1) if x.shape[-1] else np.zeros(x.shape[:-1])
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex - 1 - E4M3_EMAX, -127, 127)
    e = np.where(amax > 0, e, -127)
    y = np.ldexp(xs, -e[..., None])
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    codes = _e4m3_encode_scaled(y)
    codes = np.where(finite[..., None], codes, 0x7F)
    scales = np.where(finite, e + 127, 0xFF)
    return codes.astype(np.uint8), scales.astype(np.uint8)


def quantize_d(x):
    """Blocks along the head dim: x [T, h, d] (d % 32 == 0) -> codes [T, h, d], scales [T, h, d/32]."""
    x = np.asarray(x, dtype=np.float64)
    T, h, d = x.shape
    assert d % BLOCK == 0
    codes, scales = quantize_blocks(x.reshape(T, h, d // BLOCK, BLOCK))
    return codes.reshape(T, h, d), scales


# ---------------------------------------------------------------- E2M1 (MXFP4) elements
# E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no infinities or NaN; values
# 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6. Same block rule as E4M3 with the format's own top
# exponent: e = floor(log2 amax) - 2 (2 is the exponent of 4, the largest E2M1 power of two),
# elements x·2^-e saturated to ±6 and rounded to the nearest E2M1 value, ties to the even
# mantissa (even code). A block holding a NaN or an infinity gets scale byte 0xFF and codes 0.
E2M1_MAX = 6.0
E2M1_EMAX = 2
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (float64); bit 3 is the sign."""
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def _e2m1_encode_scaled(y):
    """Round already-scaled, finite values y (|y| <= 6) to E2M1 codes, RNE, sign kept."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    # nearest magnitude; on a tie (a midpoint) the even code, whose mantissa bit is 0
    d = np.abs(a[..., None] - E2M1_VALUES)
    best = np.argmin(d, axis=-1)
    dmin = np.take_along_axis(d, best[..., None], axis=-1)[..., 0]
    tie_up = (best + 1 <= 7) & np.isclose(np.abs(a - E2M1_VALUES[np.minimum(best + 1, 7)]), dmin, rtol=0, atol=0)
    best = np.where(tie_up & (best % 2 == 1), best + 1, best)
    return (best | np.where(np.signbit(y), 8, 0)).astype(np.int64)


def quantize_blocks_fp4(x):
    """Quantise rows of 32 values to E2M1 codes (one int per element, 0..15) and E8M0 scale bytes."""
    x = np.asarray(x, dtype=np.float64)
    finite = np.all(np.isfinite(x), axis=-1)
    xs = np.where(np.isfinite(x), x, 0.0)
    amax = np.max(np.abs(xs), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex - 1 - E2M1_EMAX, -127, 127)
    e = np.where(amax > 0, e, -127)
    y = np.clip(np.ldexp(xs, -e[..., None]), -E2M1_MAX, E2M1_MAX)
    codes = np.where(finite[..., None], _e2m1_encode_scaled(y), 0)
    scales = np.where(finite, e + 127, 0xFF)
    return codes.astype(np.uint8), scales.astype(np.uint8)


def quantize_d_fp4(x):
    """Blocks of 32 channels: x [T, h, d] -> E2M1 codes [T, h, d] (0..15), scales [T, h, d/32]."""
    x = np.asarray(x, dtype=np.float64)
    T, h, d = x.shape
    assert d % BLOCK == 0
    codes, scales = quantize_blocks_fp4(x.reshape(T, h, d // BLOCK, BLOCK))
    return codes.reshape(T, h, d), scales


def pack_fp4(codes):
    """Storage layout: two codes per byte, element 2i in the low nibble -> [..., d/2] uint8."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def dequantize_d_fp4(codes, scales):
    """Values of d-blocked E2M1 codes [T, h, d] (unpacked) with scales [T, h, d/32]."""
    T, h, d = codes.shape
    v = e2m1_decode(codes).reshape(T, h, d // BLOCK, BLOCK) * e8m0_decode(scales)[..., None]
    return v.reshape(T, h, d)


# ---------------------------------------------------------------- E2M3 (MXFP6) elements
# E2M3: 1 sign, 2 exponent (bias 1), 3 mantissa bits; no infinities or NaN. Exponent field 0
# is subnormal (m/8); field E >= 1 gives (1 + m/8)·2^(E-1): 0 .. 0.875 and 1 .. 1.875 in steps
# of 1/8, 2 .. 3.75 in steps of 1/4, 4 .. 7.5 in steps of 1/2. Same block rule as the other
# element types with the format's own top exponent: e = floor(log2 amax) - 2 (2 is the
# exponent of 4, the largest E2M3 power of two), elements x·2^-e saturated to ±7.5 and rounded
# to the nearest E2M3 value, ties to the even code. A block holding a NaN or an infinity gets
# scale byte 0xFF and codes 0.
E2M3_MAX = 7.5
E2M3_EMAX = 2


def e2m3_decode(codes):
    """Value of each 6-bit E2M3 code (float64); bit 5 is the sign."""
    c = np.asarray(codes, dtype=np.int64)
    E, m = (c >> 3) & 3, c & 7
    mag = np.where(E == 0, m / 8.0, (1.0 + m / 8.0) * np.ldexp(1.0, E - 1))
    return np.where(c & 32, -mag, mag)


E2M3_VALUES = e2m3_decode(np.arange(32))


def _e2m3_encode_scaled(y):
    """Round already-scaled, finite values y (|y| <= 7.5) to E2M3 codes, RNE, sign kept."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    d = np.abs(a[..., None] - E2M3_VALUES)
    best = np.argmin(d, axis=-1)
    dmin = np.take_along_axis(d, best[..., None], axis=-1)[..., 0]
    nxt = np.minimum(best + 1, 31)
    tie_up = (best + 1 <= 31) & (np.abs(a - E2M3_VALUES[nxt]) == dmin)
    best = np.where(tie_up & (best % 2 == 1), best + 1, best)
    return (best | np.where(np.signbit(y), 32, 0)).astype(np.int64)


# ---------------------------------------------------------------- E3M2 (MXFP6) elements
# E3M2: 1 sign, 3 exponent (bias 3), 2 mantissa bits; no infinities or NaN. Exponent field 0
# is subnormal (m/4 · 2^-2); field E >= 1 gives (1 + m/4)·2^(E-3): 0 .. 0.4375 in steps of 1/16,
# then four values per binade up to 16 .. 28 in steps of 4. Block rule as for E2M3 with the
# top exponent 4 (16 is the largest E3M2 power of two): e = floor(log2 amax) - 4, elements
# x·2^-e saturated to ±28, nearest E3M2 value, ties to the even code.
E3M2_MAX = 28.0
E3M2_EMAX = 4


def e3m2_decode(codes):
    """Value of each 6-bit E3M2 code (float64); bit 5 is the sign."""
    c = np.asarray(codes, dtype=np.int64)
    E, m = (c >> 2) & 7, c & 3
    mag = np.where(E == 0, m / 4.0 * 0.25, (1.0 + m / 4.0) * np.ldexp(1.0, E - 3))
    return np.where(c & 32, -mag, mag)


E3M2_VALUES = e3m2_decode(np.arange(32))


def _e3m2_encode_scaled(y):
    """Round already-scaled, finite values y (|y| <= 28) to E3M2 codes, RNE, sign kept."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    d = np.abs(a[..., None] - E3M2_VALUES)
    best = np.argmin(d, axis=-1)
    dmin = np.take_along_axis(d, best[..., None], axis=-1)[..., 0]
    nxt = np.minimum(best + 1, 31)
    tie_up = (best + 1 <= 31) & (np.abs(a - E3M2_VALUES[nxt]) == dmin)
    best = np.where(tie_up & (best % 2 == 1), best + 1, best)
    return (best | np.where(np.signbit(y), 32, 0)).astype(np.int64)


# the two 6-bit element types: (top exponent, largest value, encoder, decoder)
FP6_FORMATS = {
    "e2m3": (E2M3_EMAX, E2M3_MAX, _e2m3_encode_scaled, e2m3_decode),
    "e3m2": (E3M2_EMAX, E3M2_MAX, _e3m2_encode_scaled, e3m2_decode),
}


def quantize_blocks_fp6(x, fmt="e2m3"):
    """Quantise rows of 32 values to 6-bit codes of ``fmt`` ("e2m3" or "e3m2"; one int per
    element, 0..63) and E8M0 scale bytes."""
    emax, vmax, encode, _ = FP6_FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    finite = np.all(np.isfinite(x), axis=-1)
    xs = np.where(np.isfinite(x), x, 0.0)
    amax = np.max(np.abs(xs), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex - 1 - emax, -127, 127)
    e = np.where(amax > 0, e, -127)
    y = np.clip(np.ldexp(xs, -e[..., None]), -vmax, vmax)
    codes = np.where(finite[..., None], encode(y), 0)
    scales = np.where(finite, e + 127, 0xFF)
    return codes.astype(np.uint8), scales.astype(np.uint8)


def quantize_d_fp6(x, fmt="e2m3"):
    """Blocks of 32 channels: x [T, h, d] -> 6-bit codes [T, h, d] (0..63), scales [T, h, d/32]."""
    x = np.asarray(x, dtype=np.float64)
    T, h, d = x.shape
    assert d % BLOCK == 0
    codes, scales = quantize_blocks_fp6(x.reshape(T, h, d // BLOCK, BLOCK), fmt)
    return codes.reshape(T, h, d), scales


def pack_fp6(codes):
    """Storage layout of 6-bit codes (E2M3 or E3M2) [..., d] (d a multiple of 32) -> [..., 3d/4] uint8.

    Block b (channels 32b .. 32b+31) is the 192-bit little-endian number whose bits 6i .. 6i+5
    hold code i; its bytes 0-15 go to [16b, 16b+16) and bytes 16-23 to [d/2 + 8b, d/2 + 8b + 8)
    of the row (a 16-byte part per block, then an 8-byte part per block).
    """
    c = np.asarray(codes, dtype=np.uint8)
    d = c.shape[-1]
    nb = d // BLOCK
    blocks = c.reshape(c.shape[:-1] + (nb, BLOCK))
    bits = (blocks[..., None] >> np.arange(6, dtype=np.uint8)) & 1          # [..., nb, 32, 6]
    by = np.packbits(bits.reshape(bits.shape[:-2] + (192,)).reshape(bits.shape[:-2] + (24, 8)),
                     axis=-1, bitorder="little")[..., 0]                    # [..., nb, 24]
    return np.concatenate([by[..., :16].reshape(c.shape[:-1] + (16 * nb,)),
                           by[..., 16:].reshape(c.shape[:-1] + (8 * nb,))], axis=-1)


def dequantize_d_fp6(codes, scales, fmt="e2m3"):
    """Values of d-blocked 6-bit codes of ``fmt`` [T, h, d] (unpacked) with scales [T, h, d/32]."""
    T, h, d = codes.shape
    decode = FP6_FORMATS[fmt][3]
    v = decode(codes).reshape(T, h, d // BLOCK, BLOCK) * e8m0_decode(scales)[..., None]
    return v.reshape(T, h, d)


def padded_offsets(cu_seqlens):
    """Start of each document in the token-blocked layout: P_n = Σ_{m<n} 32·ceil(L_m/32).

    Returns an int64 array of n_docs+1 entries; the last one is T_pad.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    L = np.diff(cu)
    return np.concatenate([[0], np.cumsum((L + BLOCK - 1) // BLOCK * BLOCK)])


def quantize_t(x, cu_seqlens):
    """Blocks along doc-local tokens: x [T, h, d] -> codes [h, d, T_pad], scales [h, d, T_pad/32].

    Document n occupies columns [P_n, P_n + 32·ceil(L_n/32)); its block b covers doc-local tokens
    [32b, min(32b+32, L_n)). Columns past the document's end (padding) hold code 0x00.
    """
    x = np.asarray(x, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, h, d = x.shape
    P = padded_offsets(cu)
    Tp = int(P[-1])
    codes = np.zeros((h, d, Tp), dtype=np.uint8)
    scales = np.zeros((h, d, Tp // BLOCK), dtype=np.uint8)
    xt = np.transpose(x, (1, 2, 0))  # [h, d, T]
    for n in range(len(cu) - 1):
        s0, s1, p0 = int(cu[n]), int(cu[n + 1]), int(P[n])
        for b0 in range(0, s1 - s0, BLOCK):
            b1 = min(s1 - s0, b0 + BLOCK)
            c, s = quantize_blocks(xt[:, :, s0 + b0:s0 + b1])
            codes[:, :, p0 + b0:p0 + b1] = c
            scales[:, :, (p0 + b0) // BLOCK] = s
    return codes, scales


def dequantize_d(codes, scales):
    """Values of a d-blocked tensor: codes [T, h, d], scales [T, h, d/32] -> float64 [T, h, d]."""
    T, h, d = codes.shape
    v = e4m3_decode(codes).reshape(T, h, d // BLOCK, BLOCK) * e8m0_decode(scales)[..., None]
    return v.reshape(T, h, d)


def dequantize_t(codes, scales, cu_seqlens):
    """Values of a token-blocked tensor back in packed layout: -> float64 [T, h, d]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    h, d, Tp = codes.shape
    P = padded_offsets(cu)
    full = e4m3_decode(codes) * np.repeat(e8m0_decode(scales), BLOCK, axis=2)
    T = int(cu[-1])
    out = np.zeros((T, h, d), dtype=np.float64)
    for n in range(len(cu) - 1):
        s0, s1, p0 = int(cu[n]), int(cu[n + 1]), int(P[n])
        out[s0:s1] = np.transpose(full[:, :, p0:p0 + (s1 - s0)], (2, 0, 1))
    return out
