"""Pins for the E2M1 (MXFP4) quantiser and the MXFP4/FP8 attention oracle, on the CPU.

* Format facts of E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit): the 16 values.
* Rounding: every representable value round-trips; midpoints go to the even code; just above
  or below a midpoint goes to the nearer code; saturation at ±6.
* Block rule checked against an independent exhaustive formulation: for each element, the
  scaled value's nearest representable magnitude found by comparing all eight.
* Attention: on inputs exact in both E2M1 and E4M3 the MXFP4/FP8 oracle reduces to the MXFP8
  oracle and to the plain one; on general inputs causality and isolation stay bit-exact.
"""
import numpy as np

from oracle import attention as att
from oracle import mx
from oracle import mx_attention as mxa


def test_e2m1_values():
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        # exponent field (c >> 1) with bias 1; field 0 is subnormal: m · 2^0 · 0.5
        E, m = c >> 1, c & 1
        v = m * 0.5 if E == 0 else (1 + m / 2) * 2.0 ** (E - 1)
        assert v == want[c] == mx.e2m1_decode(c)
        assert mx.e2m1_decode(c | 8) == -want[c]
    assert np.signbit(mx.e2m1_decode(8))


def test_round_trip_midpoints_saturation():
    vals = mx.e2m1_decode(np.arange(8))
    assert np.array_equal(mx._e2m1_encode_scaled(vals), np.arange(8))
    assert np.array_equal(mx._e2m1_encode_scaled(-vals[1:]), np.arange(1, 8) | 8)
    for c in range(7):
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert mx._e2m1_encode_scaled(np.array([mid]))[0] == want, c
        assert mx._e2m1_encode_scaled(np.array([np.nextafter(mid, 10)]))[0] == c + 1
        assert mx._e2m1_encode_scaled(np.array([np.nextafter(mid, -10)]))[0] == c
    codes, sc = mx.quantize_blocks_fp4(np.array([[7.0, 100.0] + [0.0] * 30]))
    assert sc[0] == 127 + 4 and mx.e2m1_decode(codes[0, 1]) == 6.0   # 100 = 6.25·2^4 saturates
    assert mx.e2m1_decode(codes[0, 0]) == 0.5                          # 7 / 16 = 0.4375 -> 0.5


def _independent_block(x):
    """Exhaustive formulation: shared exponent from the largest magnitude's binary exponent,
    then per element the representable magnitude at the smallest distance (even code on a tie)."""
    amax = max(abs(float(v)) for v in x)
    if amax == 0:
        return [0] * len(x), 0
    e = int(np.floor(np.log2(amax))) - 2
    e = max(-127, min(127, e))
    codes = []
    for v in x:
        y = min(abs(float(v)) / 2.0 ** e, 6.0)
        mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
        dist = [abs(y - m) for m in mags]
        best = min(range(8), key=lambda i: (dist[i], i % 2))
        codes.append(best | (8 if np.signbit(v) else 0))
    return codes, e + 127


def test_block_rule_against_exhaustive_formulation():
    rng = np.random.default_rng(5)
    for trial in range(300):
        scale = 2.0 ** rng.integers(-20, 20)
        x = rng.standard_normal(32) * scale
        if trial % 3 == 0:
            x = np.round(x / scale * 4) / 4 * scale       # many exact midpoints
        c, s = mx.quantize_blocks_fp4(x[None, :])
        wc, ws = _independent_block(x)
        assert s[0] == ws and list(c[0]) == wc, trial
    c, s = mx.quantize_blocks_fp4(np.zeros((1, 32)))
    assert s[0] == 0 and not np.any(c)
    c, s = mx.quantize_blocks_fp4(np.array([[np.nan] + [1.0] * 31]))
    assert s[0] == 0xFF
    assert np.array_equal(mx.pack_fp4(np.array([[1, 2, 15, 8]])), np.array([[0x21, 0x8F]]))


def _exact_case(lengths, hq, hkv, d, seed):
    """Values in {0, ±1, ±2, ±3, ±4, ±6} with a ±4 or ±6 in every block of 32 channels: exact in
    E2M1 with scale 2^0 and in E4M3 with scale 2^-5 (and along tokens: integers <= 8)."""
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    pool = np.array([0, 1, 2, 3, 4, 6, -1, -2, -3, -4, -6], dtype=np.float64)

    def mk(h):
        x = rng.choice(pool, size=(T, h, d))
        x[:, :, ::32] = rng.choice([4.0, -4.0, 6.0, -6.0], size=(T, h, d // 32))
        return x
    return mk(hq), mk(hkv), mk(hkv), mk(hq), cu


def test_fp4_oracle_reduces_on_exact_inputs():
    q, k, v, do, cu = _exact_case([130, 7, 70], 2, 1, 64, seed=8)
    for x in (q, k):
        c, s = mx.quantize_d_fp4(x)
        assert np.array_equal(mx.dequantize_d_fp4(c, s), x)
    sc = 2.0 ** -9
    o4, l4 = mxa.attn_mx_fwd(q, k, v, cu, sc, qk="e2m1")
    o8, l8 = mxa.attn_mx_fwd(q, k, v, cu, sc)
    o0, l0 = att.attn_fwd(q, k, v, cu, sc)
    np.testing.assert_array_equal(o4, o8)
    np.testing.assert_array_equal(l4, l8)
    np.testing.assert_allclose(o4, o0, rtol=0, atol=1e-12 * np.abs(o0).max())
    g4 = mxa.attn_mx_bwd(q, k, v, do, cu, sc, qk="e2m1")
    g8 = mxa.attn_mx_bwd(q, k, v, do, cu, sc)
    for a, b in zip(g4, g8):
        np.testing.assert_array_equal(a, b)


def test_fp4_oracle_differs_on_general_inputs_and_keeps_causality():
    rng = np.random.default_rng(9)
    cu = np.array([0, 200])
    mk = lambda h: np.round(rng.standard_normal((200, h, 64)) * 128) / 128
    q, k, v, do = mk(2), mk(1), mk(1), mk(2)
    o4, _ = mxa.attn_mx_fwd(q, k, v, cu, 0.125, qk="e2m1")
    o8, _ = mxa.attn_mx_fwd(q, k, v, cu, 0.125)
    assert not np.array_equal(o4, o8)
    dq, _, _ = mxa.attn_mx_bwd(q, k, v, do, cu, 0.125, qk="e2m1")
    for j in (0, 31, 32, 128, 150):
        q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
        for a in (q2, k2, v2, do2):
            a[j] = a[j] * 7.5 + 30.0
        o5, _ = mxa.attn_mx_fwd(q2, k2, v2, cu, 0.125, qk="e2m1")
        dq2, _, _ = mxa.attn_mx_bwd(q2, k2, v2, do2, cu, 0.125, qk="e2m1")
        assert np.array_equal(o5[:j], o4[:j]) and np.array_equal(dq2[:j], dq[:j]), j
