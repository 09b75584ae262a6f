"""Pins for the 6-bit (MXFP6: E2M3 and E3M2) quantisers, their storage packing and the
MXFP6/FP8 attention oracles.

* Format facts of E2M3 (1 sign, 2 exponent bits with bias 1, 3 mantissa bits): the 32
  magnitudes form a grid of step 1/8 on [0, 2), 1/4 on [2, 4) and 1/2 on [4, 7.5]. E3M2 (1
  sign, 3 exponent bits with bias 3, 2 mantissa bits): step 1/16 on [0, 0.5), then four values
  per binade [2^k, 2^(k+1)) up to 28.
* Rounding: every representable value round-trips; midpoints go to the even code; just above
  or below a midpoint goes to the nearer code; saturation at ±7.5.
* Block rule checked against an independent exhaustive formulation (nearest grid point).
* Packing checked against a big-integer construction of the 192-bit blocks.
* Attention: on inputs exact in E2M3, E2M1 and E4M3 the MXFP6/FP8 oracle equals the MXFP8 and
  MXFP4/FP8 oracles; on general inputs it differs and causality stays bit-exact.
"""
import numpy as np

from oracle import attention as att
from oracle import mx
from oracle import mx_attention as mxa


def _grid():
    return np.concatenate([np.arange(16) / 8.0, 2.0 + np.arange(8) / 4.0, 4.0 + np.arange(8) / 2.0])


def test_e2m3_values():
    want = _grid()
    assert want[-1] == 7.5 and len(want) == 32
    np.testing.assert_array_equal(mx.e2m3_decode(np.arange(32)), want)
    np.testing.assert_array_equal(mx.e2m3_decode(np.arange(32) | 32), -want)
    assert np.signbit(mx.e2m3_decode(32))


def test_round_trip_midpoints_saturation():
    vals = _grid()
    assert np.array_equal(mx._e2m3_encode_scaled(vals), np.arange(32))
    assert np.array_equal(mx._e2m3_encode_scaled(-vals[1:]), np.arange(1, 32) | 32)
    for c in range(31):
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert mx._e2m3_encode_scaled(np.array([mid]))[0] == want, c
        assert mx._e2m3_encode_scaled(np.array([np.nextafter(mid, 10)]))[0] == c + 1
        assert mx._e2m3_encode_scaled(np.array([np.nextafter(mid, -10)]))[0] == c
    codes, sc = mx.quantize_blocks_fp6(np.array([[7.0, 100.0, 127.0] + [0.0] * 29]))
    assert sc[0] == 127 + 4                                          # 2^6 <= 127 < 2^7: e = 6 - 2
    assert mx.e2m3_decode(codes[0, 1]) == 6.0                        # 100/16 = 6.25: tie -> even (6.0)
    assert mx.e2m3_decode(codes[0, 2]) == 7.5                        # 127/16 = 7.94 saturates
    assert mx.e2m3_decode(codes[0, 0]) == 0.5                        # 7/16 = 0.4375: tie -> even (0.5)


def _independent_block(x, grid=None, emax=2):
    amax = max(abs(float(v)) for v in x)
    if amax == 0:
        return [0] * len(x), 0
    e = int(np.floor(np.log2(amax))) - emax
    e = max(-127, min(127, e))
    mags = list(_grid() if grid is None else grid)
    codes = []
    for v in x:
        y = min(abs(float(v)) / 2.0 ** e, mags[-1])
        dist = [abs(y - m) for m in mags]
        best = min(range(32), key=lambda i: (dist[i], i % 2))
        codes.append(best | (32 if np.signbit(v) else 0))
    return codes, e + 127


def test_block_rule_against_exhaustive_formulation():
    rng = np.random.default_rng(5)
    for trial in range(300):
        scale = 2.0 ** rng.integers(-20, 20)
        x = rng.standard_normal(32) * scale
        if trial % 3 == 0:
            x = np.round(x / scale * 16) / 16 * scale       # many exact midpoints
        c, s = mx.quantize_blocks_fp6(x[None, :])
        wc, ws = _independent_block(x)
        assert s[0] == ws and list(c[0]) == wc, trial
    c, s = mx.quantize_blocks_fp6(np.zeros((1, 32)))
    assert s[0] == 0 and not np.any(c)
    c, s = mx.quantize_blocks_fp6(np.array([[np.inf] + [1.0] * 31]))
    assert s[0] == 0xFF and not np.any(c)


def test_pack_fp6_against_big_integers():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 64, size=(3, 2, 128))
    packed = mx.pack_fp6(codes)
    assert packed.shape == (3, 2, 96)
    for t in range(3):
        for h in range(2):
            for b in range(4):
                n = sum(int(codes[t, h, 32 * b + i]) << (6 * i) for i in range(32))
                by = n.to_bytes(24, "little")
                assert bytes(packed[t, h, 16 * b:16 * b + 16]) == by[:16]
                assert bytes(packed[t, h, 64 + 8 * b:64 + 8 * b + 8]) == by[16:]
    one = np.zeros((1, 32), np.int64)
    one[0, 1] = 1                                         # bit 6 of byte 0
    one[0, 21] = 3                                        # bits 126, 127: top bits of byte 15
    one[0, 22] = 5                                        # bits 132, 134: byte 16 -> the 8-byte part
    p = mx.pack_fp6(one)[0]
    assert p[0] == 0x40 and p[15] == 0xC0 and p[16] == 0x50 and not np.any(p[[1, 2, 14, 17]])


def _exact_case(lengths, hq, hkv, d, seed):
    """Values in {0, ±1, ±2, ±3, ±4, ±6} with a ±4 or ±6 in every block of 32 channels: exact in
    E2M3 and E2M1 with scale 2^0 and in E4M3 (along tokens too)."""
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    pool = np.array([0, 1, 2, 3, 4, 6, -1, -2, -3, -4, -6], dtype=np.float64)

    def mk(h):
        x = rng.choice(pool, size=(T, h, d))
        x[:, :, ::32] = rng.choice([4.0, -4.0, 6.0, -6.0], size=(T, h, d // 32))
        return x
    return mk(hq), mk(hkv), mk(hkv), mk(hq), cu


def test_fp6_oracle_reduces_on_exact_inputs():
    q, k, v, do, cu = _exact_case([130, 7, 70], 2, 1, 64, seed=8)
    for x in (q, k):
        c, s = mx.quantize_d_fp6(x)
        assert np.array_equal(mx.dequantize_d_fp6(c, s), x)
    sc = 2.0 ** -9
    o6, l6 = mxa.attn_mx_fwd(q, k, v, cu, sc, qk="e2m3")
    o4, l4 = mxa.attn_mx_fwd(q, k, v, cu, sc, qk="e2m1")
    o8, l8 = mxa.attn_mx_fwd(q, k, v, cu, sc)
    np.testing.assert_array_equal(o6, o8)
    np.testing.assert_array_equal(l6, l8)
    np.testing.assert_array_equal(o6, o4)
    g6 = mxa.attn_mx_bwd(q, k, v, do, cu, sc, qk="e2m3")
    g8 = mxa.attn_mx_bwd(q, k, v, do, cu, sc)
    for a, b in zip(g6, g8):
        np.testing.assert_array_equal(a, b)


def test_fp6_oracle_between_fp4_and_fp8_and_keeps_causality():
    rng = np.random.default_rng(9)
    cu = np.array([0, 200])
    mk = lambda h: np.round(rng.standard_normal((200, h, 64)) * 128) / 128
    q, k, v, do = mk(2), mk(1), mk(1), mk(2)
    o6, _ = mxa.attn_mx_fwd(q, k, v, cu, 0.125, qk="e2m3")
    o4, _ = mxa.attn_mx_fwd(q, k, v, cu, 0.125, qk="e2m1")
    o8, _ = mxa.attn_mx_fwd(q, k, v, cu, 0.125)
    o0, _ = att.attn_fwd(q, k, v, cu, 0.125)
    assert not np.array_equal(o6, o8) and not np.array_equal(o6, o4)
    # 3 mantissa bits like E4M3 but a narrower block range: closer to MXFP8 than E2M1 is
    e6, e4 = np.linalg.norm(o6 - o8), np.linalg.norm(o4 - o8)
    assert e6 < 0.5 * e4, (e6, e4)
    assert np.linalg.norm(o6 - o0) < np.linalg.norm(o4 - o0)
    dq, _, _ = mxa.attn_mx_bwd(q, k, v, do, cu, 0.125, qk="e2m3")
    for j in (0, 31, 32, 128, 150):
        q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
        for a in (q2, k2, v2, do2):
            a[j] = a[j] * 7.5 + 30.0
        o5, _ = mxa.attn_mx_fwd(q2, k2, v2, cu, 0.125, qk="e2m3")
        dq2, _, _ = mxa.attn_mx_bwd(q2, k2, v2, do2, cu, 0.125, qk="e2m3")
        assert np.array_equal(o5[:j], o6[:j]) and np.array_equal(dq2[:j], dq[:j]), j


# ------------------------------------------------------------------------------- E3M2
def _grid_e3m2():
    sub = np.arange(4) / 16.0
    normal = [2.0 ** k * (1 + m / 4) for k in range(-2, 5) for m in range(4)]
    return np.concatenate([sub, normal])


def test_e3m2_values():
    want = _grid_e3m2()
    assert want[-1] == 28.0 and len(want) == 32 and np.all(np.diff(want) > 0)
    np.testing.assert_array_equal(mx.e3m2_decode(np.arange(32)), want)
    np.testing.assert_array_equal(mx.e3m2_decode(np.arange(32) | 32), -want)
    # bit fields: code 0b0_111_11 is the largest value, 0b0_001_00 the smallest normal
    assert mx.e3m2_decode(0b011111) == 28.0 and mx.e3m2_decode(0b000100) == 0.25


def test_e3m2_round_trip_midpoints_saturation():
    vals = _grid_e3m2()
    enc = mx._e3m2_encode_scaled
    assert np.array_equal(enc(vals), np.arange(32))
    assert np.array_equal(enc(-vals[1:]), np.arange(1, 32) | 32)
    for c in range(31):
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert enc(np.array([mid]))[0] == want, c
        assert enc(np.array([np.nextafter(mid, 100)]))[0] == c + 1
        assert enc(np.array([np.nextafter(mid, -100)]))[0] == c
    # amax 31 -> e = 4 - 4 = 0: 18 is halfway 16 (even code) / 20, 22 halfway 20 / 24 (even)
    codes, sc = mx.quantize_blocks_fp6(np.array([[31.0, 18.0, 22.0, 0.09375, -17.0] + [0.0] * 27]), "e3m2")
    assert sc[0] == 127
    assert list(mx.e3m2_decode(codes[0, :5])) == [28.0, 16.0, 24.0, 0.125, -16.0]
    # amax 1000 -> e = 9 - 4 = 5: 1000/32 saturates, 100/32 = 3.125 -> 3, 27/32 -> 0.875
    codes, sc = mx.quantize_blocks_fp6(np.array([[1000.0, 100.0, 27.0] + [0.0] * 29]), "e3m2")
    assert sc[0] == 127 + 5
    assert list(mx.e3m2_decode(codes[0, :3])) == [28.0, 3.0, 0.875]


def test_e3m2_block_rule_against_exhaustive_formulation():
    rng = np.random.default_rng(15)
    grid = _grid_e3m2()
    for trial in range(300):
        scale = 2.0 ** rng.integers(-20, 20)
        x = rng.standard_normal(32) * scale
        if trial % 3 == 0:
            x = np.round(x / scale * 32) / 32 * scale       # many exact midpoints
        if trial % 5 == 0:
            x[rng.integers(32)] *= 40                       # wide blocks: small values go subnormal
        c, s = mx.quantize_blocks_fp6(x[None, :], "e3m2")
        wc, ws = _independent_block(x, grid, emax=4)
        assert s[0] == ws and list(c[0]) == wc, trial
    c, s = mx.quantize_blocks_fp6(np.zeros((1, 32)), "e3m2")
    assert s[0] == 0 and not np.any(c)
    c, s = mx.quantize_blocks_fp6(np.array([[np.nan] + [1.0] * 31]), "e3m2")
    assert s[0] == 0xFF and not np.any(c)


def test_e3m2_oracle_reduces_on_exact_inputs():
    # amax 4 or 6 -> e = -2: the values times 4 are 0, 4, 8, 12, 16, 24, all E3M2 values
    q, k, v, do, cu = _exact_case([130, 7, 70], 2, 1, 64, seed=18)
    for x in (q, k):
        c, s = mx.quantize_d_fp6(x, "e3m2")
        assert np.array_equal(mx.dequantize_d_fp6(c, s, "e3m2"), x)
    sc = 2.0 ** -9
    o3, l3 = mxa.attn_mx_fwd(q, k, v, cu, sc, qk="e3m2")
    o8, l8 = mxa.attn_mx_fwd(q, k, v, cu, sc)
    np.testing.assert_array_equal(o3, o8)
    np.testing.assert_array_equal(l3, l8)
    for a, b in zip(mxa.attn_mx_bwd(q, k, v, do, cu, sc, qk="e3m2"), mxa.attn_mx_bwd(q, k, v, do, cu, sc)):
        np.testing.assert_array_equal(a, b)


def test_e3m2_oracle_accuracy_order_and_causality():
    rng = np.random.default_rng(19)
    cu = np.array([0, 200])
    mk = lambda h: np.round(rng.standard_normal((200, h, 64)) * 128) / 128
    q, k, v, do = mk(2), mk(1), mk(1), mk(2)
    o = {f: mxa.attn_mx_fwd(q, k, v, cu, 0.125, qk=f)[0] for f in ("e4m3", "e2m3", "e3m2", "e2m1")}
    err = {f: np.linalg.norm(o[f] - o["e4m3"]) for f in o}
    # two mantissa bits: between E2M3 (three) and E2M1 (one)
    assert err["e2m3"] < err["e3m2"] < err["e2m1"], err
    dq, _, _ = mxa.attn_mx_bwd(q, k, v, do, cu, 0.125, qk="e3m2")
    for j in (0, 31, 32, 128, 150):
        q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
        for a in (q2, k2, v2, do2):
            a[j] = a[j] * 7.5 + 30.0
        o5, _ = mxa.attn_mx_fwd(q2, k2, v2, cu, 0.125, qk="e3m2")
        dq2, _, _ = mxa.attn_mx_bwd(q2, k2, v2, do2, cu, 0.125, qk="e3m2")
        assert np.array_equal(o5[:j], o["e3m2"][:j]) and np.array_equal(dq2[:j], dq[:j]), j
