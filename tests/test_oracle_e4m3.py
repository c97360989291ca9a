"""Pins of the oracle's OCP E4M3 codec.

The decode table is checked against values fixed by the format (largest
finite 448, smallest normal 2**-6, smallest subnormal 2**-9, NaN codes); the
encoder is checked against a brute-force nearest-value search over the 254
finite codes, with ties going to the even mantissa, over every fp16 value and
a million random fp32 values.
"""

import numpy as np

import oracle


def test_decode_table_fixed_points():
    t = oracle.e4m3_decode_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x40] == 2.0 and t[0x3C] == 1.5
    assert t[0x77] == 240.0              # 1.875 * 2**7


def test_decode_table_structure():
    t = oracle.e4m3_decode_table()
    pos = t[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)          # strictly increasing 0x00..0x7E
    assert np.array_equal(t[0x80:0xFF], -pos)  # sign-magnitude
    assert np.count_nonzero(np.isfinite(t)) == 254


def _brute_force(y):
    t = oracle.e4m3_decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], np.int64)
    vals = t[codes]
    y = np.asarray(y, np.float64)
    d = np.abs(y[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among ties prefer the even mantissa, then the code whose sign matches y
    even = (codes & 1) == 0
    same_sign = ((codes & 0x80) != 0)[None, :] == np.signbit(y)[:, None]
    score = cand * (1 + 2 * even[None, :] + 4 * same_sign)
    out = codes[np.argmax(score, axis=1)]
    # zero results keep the sign of y
    zero = vals[np.argmax(score, axis=1)] == 0
    out = np.where(zero, np.where(np.signbit(y), 0x80, 0x00), out)
    return out.astype(np.uint8)


def test_encoder_matches_brute_force_on_all_fp16():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float32)
    y = np.clip(h, -448, 448).astype(np.float32)
    got = oracle.e4m3_encode(y)
    want = _brute_force(y)
    assert np.array_equal(got, want)


def test_encoder_matches_brute_force_random_fp32():
    rng = np.random.default_rng(7)
    y = np.concatenate([
        rng.uniform(-448, 448, 400_000),
        rng.uniform(-1, 1, 300_000),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 300_000),
    ]).astype(np.float32)
    for chunk in np.array_split(y, 20):
        assert np.array_equal(oracle.e4m3_encode(chunk), _brute_force(chunk))


def test_encoder_ties_and_signed_zero():
    # 1 + 1/16 lies halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1).
    y = np.array([1.0625, 1.1875, 2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -10,
                  -0.0, 0.0, 448.0, 464.0 - 1e-3], np.float32)
    y = np.clip(y, -448, 448)
    c = oracle.e4m3_encode(y)
    assert c.tolist() == [0x38, 0x3A, 0x00, 0x80, 0x02, 0x80, 0x00, 0x7E, 0x7E]


def test_relative_round_trip_bound():
    rng = np.random.default_rng(8)
    y = rng.uniform(-448, 448, 200_000).astype(np.float32)
    v = oracle.e4m3_decode_table()[oracle.e4m3_encode(y)]
    a = np.abs(y.astype(np.float64))
    normal = a >= 2.0 ** -6
    e = np.floor(np.log2(np.where(normal, a, 1.0)))
    bound = np.where(normal, 2.0 ** (e - 4), 2.0 ** -10)
    assert np.all(np.abs(v - y) <= bound)


def test_quantize_e4m3_lossless_and_saturating():
    t = oracle.e4m3_decode_table()
    finite = np.array([c for c in range(256) if np.isfinite(t[c])])
    x = t[finite].astype(np.float32)          # every value, amax 448
    s = oracle.absmax_scale(x, oracle.E4M3_MAX)
    assert s == np.float32(1.0)
    c = oracle.quantize_e4m3(x, s)
    assert np.array_equal(t[c], x.astype(np.float64))
    # static scale: out-of-range values saturate to +-448, never NaN
    c2 = oracle.quantize_e4m3(np.array([1000.0, -1e6, 500.0], np.float32), np.float32(1.0))
    assert c2.tolist() == [0x7E, 0xFE, 0x7E]
    # zero scale gives +0 codes
    assert oracle.quantize_e4m3(np.zeros(4, np.float32), np.float32(0)).tolist() == [0] * 4


def test_dequantize_fp8_branches():
    """oracle.dequantize reads E4M3 / E5M2 codes through the format's own
    values times the scale (fp64): fixed points of each format, per-row
    scales broadcast, and a quantize / dequantize round trip within half a
    unit in the last place of the format (E4M3 3 mantissa bits, E5M2 2)."""
    codes = np.array([[0x38, 0x7E, 0x01, 0x80], [0xB8, 0xFE, 0x08, 0x00]], np.uint8)
    s = np.array([[2.0], [0.5]])
    got = oracle.dequantize(codes, s, "fp8")
    want = np.array([[2.0, 896.0, 2.0 ** -8, 0.0], [-0.5, -224.0, 2.0 ** -7, 0.0]])
    assert np.array_equal(got, want) and np.signbit(got[0, 3])
    codes5 = np.array([[0x3C, 0x7B, 0x01, 0xBC]], np.uint8)
    got5 = oracle.dequantize(codes5, np.array([[4.0]]), "fp8e5m2")
    assert np.array_equal(got5, [[4.0, 4 * 57344.0, 4 * 2.0 ** -16, -4.0]])
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 128)).astype(np.float16)
    for dtype, mant in (("fp8", 3), ("fp8e5m2", 2)):
        q, sc = oracle.quantize_per_token(x, dtype)
        xh = oracle.dequantize(q, sc[:, None], dtype)
        xs = x.astype(np.float64) / sc[:, None].astype(np.float64)
        # normal range: relative half-ulp; near zero: half the smallest step;
        # plus the fp32 rounding of the quotient (relative 2^-24)
        tiny = 2.0 ** (-9 if dtype == "fp8" else -16)
        bound = np.maximum(np.abs(xs) * 2.0 ** -(mant + 1), tiny / 2) * sc[:, None]
        bound += np.abs(x.astype(np.float64)) * 2.0 ** -23
        assert np.all(np.abs(xh - x.astype(np.float64)) <= bound)
