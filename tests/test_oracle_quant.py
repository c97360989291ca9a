"""Pins of the oracle's symmetric INT8 / INT4 quantization.

Every check is a closed form, a printed rule or a bound fixed by the
mathematics, chosen so that a plausible slip (round-half-away or floor instead
of half-to-even, 128 instead of 127, max instead of max-abs, a multiply by the
scale instead of a divide, a wrong clamp) fails at least one of them.
"""

import numpy as np
import pytest

import oracle


def _vec_with_amax(vals, amax=127.0, n=128):
    x = np.zeros(n, np.float32)
    x[: len(vals)] = vals
    x[-1] = amax
    return x


def test_ties_round_half_to_even():
    # amax 127 -> scale exactly 1.0, so codes are round(x) itself.
    x = _vec_with_amax([2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5])
    s = oracle.absmax_scale(x, oracle.INT8_QMAX)
    assert s == np.float32(1.0)
    q = oracle.quantize_int(x, s, oracle.INT8_QMIN, oracle.INT8_QMAX)
    assert q[:8].tolist() == [2, 4, -2, -4, 0, 0, 2, 126]
    assert q[-1] == 127


def test_amax_element_maps_to_qmax_with_sign():
    rng = np.random.default_rng(1)
    for _ in range(200):
        x = rng.standard_normal(128).astype(np.float16).astype(np.float32)
        i = int(np.argmax(np.abs(x)))
        s = oracle.absmax_scale(x, oracle.INT8_QMAX)
        q = oracle.quantize_int(x, s, oracle.INT8_QMIN, oracle.INT8_QMAX)
        assert q[i] == (127 if x[i] > 0 else -127)
        assert np.all(np.abs(q.astype(int)) <= 127)
        s4 = oracle.absmax_scale(x, oracle.INT4_QMAX)
        q4 = oracle.quantize_int(x, s4, oracle.INT4_QMIN, oracle.INT4_QMAX)
        assert q4[i] == (7 if x[i] > 0 else -7)


def test_negative_amax_uses_absolute_value():
    x = _vec_with_amax([-127.0, 3.0], amax=1.0)
    s = oracle.absmax_scale(x, oracle.INT8_QMAX)
    assert s == np.float32(1.0)
    q = oracle.quantize_int(x, s, oracle.INT8_QMIN, oracle.INT8_QMAX)
    assert q[0] == -127 and q[1] == 3


def test_lossless_integer_inputs():
    rng = np.random.default_rng(2)
    x = rng.integers(-127, 128, 128).astype(np.float32)
    x[5] = 127.0
    s = oracle.absmax_scale(x, oracle.INT8_QMAX)
    q = oracle.quantize_int(x, s, oracle.INT8_QMIN, oracle.INT8_QMAX)
    assert s == np.float32(1.0)
    assert np.array_equal(q.astype(np.float32), x)
    assert np.array_equal(oracle.dequantize(q, s, "int8"), x.astype(np.float64))


def test_clamp_edges_with_static_scale():
    s = np.float32(1.0)
    x = np.array([127.6, -128.4, -128.6, -300.0, 300.0, 127.4], np.float32)
    q = oracle.quantize_int(x, s, oracle.INT8_QMIN, oracle.INT8_QMAX)
    assert q.tolist() == [127, -128, -128, -128, 127, 127]
    q4 = oracle.quantize_int(np.array([7.6, -8.4, -9.0, 6.5, -6.5], np.float32), s,
                             oracle.INT4_QMIN, oracle.INT4_QMAX)
    assert q4.tolist() == [7, -8, -8, 6, -6]


def test_zero_vector_gives_zero_scale_and_codes():
    x = np.zeros(128, np.float32)
    s = oracle.absmax_scale(x, oracle.INT8_QMAX)
    assert s == 0.0
    q = oracle.quantize_int(x, s, oracle.INT8_QMIN, oracle.INT8_QMAX)
    assert not q.any()
    c, ps = oracle.quantize_per_token(np.zeros((3, 2, 128), np.float16), "int8")
    assert not c.any() and not ps.any()


@pytest.mark.parametrize("qmax,qmin", [(127, -128), (7, -8)])
def test_round_trip_bound(qmax, qmin):
    # |x - q*s| <= s/2 plus the fp32 slack of one division (|x/s| <= qmax).
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((500, 128)) * rng.uniform(0.01, 50, (500, 1)))
    x = x.astype(np.float16).astype(np.float32)
    s = oracle.absmax_scale(x, qmax, axis=-1)
    q = oracle.quantize_int(x, s[:, None], qmin, qmax)
    err = np.abs(x.astype(np.float64) - oracle.dequantize(q, s[:, None], "int8"))
    bound = s[:, None].astype(np.float64) * (0.5 + (qmax + 0.5) * 2.0 ** -23)
    assert np.all(err <= bound)


def test_scale_is_one_fp32_division():
    # amax / 127 as a single correctly rounded fp32 division, not a multiply
    # by a rounded reciprocal: these amax values differ between the two.
    amax = np.float32(0.0)
    found = 0
    for bits in range(0x3F800000, 0x3F800000 + 20000):
        a = np.array([bits], np.uint32).view(np.float32)[0]
        div = np.float32(a) / np.float32(127)
        mul = np.float32(a) * (np.float32(1) / np.float32(127))
        if div != mul:
            x = np.zeros(128, np.float32)
            x[0] = a
            assert oracle.absmax_scale(x, 127) == div
            amax = a
            found += 1
            if found > 5:
                break
    assert found > 0 and amax > 0


def test_per_token_is_per_vector():
    # An outlier in one (token, head) vector changes only that vector's scale.
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 2, 128)).astype(np.float16)
    base_c, base_s = oracle.quantize_per_token(x, "int8")
    y = x.copy()
    y[3, 1, 7] = np.float16(100.0)
    c, s = oracle.quantize_per_token(y, "int8")
    changed = np.argwhere(s != base_s)
    assert changed.tolist() == [[3, 1]]
    assert s[3, 1] == np.float32(100.0) / np.float32(127)
    mask = np.ones((8, 2), bool)
    mask[3, 1] = False
    assert np.array_equal(c[mask], base_c[mask])


def test_static_granularities_broadcast():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 3, 128)).astype(np.float16)
    st = np.array([0.05], np.float32)
    sh = np.array([0.01, 0.02, 0.04], np.float32)
    sc = rng.uniform(0.01, 0.05, (3, 128)).astype(np.float32)
    xf = x.astype(np.float32)
    for gran, s, sb in [("tensor", st, st.reshape(1, 1, 1)),
                        ("head", sh, sh.reshape(1, 3, 1)),
                        ("channel", sc, sc.reshape(1, 3, 128))]:
        q = oracle.quantize_static(x, s, gran, "int8")
        # elementwise definition, one element at a time
        for (t, h, c) in [(0, 0, 0), (4, 2, 127), (2, 1, 64)]:
            sv = sb[0 if sb.shape[0] == 1 else t,
                    0 if sb.shape[1] == 1 else h,
                    0 if sb.shape[2] == 1 else c]
            want = int(min(127, max(-128, np.rint(np.float32(xf[t, h, c]) / np.float32(sv)))))
            assert q[t, h, c] == want
