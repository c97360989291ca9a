"""Pins of the oracle's OCP E5M2 codec and of its static-scale calibration.

E5M2: the decode table against the format's fixed points, against the
fact that an E5M2 byte is the upper byte of the fp16 with the same bits,
and against torch's float8_e5m2 type; the encoder against torch's
round-to-nearest-even cast and a brute-force nearest-value search.

Calibration: closed forms (a planted maximum), the invariant that the
largest element maps exactly onto the top of the code range, the
granularities' consistency, accumulation over batches equal to one batch
of all tokens, and brute force over a tiny input.
"""

import numpy as np
import pytest
import torch

import oracle


def test_e5m2_decode_fixed_points():
    t = oracle.e5m2_decode_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x7B] == 57344.0 and t[0xFB] == -57344.0          # largest finite
    assert t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert t[0x04] == 2.0 ** -14                                 # smallest normal
    assert t[0x01] == 2.0 ** -16 and t[0x03] == 3 * 2.0 ** -16   # subnormals
    assert t[0x3C] == 1.0 and t[0x3E] == 1.5 and t[0x40] == 2.0


def test_e5m2_is_the_upper_byte_of_fp16():
    t = oracle.e5m2_decode_table()
    f16 = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    same = (t == f16) | (np.isnan(t) & np.isnan(f16))
    assert same.all()


def test_e5m2_decode_matches_torch():
    t = oracle.e5m2_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    assert ((t == ref) | (np.isnan(t) & np.isnan(ref))).all()


def _torch_e5m2(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e5m2).view(
        torch.uint8).numpy()


def test_e5m2_encode_matches_torch_on_random_and_fp16_values():
    g = np.random.default_rng(0)
    y = np.concatenate([
        g.standard_normal(200000) * 1000.0,
        g.standard_normal(100000) * 1e-4,
        g.uniform(-57344, 57344, 100000),
        [0.0, -0.0, 57344.0, -57344.0, 2.0 ** -16, 2.0 ** -17, 3 * 2.0 ** -17],
    ]).astype(np.float32)
    y = np.clip(y, -57344, 57344).astype(np.float32)
    assert np.array_equal(oracle.e5m2_encode(y), _torch_e5m2(y))
    h = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) <= 57344)]
    assert np.array_equal(oracle.e5m2_encode(h), _torch_e5m2(h))


def test_e5m2_encode_is_nearest_with_ties_to_even():
    t = oracle.e5m2_decode_table()
    finite = [c for c in range(256) if np.isfinite(t[c])]
    vals = np.array([t[c] for c in finite])
    g = np.random.default_rng(1)
    y = np.concatenate([g.standard_normal(3000) * 100, (vals[:-1] + vals[1:]) / 2]).astype(
        np.float32)
    y = np.clip(y[np.isfinite(y)], -57344, 57344).astype(np.float32)
    codes = oracle.e5m2_encode(y)
    for yi, ci in zip(y, codes):
        d = np.abs(vals - float(yi))
        best = d.min()
        assert abs(t[ci] - float(yi)) == best
        near = [finite[i] for i in np.nonzero(d == best)[0]]
        if len(near) > 1 and float(yi) != 0.0:          # a tie: even mantissa
            assert ci & 1 == 0


def test_quantize_e5m2_saturates_and_zero_scale():
    x = np.array([1e9, -1e9, 3.0, 0.0], np.float32)
    c = oracle.quantize_e5m2(x, np.float32(1.0))
    assert c[0] == 0x7B and c[1] == 0xFB
    assert np.all(oracle.quantize_e5m2(x, np.float32(0.0)) == 0)


# --- static-scale calibration ------------------------------------------------

@pytest.mark.parametrize("dtype,top", [("int8", 127), ("fp8", 0x7E), ("fp8e5m2", 0x7B)])
def test_calibration_maps_the_maximum_onto_the_top_code(dtype, top):
    g = np.random.default_rng(3)
    x = g.standard_normal((50, 4, 128)).astype(np.float16)
    x[17, 2, 5] = np.float16(-40.0)              # the tensor's largest magnitude
    s = oracle.calibrate_scales(x, "tensor", dtype)
    assert s.shape == (1,) and s[0] == np.float32(40.0) / np.float32(oracle.quant_divisor(dtype))
    code = oracle.quantize_static(x, s, "tensor", dtype)[17, 2, 5]
    if dtype == "int8":
        assert int(code.view(np.int8)) == -127
    else:
        assert code == (top | 0x80)


def test_calibration_granularities_are_consistent():
    g = np.random.default_rng(4)
    x = (g.standard_normal((64, 3, 128)) * np.array([1.0, 5.0, 0.2])[None, :, None]).astype(
        np.float16)
    for dtype in ("int8", "fp8", "fp8e5m2"):
        sc = oracle.calibrate_scales(x, "channel", dtype)
        sh = oracle.calibrate_scales(x, "head", dtype)
        st = oracle.calibrate_scales(x, "tensor", dtype)
        assert sc.shape == (3, 128) and sh.shape == (3,) and st.shape == (1,)
        # division by a positive constant is monotone: coarser = max of finer
        assert np.array_equal(sh, sc.max(axis=1)) and st[0] == sh.max()
        # every element quantizes without saturating past the code range
        for gran, s in (("channel", sc), ("head", sh), ("tensor", st)):
            y = np.abs(x.astype(np.float32)) / np.broadcast_to(
                s.reshape((1, 3, 128) if gran == "channel" else
                          ((1, 3, 1) if gran == "head" else (1, 1, 1))), x.shape)
            assert y.max() <= np.float32(oracle.quant_divisor(dtype)) * (1 + 1e-6)


def test_calibration_accumulates_like_one_batch():
    g = np.random.default_rng(5)
    a = g.standard_normal((30, 2, 128)).astype(np.float16)
    b = (g.standard_normal((20, 2, 128)) * 3).astype(np.float16)
    for gran in ("tensor", "head", "channel"):
        s1 = oracle.calibrate_scales(a, gran, "fp8")
        s2 = oracle.calibrate_scales(b, gran, "fp8", previous=s1)
        assert np.array_equal(s2, oracle.calibrate_scales(np.concatenate([a, b]), gran, "fp8"))


def test_calibration_brute_force_tiny():
    x = np.array([[[1.0, -3.0], [0.5, 0.25]],
                  [[-2.0, 2.5], [0.0, -0.75]]], np.float16)     # [T=2, H=2, D=2]
    sc = oracle.calibrate_scales(x, "channel", "int8")
    want = np.array([[2.0, 3.0], [0.5, 0.75]], np.float32) / np.float32(127.0)
    assert np.array_equal(sc, want.astype(np.float32))
    assert np.array_equal(oracle.calibrate_scales(x, "head", "int8"),
                          np.array([3.0, 0.75], np.float32) / np.float32(127.0))
