"""Pins of the oracle's asymmetric (affine) INT4 groups.

The scale and zero point are checked bit for bit against torch's min/max
observers (an independent library routine with the same zero-containing
range and the same fp32 arithmetic), every code against a brute-force
search over the sixteen levels in exact rational arithmetic, and the
degenerate groups against their closed forms.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch
from torch.ao.quantization import PerChannelMinMaxObserver

import oracle


def _groups(seed, shape, scale=1.0, shift=0.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * scale + shift).astype(np.float16)


def _observer_params(x, axis):
    """torch's per-channel min/max observer on 4-bit unsigned codes; the
    channel axis is the one NOT reduced."""
    t = torch.from_numpy(np.asarray(x, np.float32))
    ch = 1 - axis if t.dim() == 2 else None
    ob = PerChannelMinMaxObserver(ch_axis=ch, dtype=torch.quint8,
                                  qscheme=torch.per_channel_affine, quant_min=0, quant_max=15)
    ob(t)
    s, z = ob.calculate_qparams()
    return s.numpy(), z.numpy().astype(np.int64)


@pytest.mark.parametrize("seed,scale,shift", [(0, 1.0, 0.0), (1, 3.0, 2.0), (2, 0.01, -0.5),
                                              (3, 10.0, 0.0), (4, 1.0, 6.0)])
@pytest.mark.parametrize("axis", [0, 1])
def test_params_match_torch_observer(seed, scale, shift, axis):
    x = _groups(seed, (64, 128), scale, shift)
    s, z = oracle.affine_params(x, oracle.INT4_UMAX, axis=axis)
    ts, tz = _observer_params(x, axis)
    assert np.array_equal(s.view(np.uint32), ts.astype(np.float32).view(np.uint32))
    assert np.array_equal(z, tz)


def _nearest_ok(x, q, s, z):
    """Code q is a nearest level of x among (c - z) * s, c = 0..15, in exact
    arithmetic, unless x / s sits within 2^-18 of a rounding tie (where the
    fp32 quotient may round either way)."""
    xf, sf = Fraction(float(x)), Fraction(float(s))
    dist = [abs(xf - (c - int(z)) * sf) for c in range(16)]
    if dist[int(q)] == min(dist):
        return True
    r = xf / sf
    frac = r - (r.numerator // r.denominator)
    return abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 18)


@pytest.mark.parametrize("seed", [0, 5, 9])
def test_codes_are_nearest_levels_k_group(seed):
    k = _groups(seed, (64, 128), 2.0, 0.3)
    q, s, z = oracle.kivi_affine_quantize_k_group(k)
    assert q.dtype == np.uint8 and q.max() <= 15
    for t in range(0, 64, 7):
        for c in range(128):
            assert _nearest_ok(k[t, c], q[t, c], s[c], z[c]), (t, c)


@pytest.mark.parametrize("seed", [0, 7])
def test_codes_are_nearest_levels_v_tokens(seed):
    v = _groups(seed, (40, 128), 1.5, -0.2)
    q, s, z = oracle.kivi_affine_quantize_v_tokens(v)
    assert s.shape == (40, 2) and z.shape == (40, 2)
    for t in range(40):
        for c in range(0, 128, 3):
            assert _nearest_ok(v[t, c], q[t, c], s[t, c // 64], z[t, c // 64]), (t, c)


def test_reconstruction_error_within_half_step():
    k = _groups(11, (64, 128), 4.0, 1.0)
    q, s, z = oracle.kivi_affine_quantize_k_group(k)
    err = np.abs((q.astype(np.float64) - z) * s.astype(np.float64) - k.astype(np.float64))
    assert np.all(err <= s.astype(np.float64) * (0.5 + 1e-6))


def test_degenerate_groups():
    # all zeros: scale 0, zero point 0, codes 0 (dequantized exactly 0)
    q, s, z = oracle.kivi_affine_quantize_k_group(np.zeros((64, 128), np.float16))
    assert np.all(s == 0) and np.all(z == 0) and np.all(q == 0)
    # a positive constant c: range [0, c], zero point 0, every code 15
    q, s, z = oracle.kivi_affine_quantize_k_group(np.full((64, 128), 3.0, np.float16))
    assert np.all(z == 0) and np.all(q == 15)
    assert np.all(s == np.float32(3.0) / np.float32(15.0))
    # a negative constant: range [c, 0], zero point 15, every code 0
    q, s, z = oracle.kivi_affine_quantize_k_group(np.full((64, 128), -2.5, np.float16))
    assert np.all(z == 15) and np.all(q == 0)
    # zero is always exact: a zero element dequantizes to 0
    x = _groups(3, (64, 128))
    x[5, :] = 0
    q, s, z = oracle.kivi_affine_quantize_k_group(x)
    assert np.all((q[5].astype(np.int64) - z) == 0)


def test_symmetric_range_closed_form():
    # values in {-a, +a}: scale 2a/15 and a / scale = 7.5 in exact
    # arithmetic, 7.4999996 in fp32 for a = 1: zero point 7, -a -> code 0,
    # +a -> 7 + 7 = 14 (levels 14 and 15 are equally near +a)
    x = np.array([[-1.0, 1.0, 1.0, -1.0]], np.float16).T
    x = np.repeat(x, 16, axis=0)                 # tokens 0..15 -a, 16..47 +a, 48..63 -a
    q, s, z = oracle.kivi_affine_quantize_k_group(x)
    assert s[0] == np.float32(2.0) / np.float32(15.0)
    assert z[0] == 7
    assert q[0, 0] == 0 and q[16, 0] == 14 and q[63, 0] == 0


def test_kivi_affine_sequence():
    g = np.random.default_rng(2)
    k = g.standard_normal((300, 2, 128)).astype(np.float16)
    v = (g.standard_normal((300, 2, 128)) + 0.7).astype(np.float16)
    kv = oracle.kivi_quantize(k, v, affine=True)
    assert kv["nq"] == 128 and kv["k_zp"].shape == (2, 2, 128) and kv["v_zp"].shape == (128, 2, 2)
    # groups are independent: group 1 of K equals quantizing it alone
    q1, s1, z1 = oracle.kivi_affine_quantize_k_group(k[64:128, 1])
    assert np.array_equal(kv["k_codes"][64:128, 1], q1)
    assert np.array_equal(kv["k_zp"][1, 1], z1)
    k_hat, v_hat = oracle.kivi_dequantize(kv)
    # affine reconstruction of the INT4 part within half a step; residual exact
    ks = np.repeat(kv["k_scales"], 64, axis=0).astype(np.float64)
    assert np.all(np.abs(k_hat[:128] - k[:128]) <= ks * (0.5 + 1e-6))
    assert np.array_equal(k_hat[128:], k[128:].astype(np.float64))
    assert np.array_equal(v_hat[128:], v[128:].astype(np.float64))
    # the affine form fits the shifted V better than the symmetric one
    sym = oracle.kivi_dequantize(oracle.kivi_quantize(k, v))[1]
    assert np.abs(v_hat[:128] - v[:128]).mean() < np.abs(sym[:128] - v[:128]).mean()


# --- 2-bit groups (qmax 3) -------------------------------------------------------

@pytest.mark.parametrize("seed,scale,shift", [(0, 1.0, 0.0), (6, 2.0, 1.5), (7, 0.05, -0.3)])
def test_two_bit_params_match_torch_observer(seed, scale, shift):
    x = _groups(seed, (64, 128), scale, shift)
    s, z = oracle.affine_params(x, 3, axis=0)
    t = torch.from_numpy(np.asarray(x, np.float32))
    ob = PerChannelMinMaxObserver(ch_axis=1, dtype=torch.quint8,
                                  qscheme=torch.per_channel_affine, quant_min=0, quant_max=3)
    ob(t)
    ts, tz = ob.calculate_qparams()
    assert np.array_equal(s.view(np.uint32), ts.numpy().astype(np.float32).view(np.uint32))
    assert np.array_equal(z, tz.numpy().astype(np.int64))


def test_two_bit_codes_are_nearest_levels():
    k = _groups(12, (64, 128), 1.0, 0.2)
    q, s, z = oracle.kivi_affine_quantize_k_group(k, qmax=3)
    assert q.max() <= 3
    for t in range(0, 64, 5):
        for c in range(128):
            xf, sf = Fraction(float(k[t, c])), Fraction(float(s[c]))
            dist = [abs(xf - (cc - int(z[c])) * sf) for cc in range(4)]
            if dist[int(q[t, c])] != min(dist):
                r = xf / sf
                frac = r - (r.numerator // r.denominator)
                assert abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 18), (t, c)
    v = _groups(13, (20, 128), 1.0, 0.5)
    qv, sv, zv = oracle.kivi_affine_quantize_v_tokens(v, qmax=3)
    err = np.abs((qv.astype(np.float64).reshape(20, 2, 64) - zv[..., None]) *
                 sv[..., None].astype(np.float64) - v.astype(np.float64).reshape(20, 2, 64))
    assert np.all(err <= sv[..., None] * (0.5 + 1e-6))


def test_two_bit_sequence():
    g = np.random.default_rng(9)
    k = g.standard_normal((260, 2, 128)).astype(np.float16)
    v = g.standard_normal((260, 2, 128)).astype(np.float16)
    kv = oracle.kivi_quantize(k, v, affine=True, bits=2)
    assert kv["nq"] == 128 and kv["k_codes"].max() <= 3 and kv["v_codes"].max() <= 3
    k_hat, v_hat = oracle.kivi_dequantize(kv)
    ks = np.repeat(kv["k_scales"], 64, axis=0).astype(np.float64)
    assert np.all(np.abs(k_hat[:128] - k[:128]) <= ks * (0.5 + 1e-6))
    # four levels reconstruct worse than sixteen
    k4 = oracle.kivi_dequantize(oracle.kivi_quantize(k, v, affine=True))[0]
    assert np.abs(k_hat[:128] - k[:128]).mean() > np.abs(k4[:128] - k[:128]).mean()
