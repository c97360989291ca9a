"""Pins of the oracle's KIVI-style INT4 cache: group/residual split, the
per-channel (K) and per-token (V) scale axes, and the nibble packing."""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("s,nq", [(0, 0), (1, 0), (127, 0), (128, 0), (191, 0),
                                  (192, 64), (255, 64), (256, 128),
                                  (32767, 32576), (32768, 32640)])
def test_quantized_length_closed_form(s, nq):
    assert oracle.kivi_quantized_len(s) == nq


def test_residual_window_invariants():
    for s in range(0, 3000):
        nq = oracle.kivi_quantized_len(s)
        r = s - nq
        assert nq % 64 == 0
        if s >= 128:
            assert 128 <= r < 192
        else:
            assert r == s
    # the 32767 -> 32768 decode step quantizes exactly one more group and
    # leaves exactly 128 fp16 tokens
    assert oracle.kivi_quantized_len(32768) - oracle.kivi_quantized_len(32767) == 64
    assert 32768 - oracle.kivi_quantized_len(32768) == 128


def test_pack_explicit_bytes():
    codes = np.array([[1, -1, -8, 7, 0, -2, 3, 4]], np.int8)
    packed = oracle.pack_int4(codes)
    assert packed.tolist() == [[0xF1, 0x78, 0xE0, 0x43]]
    assert np.array_equal(oracle.unpack_int4(packed), codes)


def test_pack_unpack_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(b)), b)


def test_k_scales_are_per_channel_over_the_group():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((64, 128)).astype(np.float16)
    k[10, 5] = np.float16(70.0)                 # outlier in channel 5 only
    codes, s = oracle.kivi_quantize_k_group(k)
    assert s.shape == (128,)
    assert s[5] == np.float32(70.0) / np.float32(7)
    for c in range(128):
        col = np.abs(k[:, c].astype(np.float32))
        assert s[c] == np.float32(col.max()) / np.float32(7)
        i = int(np.argmax(col))
        assert abs(int(codes[i, c])) == 7
    assert codes.min() >= -8 and codes.max() <= 7


def test_v_scales_are_per_token_per_channel_group():
    rng = np.random.default_rng(12)
    v = rng.standard_normal((20, 128)).astype(np.float16)
    v[3, 100] = np.float16(-50.0)               # token 3, channel group 1
    codes, s = oracle.kivi_quantize_v_tokens(v)
    assert s.shape == (20, 2)
    assert s[3, 1] == np.float32(50.0) / np.float32(7)
    assert codes[3, 100] == -7
    for t in range(20):
        for j in range(2):
            blk = np.abs(v[t, 64 * j:64 * j + 64].astype(np.float32))
            assert s[t, j] == np.float32(blk.max()) / np.float32(7)


def test_kivi_whole_sequence_layout_and_residual():
    rng = np.random.default_rng(13)
    s_len, hkv, d = 300, 2, 128
    k = rng.standard_normal((s_len, hkv, d)).astype(np.float16)
    v = rng.standard_normal((s_len, hkv, d)).astype(np.float16)
    kv = oracle.kivi_quantize(k, v)
    assert kv["nq"] == 128
    assert np.array_equal(kv["k_resid"], k[128:]) and np.array_equal(kv["v_resid"], v[128:])
    k_hat, v_hat = oracle.kivi_dequantize(kv)
    assert k_hat.shape == (s_len, hkv, d)
    # residual tokens are exact; quantized ones within half a step
    assert np.array_equal(k_hat[128:], k[128:].astype(np.float64))
    ks = np.repeat(kv["k_scales"], 64, axis=0).astype(np.float64)
    err = np.abs(k_hat[:128] - k[:128].astype(np.float64))
    assert np.all(err <= ks * (0.5 + 7.5 * 2.0 ** -23))
    # group-by-group equals whole-sequence (each group depends on itself only)
    kv2 = oracle.kivi_quantize(k[:192], v[:192])
    assert np.array_equal(kv2["k_codes"], kv["k_codes"][:64])
    assert np.array_equal(kv2["v_scales"], kv["v_scales"][:64])
