"""Pins of the oracle's fp64 decode attention, split merge and paging.

Independent checks: PyTorch's scaled_dot_product_attention in fp64 (a library
routine the oracle does not call), closed forms (one token; identical keys;
zero query), softmax shift invariance built from an extra channel, split
merge versus unsplit, and identity versus shuffled block tables.
"""

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("hq,hkv,s", [(4, 2, 37), (8, 8, 5), (8, 1, 64), (16, 2, 300)])
def test_matches_torch_sdpa_fp64(hq, hkv, s):
    d = 128
    q = _rand((hq, d), 1)
    k = _rand((s, hkv, d), 2)
    v = _rand((s, hkv, d), 3)
    scale = 1.0 / np.sqrt(d)
    got = oracle.decode_attention(q, k, v, scale)
    g = hq // hkv
    qt = torch.from_numpy(q).reshape(1, hq, 1, d)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)
    want = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.contiguous(), vt.contiguous(), scale=scale).reshape(hq, d).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value():
    q = _rand((4, 128), 4)
    k = _rand((1, 2, 128), 5)
    v = _rand((1, 2, 128), 6)
    out = oracle.decode_attention(q, k, v, 0.1)
    assert np.array_equal(out[0], v[0, 0]) and np.array_equal(out[3], v[0, 1])


def test_identical_keys_or_zero_query_average_values():
    v = _rand((50, 2, 128), 7)
    k_same = np.repeat(_rand((1, 2, 128), 8), 50, axis=0)
    q = _rand((4, 128), 9)
    for kk, qq in [(k_same, q), (_rand((50, 2, 128), 10), np.zeros((4, 128)))]:
        out = oracle.decode_attention(qq, kk, v, 0.088)
        assert np.allclose(out[0], v[:, 0].mean(0), rtol=0, atol=1e-13)
        assert np.allclose(out[2], v[:, 1].mean(0), rtol=0, atol=1e-13)


def test_softmax_shift_invariance():
    # A constant added to every score (the "+0.01" of the FAQ) changes nothing:
    # build it with an extra channel whose key is 1 for every token.
    q = _rand((4, 128), 11)
    k = _rand((40, 2, 128), 12)
    v = _rand((40, 2, 128), 13)
    base = oracle.decode_attention(q, k, v, 0.1)
    q2 = np.concatenate([q, np.full((4, 1), 7.5)], axis=1)
    k2 = np.concatenate([k, np.ones((40, 2, 1))], axis=2)
    v2 = np.concatenate([v, np.zeros((40, 2, 1))], axis=2)
    shifted = oracle.decode_attention(q2, k2, v2, 0.1)[:, :128]
    assert np.allclose(base, shifted, rtol=1e-13, atol=1e-13)


def test_empty_sequence_is_zero():
    out = oracle.decode_attention(_rand((4, 128), 1), np.zeros((0, 2, 128)),
                                  np.zeros((0, 2, 128)), 0.1)
    assert not out.any()


def test_split_merge_equals_unsplit():
    q = _rand((8, 128), 14) * 3
    k = _rand((500, 2, 128), 15)
    v = _rand((500, 2, 128), 16)
    full = oracle.decode_attention(q, k, v, 0.088)
    for bounds in [[(0, 500)], [(0, 100), (100, 500)],
                   [(0, 16), (16, 17), (17, 400), (400, 500), (500, 500)]]:
        parts = oracle.decode_attention_partials(q, k, v, 0.088, bounds)
        assert np.allclose(oracle.merge_partials(parts), full, rtol=1e-12, atol=1e-12)


def test_paging_is_transparent():
    rng = np.random.default_rng(17)
    s_len, nb = 75, 12
    logical = rng.integers(-128, 128, (s_len, 2, 128)).astype(np.int8)
    ident = np.arange(nb)
    shuf = rng.permutation(nb)
    pool_a = oracle.paged_scatter(np.zeros((nb, 16, 2, 128), np.int8), logical, ident, s_len)
    pool_b = oracle.paged_scatter(np.zeros((nb, 16, 2, 128), np.int8), logical, shuf, s_len)
    assert np.array_equal(pool_a.reshape(-1, 2, 128)[:s_len], logical)
    assert np.array_equal(oracle.paged_gather(pool_b, shuf, s_len), logical)
    assert not np.array_equal(pool_a, pool_b)


def test_quantized_attention_lossless_case_matches_sdpa():
    # Integer-valued K/V with amax 127 per token quantize losslessly (scale 1),
    # so attention over the dequantized cache equals attention over the inputs.
    rng = np.random.default_rng(18)
    k = rng.integers(-127, 128, (30, 2, 128)).astype(np.float16)
    v = rng.integers(-127, 128, (30, 2, 128)).astype(np.float16)
    k[:, :, 0] = 127
    v[:, :, 0] = -127
    kc, ks = oracle.quantize_per_token(k, "int8")
    vc, vs = oracle.quantize_per_token(v, "int8")
    assert np.all(ks == 1) and np.all(vs == 1)
    q = rng.standard_normal((4, 128)) * 0.01
    a = oracle.decode_attention(q, oracle.dequantize(kc, ks[..., None], "int8"),
                                oracle.dequantize(vc, vs[..., None], "int8"), 0.088)
    b = oracle.decode_attention(q, k.astype(np.float64), v.astype(np.float64), 0.088)
    assert np.array_equal(a, b)


# --- several query tokens per sequence (causal) -------------------------------

@pytest.mark.parametrize("nq,hq,hkv,s", [(1, 4, 2, 37), (4, 8, 2, 50), (8, 2, 2, 9),
                                         (3, 4, 4, 2)])
def test_multi_query_matches_torch_causal_sdpa(nq, hq, hkv, s):
    # the queries are the last nq positions of a causal self-attention over
    # the s cached tokens: torch's SDPA with a boolean mask (an independent
    # library routine, fp64, KV heads repeated)
    g = np.random.default_rng(nq * 100 + s)
    q = g.standard_normal((nq, hq, 128))
    k = g.standard_normal((s, hkv, 128))
    v = g.standard_normal((s, hkv, 128))
    scale = 1 / np.sqrt(128)
    got = oracle.multi_query_attention(q, k, v, scale)
    rep = hq // hkv
    kt = torch.from_numpy(np.repeat(k, rep, axis=1)).permute(1, 0, 2)     # [hq, s, d]
    vt = torch.from_numpy(np.repeat(v, rep, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(q).permute(1, 0, 2)                             # [hq, nq, d]
    pos = np.arange(nq)[:, None] + (s - nq)
    mask = torch.from_numpy(np.arange(s)[None, :] <= pos)                 # [nq, s]
    want = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale).permute(1, 0, 2).numpy()
    visible = (pos[:, 0] >= 0)
    assert np.allclose(got[visible], want[visible], atol=1e-12, rtol=1e-12)
    assert np.all(got[~visible] == 0)


def test_multi_query_last_query_is_plain_decode():
    g = np.random.default_rng(8)
    q = g.standard_normal((5, 4, 128))
    k = g.standard_normal((40, 2, 128))
    v = g.standard_normal((40, 2, 128))
    got = oracle.multi_query_attention(q, k, v, 0.1)
    assert np.array_equal(got[-1], oracle.decode_attention(q[-1], k, v, 0.1))
    # query 0 sees 36 tokens: the value of token 39 cannot reach it
    v2 = v.copy()
    v2[39] += 100.0
    got2 = oracle.multi_query_attention(q, k, v2, 0.1)
    assert np.array_equal(got2[0], got[0]) and not np.allclose(got2[-1], got[-1])
