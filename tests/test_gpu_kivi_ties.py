"""GPU parity of KIVI group codes whose quotients x / scale sit on or next to
a rounding boundary.

A flush computes each code as round(x / scale) with the quotient rounded as
IEEE fp32 division rounds it, then half-to-even.  These cases build groups
from pairs (group amax a, value x) whose float32 quotient x / fl(a / qmax)
is exactly a half-integer or lies within 2^-17 of one, or lies just outside
that (found by brute force on the host, in float32, as the oracle
computes): the flush takes divisions for the first kind and multiplies by a
reciprocal for the second.  Keys carry them along each
channel's 64 tokens, values along each token's 64-channel groups.  Codes,
scales (and zero points) must equal the oracle's bit for bit; attention is
checked against the oracle as everywhere else.
"""

import numpy as np
import pytest
import torch

from quantized_paged_kv_02_amd import inputs
from tests.gpu_harness import check_rows, run_case

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS
WINDOW = np.float32(2.0 ** -17)


def _boundary_pairs(qmax, signed):
    """Two maps {fp16 amax a: fp16 values x}: quotients fl(x / fl(a / qmax))
    within 2^-17 of a half-integer (exact ties included; the flush divides
    for them), and ones just outside, 2^-17 .. 2^-9 away (the flush
    multiplies by the reciprocal there, where its error bound is tightest).
    |x| <= a, and x >= 0 unless ``signed``."""
    a16 = np.arange(0x3800, 0x5400, 7, dtype=np.uint16).view(np.float16)  # 0.5 .. 64
    near, close = {}, {}
    for a in a16:
        s = np.float32(a) / np.float32(qmax)
        ks = np.arange(-qmax - 1 if signed else 0, qmax)
        x0 = ((ks + 0.5) * np.float64(s)).astype(np.float16)
        bits = x0.view(np.uint16).astype(np.int32)
        cand = np.concatenate([bits + d for d in range(-6, 7)]).astype(np.uint16)
        x = np.unique(cand.view(np.float16))
        x = x[np.isfinite(x) & (np.abs(x.astype(np.float32)) <= np.float32(a))]
        if not signed:
            x = x[x >= 0]
        t = x.astype(np.float32) / s
        d = np.abs(t - np.floor(t) - np.float32(0.5))
        if (d <= WINDOW).any():
            near[a] = x[d <= WINDOW]
        if ((d > WINDOW) & (d <= 2.0 ** -9)).any():
            close[a] = x[(d > WINDOW) & (d <= 2.0 ** -9)]
    return near, close


def _vectors(rng, pairs, n, signed, qmax, clean):
    """n vectors of 64 fp16 values: element 0 is +-a (the vector's amax, so
    its scale is fl(a / qmax) in both the symmetric and the affine rule),
    the rest boundary values of that a mixed with ordinary ones.  ``clean``:
    ordinary values that fall within 2^-17 of a rounding boundary are
    swapped for boundary values from ``pairs`` (the just-outside kind)."""
    keys = list(pairs)
    out = np.empty((n, 64), np.float16)
    for i in range(n):
        a = keys[rng.integers(len(keys))]
        g = rng.choice(pairs[a], 64)
        ordinary = (rng.uniform(-1 if signed else 0, 1, 64) * np.float32(a)).astype(np.float16)
        g = np.where(rng.random(64) < 0.75, g, ordinary)
        g[0] = -a if (signed and rng.random() < 0.5) else a
        if clean:
            t = g.astype(np.float32) / (np.float32(a) / np.float32(qmax))
            inside = np.abs(t - np.floor(t) - np.float32(0.5)) <= WINDOW
            inside[0] = False
            g[inside] = rng.choice(pairs[a], int(inside.sum()))
        out[i] = rng.permutation(g)
    return out


def _crafted_kv(w, n_tokens, seed, qmax, signed):
    """K, V [S, H, 128].  Each (64-token group, KV head) takes either the
    near-tie or the just-outside values throughout: K along each channel's
    64 tokens, V along each token's two 64-channel groups."""
    rng = np.random.default_rng(seed)
    near, close = _boundary_pairs(qmax, signed)
    h = w.num_kv_heads
    groups = -(-n_tokens // 64)
    k = np.empty((groups * 64, h, 128), np.float16)
    v = np.empty((groups * 64, h, 128), np.float16)
    for g in range(groups):
        for hh in range(h):
            clean = rng.random() < 0.5
            pairs = close if clean else near
            k[64 * g:64 * (g + 1), hh, :] = _vectors(rng, pairs, 128, signed, qmax, clean).T
            v[64 * g:64 * (g + 1), hh, :] = _vectors(rng, pairs, 128, signed, qmax,
                                                     clean).reshape(64, 128)
    return k[:n_tokens], v[:n_tokens]


@pytest.mark.parametrize("dtype,qmax,signed", [("int4", 7, True), ("int4-affine", 15, False),
                                               ("int2-affine", 3, False)])
@pytest.mark.parametrize("fused", [False, True])
def test_kivi_codes_at_rounding_boundaries(monkeypatch, dtype, qmax, signed, fused):
    w = inputs.scaled_down(W["tiny"], name=f"ties-{dtype}", batch=3, num_q_heads=8,
                           num_kv_heads=2, dtype=dtype, k_gran="channel", v_gran="token")
    lens = [128 + 64 * 5, 128 + 64 * 2 + 17, 256, 128 + 64 * 3 - 1]

    def crafted(wl, layer, row, n_tokens, device="cpu", seed=0, offset=0):
        k, v = _crafted_kv(wl, n_tokens, 1000 * seed + 10 * row + layer, qmax, signed)
        return (torch.as_tensor(k, device=device), torch.as_tensor(v, device=device))

    monkeypatch.setattr(inputs, "gen_kv", crafted)
    # fused: the last token arrives with kvq_write_decode; at 319 the step
    # flushes the group [128, 192) in workgroups of its decode launch (one
    # token before it leaves the window), at 256 it reads [64, 128) flushed
    # by the write before
    res = run_case(w, lens, split_tokens=64, fused=fused)
    check_rows(res)
