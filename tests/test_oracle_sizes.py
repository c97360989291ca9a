"""Pins of the oracle's size model against the numbers the pages print."""

import os
from fractions import Fraction

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split("|")]


@pytest.mark.parametrize("row", list(_rows("kv_sizes.txt")), ids=lambda r: r[0])
def test_printed_cache_sizes(row):
    _, layers, heads, dim, seq, batch, dtype, value, unit, tol, _cite = row
    got = oracle.kv_cache_bytes(int(layers), int(heads), int(dim), int(seq),
                                oracle.BYTES_PER_VALUE[dtype], int(batch))
    unit_bytes = {"GiB": 2 ** 30, "GB": 10 ** 9}[unit]
    want = Fraction(value) * unit_bytes
    if float(tol) == 0:
        assert got == want
    else:
        assert abs(float(got) / float(want) - 1) <= float(tol)


def test_bytes_per_value_table():
    for fmt, nbytes, ratio in _rows("bytes_per_value.txt"):
        assert oracle.BYTES_PER_VALUE[fmt] == Fraction(nbytes)
        assert oracle.BYTES_PER_VALUE["fp16"] / oracle.BYTES_PER_VALUE[fmt] == Fraction(ratio)


def test_exact_llama2_7b_closed_form():
    # 2 * 4 * 32 * 32 * 2048 * 128 * 2 bytes is exactly 4 GiB, INT8 half of it.
    assert oracle.kv_cache_bytes(32, 32, 128, 2048, 2, 4) == 4 * 2 ** 30
    assert oracle.kv_cache_bytes(32, 32, 128, 2048, 1, 4) == 2 * 2 ** 30
    # 7B at 10 000 tokens, fp16: 5 242 880 000 bytes.
    assert oracle.kv_cache_bytes(32, 32, 128, 10000, 2) == 5_242_880_000


def test_int4_code_bytes_are_half_the_values():
    # 1 000 values at 0.5 byte each, and the packer agrees.
    assert oracle.kv_cache_bytes(1, 1, 125, 4, oracle.BYTES_PER_VALUE["int4"]) == 500
    import numpy as np
    codes = np.zeros((3, 128), np.int8)
    assert oracle.pack_int4(codes).nbytes == 3 * 64


def test_gqa_uses_kv_heads():
    # 32 query heads over 8 KV heads: the cache is sized by the 8 KV heads.
    mha = oracle.kv_cache_bytes(32, 32, 128, 8192, 2)
    gqa = oracle.kv_cache_bytes(32, 8, 128, 8192, 2)
    assert mha == 4 * gqa
