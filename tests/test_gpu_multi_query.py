"""GPU parity of kvq_paged_decode_mq (several query tokens per row over the
cache, causal): every query's output against the oracle's multi-query
attention over the same dequantized cache, for every format, query
counts up to the 16 product columns, rows shorter than the query count
(queries that see no token give zeros), masked spans crossing pair and
partition boundaries, and n_query = 1 equal bit for bit to plain decode."""

import numpy as np
import pytest

from quantized_paged_kv_02_amd import inputs
from tests.gpu_harness import check_rows, run_case

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _w(dtype, kg, vg, hq, hkv, table="shuffled"):
    return inputs.scaled_down(W["tiny"], name=f"mq-{dtype}-{kg}-{vg}-{hq}-{hkv}", batch=4,
                              num_q_heads=hq, num_kv_heads=hkv, dtype=dtype, k_gran=kg,
                              v_gran=vg, table=table)


FORMATS = [("int8", "token", "token"), ("fp8", "head", "head"), ("fp16", "none", "none"),
           ("bf16", "none", "none"),
           ("fp8e5m2", "channel", "token"), ("int4", "channel", "token"),
           ("int4-affine", "channel", "token"), ("int2-affine", "channel", "token")]


@pytest.mark.parametrize("dtype,kg,vg", FORMATS)
@pytest.mark.parametrize("n_query,hq,hkv", [(2, 8, 4), (4, 8, 2), (8, 4, 2), (16, 2, 2)])
@pytest.mark.parametrize("split", [0, 64])
def test_multi_query_matches_oracle(dtype, kg, vg, n_query, hq, hkv, split):
    lens = [1, 3, 17, 31, 33, 300, 1000, 0]
    res = run_case(_w(dtype, kg, vg, hq, hkv), lens, split_tokens=split, n_query=n_query,
                   decode_twice=True)
    assert res.out.shape == (len(lens), n_query, hq, 128)
    check_rows(res, rows=[r for r, s in enumerate(lens) if s > 0])
    for r, s in enumerate(lens):
        for j in range(n_query):
            if s - n_query + j < 0:
                assert np.all(res.out[r, j] == 0), (r, j)
    assert np.array_equal(res.out.view(np.uint32), res.out2.view(np.uint32))


@pytest.mark.parametrize("dtype,kg,vg", FORMATS)
def test_single_query_equals_decode(dtype, kg, vg):
    w = _w(dtype, kg, vg, 8, 2)
    lens = [5, 64, 300, 1]
    one = run_case(w, lens, split_tokens=64, n_query=1)
    dec = run_case(w, lens, split_tokens=64)
    assert np.array_equal(one.out[:, 0].view(np.uint32), dec.out.view(np.uint32))


@pytest.mark.parametrize("dtype,kg,vg", FORMATS)
@pytest.mark.parametrize("n_query,hq,hkv", [(3, 3, 1), (5, 6, 2), (7, 4, 2), (3, 5, 5),
                                            (2, 14, 2), (5, 3, 3)])
@pytest.mark.parametrize("split", [0, 64])
def test_multi_query_odd_columns(dtype, kg, vg, n_query, hq, hkv, split):
    # n_query x g score columns that are not powers of two (9, 15, 14, 3,
    # 14, 5): column c is query token c / g of head c % g, each with its own
    # causal mask
    lens = [1, 4, 17, 31, 33, 300, 1000, 0]
    res = run_case(_w(dtype, kg, vg, hq, hkv), lens, split_tokens=split, n_query=n_query)
    assert res.out.shape == (len(lens), n_query, hq, 128)
    check_rows(res, rows=[r for r, s in enumerate(lens) if s > 0])
    for r, s in enumerate(lens):
        for j in range(n_query):
            if s - n_query + j < 0:
                assert np.all(res.out[r, j] == 0), (r, j)
