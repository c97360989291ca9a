"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Codes and scales must match bit for bit; attention outputs within
atol 2e-3 + rtol 1e-2 of the oracle's fp64 attention over the same
dequantized values.  Sizes here span several blocks, partitions and a
ragged tail; the full-size workloads are in test_gpu_fullsize.py.
"""

import numpy as np
import pytest

from quantized_paged_kv_02_amd import inputs
from tests.gpu_harness import check_rows, run_case

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _small(dtype, kg, vg, hq=8, hkv=2, table="identity", **kw):
    return inputs.scaled_down(W["tiny"], name=f"small-{dtype}-{kg}-{vg}-{hq}-{hkv}",
                              batch=3, num_q_heads=hq, num_kv_heads=hkv, dtype=dtype,
                              k_gran=kg, v_gran=vg, table=table, **kw)


def test_tiny_workload_whole():
    w = W["tiny"]
    res = run_case(w, inputs.seq_lens(w), decode_twice=True)
    err = check_rows(res)
    assert np.array_equal(res.out, res.out2), "decode is not bitwise reproducible"
    print(f"tiny: max abs err {err:.2e}")


GRANS = ["tensor", "head", "channel", "token"]


@pytest.mark.parametrize("dtype", ["int8", "fp8", "fp8e5m2"])
@pytest.mark.parametrize("kg", GRANS)
@pytest.mark.parametrize("vg", GRANS)
def test_granularities(dtype, kg, vg):
    w = _small(dtype, kg, vg)
    res = run_case(w, [1, 37, 300], split_tokens=64)
    check_rows(res)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1), (16, 2), (32, 2), (12, 3)])
def test_group_sizes(hq, hkv):
    w = _small("int8", "token", "token", hq=hq, hkv=hkv)
    check_rows(run_case(w, [16, 33, 129], split_tokens=32))


@pytest.mark.parametrize("split", [0, 16, 64, 256, 4096])
def test_partition_sweep_fp8_shuffled(split):
    w = _small("fp8", "head", "head", table="shuffled")
    res = run_case(w, [15, 17, 700], split_tokens=split)
    check_rows(res)


def test_identity_vs_shuffled_tables_bitwise():
    wi = _small("int8", "token", "token", table="identity")
    ws = _small("int8", "token", "token", table="shuffled")
    a = run_case(wi, [100, 257, 31], split_tokens=64)
    b = run_case(ws, [100, 257, 31], split_tokens=64)
    assert not np.array_equal(a.table, b.table)
    assert np.array_equal(a.out, b.out)


def test_empty_rows_and_single_token():
    w = _small("int8", "token", "token")
    res = run_case(w, [0, 1, 0])
    assert np.all(res.out[0] == 0) and np.all(res.out[2] == 0)
    check_rows(res, rows=[1])


@pytest.mark.parametrize("lens,split", [([100, 192, 777], 64), ([1, 128, 129], 0),
                                        ([191, 192, 193], 128), ([640, 64, 2000], 256)])
def test_int4_kivi(lens, split):
    w = _small("int4", "channel", "token", channel_outliers=(8, 10.0, "k"))
    res = run_case(w, lens, split_tokens=split, decode_twice=True)
    check_rows(res)
    assert np.array_equal(res.out, res.out2)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (16, 2), (32, 2), (12, 3)])
@pytest.mark.parametrize("fused", [False, True])
def test_int4_group_sizes(hq, hkv, fused):
    # symmetric INT4, one query per row: query groups 1, 2 and 4 run the
    # compact layout, 8 and 16 the generic one
    w = _small("int4", "channel", "token", hq=hq, hkv=hkv, channel_outliers=(8, 10.0, "k"))
    check_rows(run_case(w, [300, 700, 191, 1000], split_tokens=128, fused=fused))


@pytest.mark.parametrize("chunks", [2, 3, 7])
def test_int4_chunked_writes(chunks):
    # groups flushed from a mix of ring tokens and new tokens, ring slots reused
    w = _small("int4", "channel", "token", channel_outliers=(8, 10.0, "k"))
    check_rows(run_case(w, [300, 1000, 450], chunks=chunks, split_tokens=64))


def test_int4_residual_64_shuffled():
    w = _small("int4", "channel", "token", residual_len=64, table="shuffled")
    check_rows(run_case(w, [63, 64, 65, 500], split_tokens=64))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype", ["int4", "int4-affine", "int2-affine"])
@pytest.mark.parametrize("residual", [256, 512])
def test_kivi_long_residual_windows(residual, dtype, fused):
    # fp16 windows of 256 and 512 tokens (rings of 320 and 576 slots): rows
    # inside the window, one group past it, at the next group's first token
    # and far past it, written in three chunks so the ring wraps between
    # writes
    w = _small(dtype, "channel", "token", residual_len=residual, table="shuffled",
               channel_outliers=(8, 10.0, "k"))
    lens = [residual - 1, residual + 64, residual + 65, 2000]
    check_rows(run_case(w, lens, chunks=3, split_tokens=128, fused=fused))


@pytest.mark.parametrize("chunks", [2, 5])
def test_int8_chunked_writes(chunks):
    w = _small("int8", "token", "channel")
    check_rows(run_case(w, [300, 1000, 17], chunks=chunks, split_tokens=128))


@pytest.mark.parametrize("dtype,kg,vg", [("int8", "token", "token"), ("int4", "channel", "token"),
                                         ("fp16", "none", "none"),
                                         ("int4-affine", "channel", "token"),
                                         ("int2-affine", "channel", "token")])
def test_repeated_split_launches_on_one_workspace(dtype, kg, vg):
    # many partitions per row; launches that reuse one workspace (partials
    # left by the previous launch) must agree bit for bit
    w = _small(dtype, kg, vg, table="shuffled")
    res = run_case(w, [1000, 64, 0, 777], split_tokens=64, repeats=6)
    for o in res.repeat_outs:
        assert np.array_equal(o.view(np.uint32), res.out.view(np.uint32))
    check_rows(res, rows=[0, 1, 3])
    assert np.all(res.out[2] == 0)


# --- unquantized FP16 cache: values stored bit for bit, attended as they are

@pytest.mark.parametrize("lens,split", [([1, 37, 300], 64), ([16, 17, 31, 32, 33], 0),
                                        ([0, 1, 0, 2], 0), ([777, 15, 2000], 256),
                                        ([100, 257, 31], 4096)])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fp16_cache(lens, split, dtype):
    w = _small(dtype, "none", "none", table="shuffled",
               channel_outliers=(4, 10.0, "kvq"))
    res = run_case(w, lens, split_tokens=split, decode_twice=True)
    live = [r for r, s in enumerate(lens) if s > 0]
    check_rows(res, rows=live)
    for r, s in enumerate(lens):
        if s == 0:
            assert np.all(res.out[r] == 0)
    assert np.array_equal(res.out, res.out2)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1), (16, 2), (12, 3)])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fp16_group_sizes(hq, hkv, dtype):
    w = _small(dtype, "none", "none", hq=hq, hkv=hkv)
    check_rows(run_case(w, [16, 33, 129], split_tokens=32))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fp16_chunked_writes(dtype):
    w = _small(dtype, "none", "none", table="shuffled")
    check_rows(run_case(w, [300, 1000, 17], chunks=3, split_tokens=128))


def test_bf16_cache_large_values():
    """bf16 values beyond fp16's range (V ~ N(0,1) * 1e6 on four channels)
    and below its smallest normal: the BF16 path never passes through fp16."""
    w = _small("bf16", "none", "none", channel_outliers=(4, 1.0e6, "v"))
    res = run_case(w, [300, 1000], split_tokens=128)
    check_rows(res)


# --- asymmetric (affine) INT4 KIVI groups: codes, scales and zero points bit
# for bit, attention within tolerance

def _affine(**kw):
    kw.setdefault("channel_outliers", (8, 10.0, "k"))
    return _small("int4-affine", "channel", "token", shift=(0.5, "v"), **kw)


@pytest.mark.parametrize("lens,split", [([100, 192, 777], 64), ([1, 128, 129], 0),
                                        ([191, 192, 193], 128), ([640, 64, 2000], 256),
                                        ([0, 255, 0], 0)])
def test_int4_affine(lens, split):
    w = _affine(table="shuffled")
    res = run_case(w, lens, split_tokens=split, decode_twice=True)
    check_rows(res, rows=[r for r, s in enumerate(lens) if s > 0])
    for r, s in enumerate(lens):
        if s == 0:
            assert np.all(res.out[r] == 0)
    assert np.array_equal(res.out, res.out2)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1), (8, 2), (16, 2)])
def test_int4_affine_group_sizes(hq, hkv):
    check_rows(run_case(_affine(hq=hq, hkv=hkv), [300, 700, 192], split_tokens=128))


@pytest.mark.parametrize("chunks", [2, 7])
def test_int4_affine_chunked_writes(chunks):
    check_rows(run_case(_affine(), [300, 1000, 450], chunks=chunks, split_tokens=64))


def test_int4_affine_residual_64_and_constant_groups():
    # residual window 64; no outliers and V without shift (zero points near 8)
    w = _small("int4-affine", "channel", "token", residual_len=64, table="shuffled")
    check_rows(run_case(w, [63, 64, 65, 500], split_tokens=64))


# --- 2-bit affine KIVI groups (compact path for query groups of at most
# four, generic path above)

def _two_bit(**kw):
    kw.setdefault("channel_outliers", (8, 10.0, "k"))
    return _small("int2-affine", "channel", "token", shift=(0.5, "v"), **kw)


@pytest.mark.parametrize("lens,split", [([100, 192, 777], 64), ([1, 128, 129], 0),
                                        ([191, 192, 193], 128), ([640, 64, 2000], 256),
                                        ([0, 255, 0], 0)])
def test_int2_affine(lens, split):
    res = run_case(_two_bit(table="shuffled"), lens, split_tokens=split, decode_twice=True)
    check_rows(res, rows=[r for r, s in enumerate(lens) if s > 0])
    for r, s in enumerate(lens):
        if s == 0:
            assert np.all(res.out[r] == 0)
    assert np.array_equal(res.out, res.out2)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (4, 1), (16, 2), (32, 2), (12, 3),
                                    (64, 8), (16, 1)])
@pytest.mark.parametrize("fused", [False, True])
def test_int2_affine_group_sizes(hq, hkv, fused):
    res = run_case(_two_bit(hq=hq, hkv=hkv, table="shuffled"), [300, 700, 192, 65],
                   split_tokens=128, fused=fused, decode_twice=True)
    check_rows(res)
    assert np.array_equal(res.out, res.out2)


@pytest.mark.parametrize("chunks", [3, 7])
def test_int2_affine_chunked_writes(chunks):
    check_rows(run_case(_two_bit(), [300, 1000, 450], chunks=chunks, split_tokens=64))


def test_int2_affine_residual_64():
    w = _small("int2-affine", "channel", "token", residual_len=64, table="shuffled")
    check_rows(run_case(w, [63, 64, 65, 500], split_tokens=64))


@pytest.mark.parametrize("dtype,kg,vg", [("int8", "token", "token"), ("fp8", "head", "head"),
                                         ("int4", "channel", "token")])
def test_planned_split_on_ragged_rows(dtype, kg, vg):
    # the host planner's partition length for unequal rows
    from quantized_paged_kv_02_amd import kvq
    extra = {"channel_outliers": (8, 10.0, "k")} if dtype == "int4" else {}
    w = _small(dtype, kg, vg, table="shuffled", **extra)
    lens = np.array([17, 300, 1000, 5, 64, 777, 2000, 130], np.int32)
    table, nb = inputs.block_tables(w, lens)
    lay = kvq.make_layout(w.dtype, w.k_gran, w.v_gran, w.num_q_heads, w.num_kv_heads, nb,
                          table.shape[1], 0, w.residual_len)
    split = kvq.plan_split_tokens(lay, lens)
    res = run_case(w, lens, split_tokens=split, table=table)
    check_rows(res)


# --- balanced partitions (the rows of a KV head cut into equal block ranges)

BAL_LENS = [1, 0, 300, 1000, 17, 64, 2000, 5]


@pytest.mark.parametrize("dtype,kg,vg,table", [("int8", "token", "token", "identity"),
                                               ("fp8", "head", "head", "shuffled"),
                                               ("fp8e5m2", "channel", "token", "shuffled"),
                                               ("int8", "channel", "tensor", "shuffled"),
                                               ("fp16", "none", "none", "shuffled"),
                                               ("bf16", "none", "none", "shuffled")])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("hkv", [2, 8])
def test_balanced_partitions(dtype, kg, vg, table, fused, hkv):
    # 2 KV heads: 128 ranges per head of one or two blocks, so rows span many
    # workgroups and many ranges hold several rows; 8 KV heads: 32 per head
    w = _small(dtype, kg, vg, hq=2 * hkv, hkv=hkv, table=table)
    res = run_case(w, BAL_LENS, partition="balanced", fused=fused, decode_twice=True)
    check_rows(res, rows=[r for r, s in enumerate(BAL_LENS) if s > 0])
    assert np.all(res.out[1] == 0)
    assert np.array_equal(res.out, res.out2)


def test_balanced_matches_per_row_closely():
    # the same attention; the partitions' running maxima differ, so the
    # weights' fp16 operands round differently
    w = _small("int8", "token", "token", hq=16, hkv=4, table="shuffled")
    a = run_case(w, BAL_LENS, partition="balanced", split_tokens=0)
    b = run_case(w, BAL_LENS, partition="per-row", split_tokens=64)
    assert np.allclose(a.out, b.out, atol=1e-3, rtol=1e-3)


@pytest.mark.parametrize("n_query", [2, 4])
def test_balanced_multi_query(n_query):
    w = _small("int8", "token", "token", hq=8, hkv=2, table="shuffled")
    res = run_case(w, [3, 1000, 40, 1], partition="balanced", n_query=n_query)
    check_rows(res)


@pytest.mark.parametrize("dtype,kg,vg", [("int8", "token", "token"), ("fp8", "head", "head"),
                                         ("fp8e5m2", "tensor", "token"),
                                         ("fp16", "none", "none"), ("bf16", "none", "none")])
@pytest.mark.parametrize("g,n_query", [(3, 1), (5, 1), (3, 3), (1, 5), (7, 2)])
def test_balanced_odd_columns(dtype, kg, vg, g, n_query):
    # balanced ranges with query groups and column counts (g x queries: 3,
    # 5, 9, 5, 14) that are not powers of two
    w = _small(dtype, kg, vg, hq=2 * g, hkv=2, table="shuffled")
    res = run_case(w, BAL_LENS, partition="balanced", n_query=n_query if n_query > 1 else 0)
    check_rows(res, rows=[r for r, s in enumerate(BAL_LENS) if s > 0])
    if n_query > 1:
        for r, s in enumerate(BAL_LENS):
            for j in range(n_query):
                if s - n_query + j < 0:
                    assert np.all(res.out[r, j] == 0), (r, j)
    else:
        assert np.all(res.out[1] == 0)


# Query groups that are not powers of two: the score tiles carry g live
# columns of 16 (8-bit and 16-bit caches, generic INT4 layout) or of 4
# (compact INT4 layout, g = 3), the rest zero queries whose outputs are
# never written.
ODD_GROUP_FORMATS = [("int8", "token", "token"), ("fp8", "head", "head"),
                     ("fp8e5m2", "tensor", "token"), ("int8", "channel", "tensor"),
                     ("fp16", "none", "none"), ("bf16", "none", "none"),
                     ("int4", "channel", "token"), ("int4-affine", "channel", "token"),
                     ("int2-affine", "channel", "token")]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("g", [3, 5, 6, 7])
@pytest.mark.parametrize("dtype,kg,vg", ODD_GROUP_FORMATS)
def test_odd_query_groups(dtype, kg, vg, g, fused):
    w = _small(dtype, kg, vg, hq=2 * g, hkv=2, table="shuffled",
               channel_outliers=(8, 10.0, "k"))
    res = run_case(w, [300, 700, 65], split_tokens=128, fused=fused, decode_twice=True)
    check_rows(res)
    assert np.array_equal(res.out, res.out2)
