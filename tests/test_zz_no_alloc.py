"""GPU test of kvq_write_decode_noalloc, the decode step whose split-K
partials live in the library's per-GPU array instead of a workspace.

It must give what kvq_write_decode gives on the same inputs, bit for bit
(same kernels; outputs and every cache array), on two calls in a row on one
device, the second smaller than the first (fewer rows, shorter rows,
another format), so the second runs over the partials the first left in
the shared array.  Both calls are split into several partitions per row,
so the partials are really used.  Four more calls in a row cover the
2-bit KIVI, BF16 and FP8 E5M2 paths and balanced partitions.  A call
whose partials would not fit is rejected on the host.
"""

import math

import numpy as np
import pytest
import torch

from quantized_paged_kv_02_amd import inputs

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _prefilled(w, lens, split, layer=0, partition="per-row"):
    """A cache holding the prefill (S-1 tokens) of rows ``lens`` plus the
    decode-step inputs."""
    from quantized_paged_kv_02_amd import kvq
    lens = np.asarray(lens, np.int32)
    table, nb = inputs.block_tables(w, lens)
    lay = kvq.make_layout(w.dtype, w.k_gran, w.v_gran, w.num_q_heads, w.num_kv_heads, nb,
                          table.shape[1], split, w.residual_len, partition=partition)
    static = ("tensor", "head", "channel")
    ks = np.full(kvq.scale_shape(lay, lay.k_gran), 0.05, np.float32) \
        if w.k_gran in static and w.dtype not in ("int4", "fp16") else None
    vs = np.full(kvq.scale_shape(lay, lay.v_gran), 0.05, np.float32) \
        if w.v_gran in static and w.dtype not in ("int4", "fp16") else None
    cache = kvq.alloc_cache(lay, ring_rows=len(lens), k_static=ks, v_static=vs)
    kk, vv = zip(*[inputs.gen_kv(w, layer, r, int(s), "cuda", 5) for r, s in enumerate(lens)])
    tab = torch.as_tensor(table, device="cuda")
    pre = lens - 1
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(pre)]).astype(np.int32), device="cuda")
    kvq.write(cache, torch.cat([k[:-1] for k in kk]).contiguous(),
              torch.cat([v[:-1] for v in vv]).contiguous(), cu, tab,
              torch.as_tensor(pre, device="cuda"), int(pre.max()))
    step = dict(k_new=torch.stack([k[-1] for k in kk]).contiguous(),
                v_new=torch.stack([v[-1] for v in vv]).contiguous(),
                q=inputs.gen_q(w, layer, "cuda", 5, batch=len(lens)),
                block_tables=tab, seq_lens=torch.as_tensor(lens, device="cuda"),
                max_seq_len=int(lens.max()), softmax_scale=1.0 / math.sqrt(128))
    return lay, cache, step


def _clone(cache):
    import copy
    c = copy.copy(cache)
    for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_resid", "v_resid"):
        t = getattr(cache, name)
        setattr(c, name, None if t is None else t.clone())
    return c


def _same_cache(a, b):
    for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_resid", "v_resid"):
        x, y = getattr(a, name), getattr(b, name)
        if x is None:
            continue
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"cache.{name} differs"


def _both(w, lens, split, partition="per-row"):
    """kvq_write_decode and kvq_write_decode_noalloc from one prefilled
    cache; compares outputs and caches bit for bit."""
    from quantized_paged_kv_02_amd import kvq
    lay, cache, step = _prefilled(w, lens, split, partition=partition)
    assert kvq.decode_workspace_bytes(lay, len(lens), step["max_seq_len"]) > 0, \
        "the case must use partials"
    other = _clone(cache)
    b, hq = len(lens), w.num_q_heads
    out_ref = torch.full((b, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    out_na = torch.full_like(out_ref, float("nan"))
    ws = kvq.alloc_workspace(lay, b, step["max_seq_len"])
    kvq.write_decode(cache, out=out_ref, workspace=ws, **step)
    kvq.write_decode_noalloc(other, out=out_na, **step)
    torch.cuda.synchronize()
    assert torch.isfinite(out_ref).all()
    assert torch.equal(out_ref.view(torch.int32), out_na.view(torch.int32)), \
        "kvq_write_decode_noalloc output differs from kvq_write_decode"
    _same_cache(cache, other)


def test_noalloc_matches_write_decode_twice():
    # first call: INT8 per-token, 6 rows of 600-1000 tokens in 128-token
    # partitions; second: KIVI INT4, 3 shorter rows in 64-token partitions
    w1 = inputs.scaled_down(W["tiny"], name="noalloc-int8", batch=6, num_q_heads=8,
                            num_kv_heads=2, table="shuffled")
    _both(w1, [1000, 600, 777, 999, 640, 1000], 128)
    w2 = inputs.scaled_down(W["tiny"], name="noalloc-int4", batch=3, num_q_heads=8,
                            num_kv_heads=2, dtype="int4", k_gran="channel", v_gran="token",
                            channel_outliers=(8, 10.0, "k"))
    _both(w2, [500, 383, 300], 64)


def test_noalloc_other_formats_in_a_row():
    # 2-bit KIVI (compact layout), then a BF16 cache, then FP8 E5M2 per
    # token, each smaller than the one before and each over the partials the
    # previous call left in the array
    w3 = inputs.scaled_down(W["tiny"], name="noalloc-int2", batch=4, num_q_heads=8,
                            num_kv_heads=2, dtype="int2-affine", k_gran="channel",
                            v_gran="token")
    _both(w3, [900, 450, 700, 333], 128)
    w4 = inputs.scaled_down(W["tiny"], name="noalloc-bf16", batch=3, num_q_heads=16,
                            num_kv_heads=2, dtype="bf16", k_gran="none", v_gran="none")
    _both(w4, [800, 500, 257], 64)
    w5 = inputs.scaled_down(W["tiny"], name="noalloc-e5m2", batch=2, num_q_heads=8,
                            num_kv_heads=2, dtype="fp8e5m2", k_gran="token", v_gran="token")
    _both(w5, [400, 130], 32)
    # balanced ranges (partials per row segment), over what the calls above left
    w6 = inputs.scaled_down(W["tiny"], name="noalloc-balanced", batch=5, num_q_heads=6,
                            num_kv_heads=2, table="shuffled")
    _both(w6, [1, 900, 40, 333, 17], 0, partition="balanced")


def test_noalloc_rejects_partials_beyond_the_array():
    from quantized_paged_kv_02_amd import kvq
    w = inputs.scaled_down(W["tiny"], name="noalloc-big", batch=64, num_q_heads=32,
                           num_kv_heads=32)
    lay, cache, step = _prefilled(w, [64] * 63 + [2048], 16)
    # 64 rows x 32 heads x 4 partitions x 130 floats = 4.3 MB would fit ...
    assert kvq.decode_workspace_bytes(lay, 64, 64) <= kvq.NOALLOC_SCRATCH_BYTES
    # ... a 2048-token bound with 16-token partitions (128 of them) does not
    assert step["max_seq_len"] == 2048
    assert kvq.decode_workspace_bytes(lay, 64, 2048) > kvq.NOALLOC_SCRATCH_BYTES
    out = torch.zeros((64, 32, 128), dtype=torch.float32, device="cuda")
    before = out.clone()
    with pytest.raises(kvq.KvqError, match="WORKSPACE"):
        kvq.write_decode_noalloc(cache, out=out, **step)
    torch.cuda.synchronize()
    assert torch.equal(out, before), "a rejected call must enqueue nothing"
