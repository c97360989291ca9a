"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/kvq.h declares, and rejects bad arguments on the
host before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

from quantized_paged_kv_02_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

FAKE = 0x10000      # an aligned non-null "device" address; never dereferenced


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(kvq.EXPORTED)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(kvq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_struct_sizes_match_header():
    # kvq_layout: 1 uint32 + 13 int32; kvq_cache: 6 pointers + int32 (+pad)
    assert ctypes.sizeof(kvq.Layout) == 56
    assert ctypes.sizeof(kvq.Cache) == 56


def _cache(int4=False, ring_rows=4, **over):
    c = kvq.Cache(FAKE, FAKE, FAKE, FAKE, FAKE if int4 else None, FAKE if int4 else None,
                  ring_rows)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def _layout(**over):
    lay = kvq.make_layout("int8", "token", "token", 8, 2, 64, 16)
    for k, v in over.items():
        setattr(lay, k, v)
    return lay


OK, INV, UNS, ALN, WS, CAP, HIP = 0, -1, -2, -3, -4, -5, -6


@pytest.mark.parametrize("over,code", [
    ({}, OK),
    ({"struct_size": 12}, INV),
    ({"dtype": 0}, INV),
    ({"dtype": 9}, INV),
    ({"k_gran": 4}, INV),
    ({"v_gran": -1}, INV),
    ({"num_q_heads": 7}, INV),          # not a multiple of the KV heads
    ({"num_kv_heads": 0}, INV),
    ({"num_blocks": 0}, INV),
    ({"max_blocks_per_seq": 0}, INV),
    ({"split_tokens": 8}, INV),         # not a multiple of 16
    ({"split_tokens": -16}, INV),
    ({"head_dim": 64}, UNS),
    ({"block_size": 32}, UNS),
    ({"num_q_heads": 34}, UNS),         # 17 query heads per KV head
])
def test_validate_layout(over, code):
    assert kvq.validate(_layout(**over), _cache(), 2, 100) == code


def test_validate_int4_rules():
    base = dict(dtype=3, k_gran=2, v_gran=3, residual_len=128, group_size=64)
    assert kvq.validate(_layout(**base), _cache(int4=True), 2, 100) == OK
    assert kvq.validate(_layout(**{**base, "k_gran": 3}), _cache(int4=True), 2, 100) == UNS
    assert kvq.validate(_layout(**{**base, "group_size": 32}), _cache(int4=True), 2, 100) == UNS
    assert kvq.validate(_layout(**{**base, "residual_len": 100}), _cache(int4=True), 2, 100) == UNS
    assert kvq.validate(_layout(**{**base, "split_tokens": 48}), _cache(int4=True), 2, 100) == INV
    assert kvq.validate(_layout(**base), _cache(int4=False), 2, 100) == INV      # no rings
    assert kvq.validate(_layout(**base), _cache(int4=True, ring_rows=1), 2, 100) == CAP


def test_validate_cache_and_sizes():
    lay = _layout()
    assert kvq.validate(lay, None, 2, 100) == INV
    assert kvq.validate(lay, _cache(k_codes=None), 2, 100) == INV
    assert kvq.validate(lay, _cache(v_scales=FAKE + 4), 2, 100) == ALN
    assert kvq.validate(lay, _cache(), -1, 100) == INV
    assert kvq.validate(lay, _cache(), 2, -1) == INV
    assert kvq.validate(lay, _cache(), 2, 16 * 16) == OK
    assert kvq.validate(lay, _cache(), 2, 16 * 16 + 1) == CAP
    assert kvq.validate(lay, _cache(), 0, 0) == OK


def test_status_strings():
    for code in (OK, INV, UNS, ALN, WS, CAP, HIP):
        assert kvq.status_str(code).startswith(kvq.STATUS[code])
    assert kvq.status_str(-99) == "KVQ_ERR_UNKNOWN"


def test_workspace_bytes():
    lay = _layout()
    a = kvq.decode_workspace_bytes(lay, 4, 256)
    assert a > 0 and a % 256 == 0
    assert kvq.decode_workspace_bytes(lay, 8, 256) > a
    assert kvq.decode_workspace_bytes(_layout(head_dim=64), 4, 256) == 0
    # explicit partitions: 4 rows x 8 q heads x ceil(256/64) slots of (m, l, o[128])
    lay64 = _layout(split_tokens=64)
    rows = 4 * 8 * 4
    want = 2 * ((rows * 4 + 255) // 256 * 256) + rows * 512
    assert kvq.decode_workspace_bytes(lay64, 4, 256) == want
    # one partition per row: the decode kernel writes the output directly
    assert kvq.decode_workspace_bytes(_layout(split_tokens=256), 4, 256) == 0
    # INT4 always has a residual partition beside the INT4 ones
    lay4 = _layout(dtype=3, k_gran=2, v_gran=3, split_tokens=64)
    assert kvq.decode_workspace_bytes(lay4, 2, 100) == 0          # residual only
    assert kvq.decode_workspace_bytes(lay4, 2, 128 + 64 + 64) > 0


def _decode(lay, cache, q=FAKE, bt=FAKE, sl=FAKE, batch=2, max_len=100, scale=0.1,
            out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return kvq.LIB.kvq_paged_decode(ctypes.byref(lay), ctypes.byref(cache), q, bt, sl, batch,
                                    max_len, scale, out, ws, ws_bytes, None)


def _write(lay, cache, kn=FAKE, vn=FAKE, cu=FAKE, bt=FAKE, sl=FAKE, batch=2, total=4, max_new=2):
    return kvq.LIB.kvq_write(ctypes.byref(lay), ctypes.byref(cache), kn, vn, cu, bt, sl, batch,
                             total, max_new, None)


def _write_decode(lay, cache, kn=FAKE, vn=FAKE, q=FAKE, bt=FAKE, sl=FAKE, batch=2, max_len=100,
                  scale=0.1, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return kvq.LIB.kvq_write_decode(ctypes.byref(lay), ctypes.byref(cache), kn, vn, q, bt, sl,
                                    batch, max_len, scale, out, ws, ws_bytes, None)


def test_write_decode_rejects_before_launch():
    lay, c = _layout(), _cache()
    assert _write_decode(lay, c, kn=None) == INV
    assert _write_decode(lay, c, vn=None) == INV
    assert _write_decode(lay, c, kn=FAKE + 8) == ALN
    assert _write_decode(lay, c, q=None) == INV
    assert _write_decode(lay, c, out=FAKE + 4) == ALN
    assert _write_decode(lay, c, scale=float("inf")) == INV
    assert _write_decode(lay, c, max_len=10 ** 6) == CAP
    split = _layout(split_tokens=16)
    assert _write_decode(split, c, ws_bytes=16) == WS
    assert _write_decode(lay, c, batch=0) == OK            # nothing to do, nothing launched
    assert _write_decode(lay, c, batch=0, kn=None) == OK
    lay4 = _layout(dtype=3, k_gran=2, v_gran=3, residual_len=128, group_size=64)
    c4 = _cache(int4=True)
    assert kvq.validate(lay4, c4, 2, 100) == OK
    assert _write_decode(lay4, c4, vn=None) == INV
    assert _write_decode(lay4, c4, kn=FAKE + 2) == ALN


def test_entry_points_reject_before_launch():
    lay, c = _layout(), _cache()
    assert _decode(lay, c, q=None) == INV
    assert _decode(lay, c, out=FAKE + 8) == ALN
    split = _layout(split_tokens=16)              # 7 partitions: partials needed
    assert _decode(split, c, ws=FAKE + 16) == WS
    assert _decode(split, c, ws_bytes=16) == WS
    assert _decode(split, c, ws=None) == WS
    assert _decode(lay, c, scale=float("nan")) == INV
    assert _decode(lay, c, max_len=10 ** 6) == CAP
    assert _decode(lay, c, batch=0) == OK            # nothing to do, nothing launched
    assert _write(lay, c, kn=None) == INV
    assert _write(lay, c, cu=FAKE + 4) == ALN
    assert _write(lay, c, total=-1) == INV
    assert _write(lay, c, max_new=10 ** 6) == CAP
    assert _write(lay, c, total=0) == OK             # empty write is a no-op
    assert _write(lay, c, batch=0) == OK


def test_decode_rejects_oversized_grid():
    # one block per partition over 2^20 tokens: 65536 partitions per row, so
    # 128 rows x 2 KV heads need 2^24 workgroups of 256 threads (the 1-D
    # grid's 32-bit work-item count overflows)
    lay = _layout(split_tokens=16, max_blocks_per_seq=65536, num_blocks=1 << 20)
    c = _cache()
    assert _decode(lay, c, batch=128, max_len=1 << 20) == UNS
    assert _write_decode(lay, c, batch=128, max_len=1 << 20) == UNS
    # one row fewer fits the grid; its partials then exceed the workspace
    assert _decode(lay, c, batch=127, max_len=1 << 20) == WS


@pytest.mark.parametrize("dt", [4, 8])
def test_fp16_cache_rules(dt):
    # an FP16 or BF16 cache has no scales: NULL scale pointers and any
    # granularity field are accepted, the code arrays are still required and
    # aligned
    lay = _layout(dtype=dt, k_gran=77, v_gran=-5)
    bare = _cache(k_scales=None, v_scales=None)
    assert kvq.validate(lay, bare, 2, 100) == OK
    assert kvq.validate(lay, _cache(k_codes=None, k_scales=None, v_scales=None), 2, 100) == INV
    assert kvq.validate(lay, _cache(v_codes=FAKE + 2, k_scales=None, v_scales=None), 2,
                        100) == ALN
    assert kvq.validate(_layout(dtype=6), bare, 2, 100) == INV
    assert kvq.validate(_layout(dtype=dt, split_tokens=24), bare, 2, 100) == INV
    assert _decode(lay, bare, q=None) == INV
    assert _write(lay, bare, cu=FAKE + 4) == ALN
    assert _write_decode(lay, bare, vn=None) == INV
    # same partition plan rules: a split launch needs partials
    assert kvq.decode_workspace_bytes(_layout(dtype=dt, split_tokens=16), 2, 100) > 0


def test_int4_affine_rules():
    # same rules as the symmetric INT4 cache: K per channel, V per token,
    # group 64, residual a multiple of 64, rings required
    base = dict(dtype=5, k_gran=2, v_gran=3, residual_len=128, group_size=64)
    assert kvq.validate(_layout(**base), _cache(int4=True), 2, 100) == OK
    assert kvq.validate(_layout(**{**base, "v_gran": 2}), _cache(int4=True), 2, 100) == UNS
    assert kvq.validate(_layout(**{**base, "group_size": 128}), _cache(int4=True), 2, 100) == UNS
    assert kvq.validate(_layout(**{**base, "split_tokens": 16}), _cache(int4=True), 2, 100) == INV
    assert kvq.validate(_layout(**base), _cache(int4=False), 2, 100) == INV
    assert kvq.validate(_layout(**base), _cache(int4=True, k_scales=None), 2, 100) == INV
    assert kvq.validate(_layout(**base), _cache(int4=True, v_scales=FAKE + 4), 2, 100) == ALN
    lay = _layout(**{**base, "split_tokens": 64})
    assert kvq.decode_workspace_bytes(lay, 2, 100) == 0             # residual only
    assert kvq.decode_workspace_bytes(lay, 2, 128 + 64 + 64) > 0
    assert _write_decode(_layout(**base), _cache(int4=True), kn=None) == INV


def _calibrate(lay, k=FAKE, v=FAKE, n=100, ks=FAKE, vs=FAKE, acc=0, ws=FAKE, ws_bytes=1 << 30):
    return kvq.LIB.kvq_calibrate(ctypes.byref(lay), k, v, n, ks, vs, acc, ws, ws_bytes, None)


def test_calibrate_rules():
    lay = _layout(dtype=2, k_gran=0, v_gran=1)                 # FP8, tensor / head
    need = kvq.calibrate_workspace_bytes(lay, 100)
    # two chunks of partial channel maxima (100 tokens, 64 per chunk), K and V
    assert need == 2 * 2 * 2 * 128 * 4
    assert kvq.calibrate_workspace_bytes(lay, 10 ** 6) == 256 * 2 * 2 * 128 * 4   # capped
    assert kvq.calibrate_workspace_bytes(lay, 0) == 0
    assert _calibrate(lay, n=-1) == INV
    assert _calibrate(lay, n=0) == OK                      # nothing to do
    assert _calibrate(lay, k=None) == INV
    assert _calibrate(lay, vs=None) == INV
    assert _calibrate(lay, k=FAKE + 2) == ALN
    assert _calibrate(lay, ws=None) == WS
    assert _calibrate(lay, ws=FAKE + 64) == WS
    assert _calibrate(lay, ws_bytes=need - 1) == WS
    # per-token tensors are not calibrated: their pointers may be NULL
    tok = _layout(dtype=1, k_gran=3, v_gran=3)
    assert _calibrate(tok, k=None, v=None, ks=None, vs=None) == OK
    # no static scales: INT4, affine INT4, FP16, BF16
    for dt, kg, vg in ((3, 2, 3), (5, 2, 3), (4, 0, 0), (8, 0, 0)):
        assert _calibrate(_layout(dtype=dt, k_gran=kg, v_gran=vg)) == UNS
    assert _calibrate(_layout(dtype=2, k_gran=0, v_gran=0, num_kv_heads=257,
                              num_q_heads=257)) == UNS


def test_fp8_e5m2_layout_is_accepted():
    lay = _layout(dtype=6, k_gran=3, v_gran=0)
    assert kvq.validate(lay, _cache(), 2, 100) == OK
    assert kvq.decode_workspace_bytes(_layout(dtype=6, split_tokens=16), 2, 100) > 0


def _decode_mq(lay, cache, nq=2, q=FAKE, batch=2, max_len=100, ws=FAKE, ws_bytes=1 << 30):
    return kvq.LIB.kvq_paged_decode_mq(ctypes.byref(lay), ctypes.byref(cache), q, nq, FAKE,
                                       FAKE, batch, max_len, 0.1, FAKE, ws, ws_bytes, None)


def test_multi_query_rules():
    lay = _layout(split_tokens=16)                        # g = 4
    one = kvq.paged_decode_mq_workspace_bytes(lay, 1, 2, 100)
    assert one == kvq.decode_workspace_bytes(lay, 2, 100) and one > 0
    assert kvq.paged_decode_mq_workspace_bytes(lay, 4, 2, 100) > one
    assert kvq.paged_decode_mq_workspace_bytes(lay, 5, 2, 100) == 0      # 5 x 4 > 16 columns
    assert _decode_mq(lay, _cache(), nq=0) == INV
    assert _decode_mq(lay, _cache(), nq=5) == UNS
    assert _decode_mq(lay, _cache(), q=None) == INV
    assert _decode_mq(lay, _cache(), ws_bytes=16) == WS
    assert _decode_mq(lay, _cache(), batch=0) == OK
    lay4 = _layout(dtype=3, k_gran=2, v_gran=3)
    assert _decode_mq(lay4, _cache(int4=True), nq=5) == UNS
    assert kvq.paged_decode_mq_workspace_bytes(_layout(dtype=5, k_gran=2, v_gran=3,
                                                       split_tokens=64), 4, 2, 1000) > 0


def test_int2_affine_rules():
    base = dict(dtype=7, k_gran=2, v_gran=3, residual_len=128, group_size=64)
    assert kvq.validate(_layout(**base), _cache(int4=True), 2, 100) == OK         # g = 4
    assert kvq.validate(_layout(**{**base, "num_q_heads": 16}), _cache(int4=True), 2,
                        100) == OK                                               # g = 8
    assert kvq.validate(_layout(**{**base, "num_q_heads": 64}), _cache(int4=True), 2,
                        100) == UNS                                              # g = 32
    assert kvq.validate(_layout(**{**base, "k_gran": 3}), _cache(int4=True), 2, 100) == UNS
    assert kvq.validate(_layout(**base), _cache(int4=False), 2, 100) == INV
    assert _decode_mq(_layout(**base), _cache(int4=True), nq=2, batch=0) == OK
    assert _decode_mq(_layout(**base), _cache(int4=True), nq=5) == UNS         # 20 columns
    assert kvq.paged_decode_mq_workspace_bytes(_layout(**base, split_tokens=64), 2, 2,
                                               1000) > 0
    assert _calibrate(_layout(**base)) == UNS


def test_plan_split_tokens():
    lay = _layout()                                              # INT8, 16 blocks per row max
    lens = [256, 256]
    sp = kvq.plan_split_tokens(lay, lens)
    assert sp > 0 and sp % 16 == 0
    # equal lengths: the automatic plan's workspace
    lay2 = _layout(split_tokens=sp)
    assert kvq.decode_workspace_bytes(lay2, 2, 256) == kvq.decode_workspace_bytes(lay, 2, 256)
    # INT4: a multiple of 64 tokens
    lay4 = _layout(dtype=3, k_gran=2, v_gran=3, max_blocks_per_seq=64)
    assert kvq.plan_split_tokens(lay4, [1000, 200]) % 64 == 0
    lib = kvq.LIB
    assert lib.kvq_plan_split_tokens(ctypes.byref(lay), None, 2) == INV
    import numpy as np
    neg = np.array([5, -1], np.int32)
    assert lib.kvq_plan_split_tokens(ctypes.byref(lay), neg.ctypes.data, 2) == INV
    big = np.array([16 * 16 + 1], np.int32)
    assert lib.kvq_plan_split_tokens(ctypes.byref(lay), big.ctypes.data, 1) == CAP
    assert lib.kvq_plan_split_tokens(ctypes.byref(lay), None, 0) > 0
    assert lib.kvq_plan_split_tokens(ctypes.byref(_layout(head_dim=64)), None, 0) == UNS


def test_plans_of_the_measured_shapes():
    """The partition plans measured fastest on MI355X (host-only planner)."""
    import numpy as np
    from quantized_paged_kv_02_amd import inputs
    W = inputs.WORKLOADS

    def layout(w, mbs):
        return kvq.make_layout(w.dtype, w.k_gran, w.v_gran, w.num_q_heads, w.num_kv_heads,
                               w.batch * mbs, mbs, 0, w.residual_len)

    # INT8 short rows: one workgroup per CU per round (2 x 1024 tokens per row)
    l2 = layout(W["llama2-7b"], 128)
    assert kvq.plan_split_tokens(l2, np.full(4, 2048, np.int32)) == 1024
    # compact INT4: at most one workgroup per CU, the shortest such partition
    k4 = layout(W["kivi-int4"], 2048)
    lens = np.full(16, 32768, np.int32)
    assert kvq.plan_split_tokens(k4, lens) == 16384
    # 128 partials of 2 slots: (m, l) and o for 16 x 32 query heads
    one = kvq.decode_workspace_bytes(k4, 16, 32768)
    assert one == kvq.paged_decode_mq_workspace_bytes(k4, 1, 16, 32768)
    # several queries per row run on the generic INT4 layout: two
    # workgroups per CU, so twice the partitions, per query
    assert kvq.paged_decode_mq_workspace_bytes(k4, 2, 16, 32768) == 4 * one
    # affine INT4 groups: two workgroups per CU (arithmetic-bound)
    ka = layout(W["kivi-int4-affine"], 2048)
    assert kvq.plan_split_tokens(ka, lens) == 8192
    # FP16 short rows keep two resident workgroups per CU per round
    f16 = layout(W["llama2-7b-fp16"], 128)
    assert kvq.plan_split_tokens(f16, np.full(4, 2048, np.int32)) == 512


# --- host-side check of block tables and lengths (kvq_check_tables)

def _tab_layout(dtype="int8", nb=10, mbs=4):
    kg, vg = ("channel", "token") if dtype == "int4" else ("token", "token")
    return kvq.make_layout(dtype, kg, vg, 8, 2, nb, mbs)


def test_check_tables_accepts_valid_tables():
    lay = _tab_layout()
    tab = [[0, 1, 2, 0], [3, 4, 5, 6]]        # row 0 uses 3 entries (S = 40)
    assert kvq.check_tables(lay, tab, [40, 64], 64) == (OK, -1)
    assert kvq.check_tables(lay, tab, [0, 0], 0) == (OK, -1)
    assert kvq.check_tables(lay, [[0] * 4] * 0, [], 0) == (OK, -1)


@pytest.mark.parametrize("tab,lens,max_len,want", [
    ([[0, 1, 2, 0], [3, 4, 5, 6]], [40, 65], 64, (CAP, 1)),     # length above max_seq_len
    ([[0, 1, 2, 0], [3, 4, 5, 6]], [-1, 64], 64, (INV, 0)),     # negative length
    ([[0, 1, 10, 0], [3, 4, 5, 6]], [40, 64], 64, (INV, 0)),    # id == num_blocks
    ([[0, 1, 2, 0], [3, -4, 5, 6]], [40, 64], 64, (INV, 1)),    # negative id
    ([[0, 1, 2, 0], [3, 4, 2, 6]], [40, 64], 64, (INV, 1)),     # block used by two rows
    ([[0, 0, 2, 0], [3, 4, 5, 6]], [40, 64], 64, (INV, 0)),     # used twice in one row
    ([[0, 1, 2, 0], [3, 4, 5, 6]], [40, 64], 65, (CAP, -1)),    # beyond MBS * 16
])
def test_check_tables_rejects(tab, lens, max_len, want):
    assert kvq.check_tables(_tab_layout(), tab, lens, max_len) == want


def test_check_tables_kivi_counts_int4_blocks_only():
    # KIVI: a row of length S touches the INT4 blocks of groups below
    # nq(S + 1); S = 255 -> nq(256) = 128 -> 8 blocks, S = 191 -> 4 blocks
    lay = _tab_layout("int4", nb=20, mbs=16)
    tab = np.full((2, 16), -1, np.int32)
    tab[0, :8] = np.arange(8)
    tab[1, :4] = np.arange(8, 12)
    assert kvq.check_tables(lay, tab, [255, 191], 256) == (OK, -1)
    tab[1, 3] = -1
    assert kvq.check_tables(lay, tab, [255, 191], 256) == (INV, 1)
    assert kvq.check_tables(lay, tab, [255, 190], 256) == (OK, -1)   # nq(191) = 0


def test_binding_rejects_host_tensors():
    # the binding checks every tensor before a pointer crosses the ABI
    import torch
    lay = _tab_layout()
    t = lambda *s, d=torch.uint8: torch.zeros(s, dtype=d)   # noqa: E731
    cache = kvq.KVCache(lay, t(10, 2, 2048), t(10, 2, 2048), t(10, 2, 16, d=torch.float32),
                        t(10, 2, 16, d=torch.float32), None, None, 0)
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.paged_decode(cache, t(1, 8, 128, d=torch.float16), t(1, 4, d=torch.int32),
                         t(1, d=torch.int32), 16, 0.1, t(1, 8, 128, d=torch.float32),
                         t(256))


def test_noalloc_rejects_oversized_partials_before_any_hip_call():
    # 64 rows x 32 query heads x 128 partitions x 520 bytes > 16 MiB: rejected
    # on the host (fake pointers: nothing is dereferenced or launched)
    lay = kvq.make_layout("int8", "token", "token", 32, 32, 8192, 128, 16)
    assert kvq.decode_workspace_bytes(lay, 64, 2048) > kvq.NOALLOC_SCRATCH_BYTES
    st = kvq.LIB.kvq_write_decode_noalloc(ctypes.byref(lay), ctypes.byref(_cache()), FAKE, FAKE,
                                          FAKE, FAKE, FAKE, 64, 2048, 0.1, FAKE, None)
    assert st == WS
    # argument errors come first, as for kvq_write_decode
    st = kvq.LIB.kvq_write_decode_noalloc(ctypes.byref(lay), ctypes.byref(_cache()), FAKE, FAKE,
                                          FAKE, FAKE, FAKE, 64, 4096, 0.1, FAKE, None)
    assert st == CAP
    assert kvq.LIB.kvq_write_decode_noalloc(ctypes.byref(lay), ctypes.byref(_cache()), FAKE,
                                            FAKE, FAKE, FAKE, FAKE, 0, 2048, 0.1, FAKE,
                                            None) == OK


def test_balanced_partition_rules():
    assert kvq.validate(_layout(partition=1), _cache(), 256, 100) == OK
    assert kvq.validate(_layout(partition=1), _cache(), 257, 100) == UNS     # > 256 rows
    assert kvq.validate(_layout(partition=2), _cache(), 2, 100) == INV
    lay4 = kvq.make_layout("int4", "channel", "token", 8, 2, 64, 16, partition="balanced")
    assert kvq.validate(lay4, _cache(int4=True), 2, 100) == UNS              # KIVI caches
    # the plan: ragged rows that fit one round go balanced; KIVI never
    lay = kvq.make_layout("fp8", "head", "head", 32, 8, 20000, 1024)
    lens = [1024, 16384] + [2000] * 30
    assert kvq.plan_partition(lay, lens) == kvq.PARTITION_BALANCED
    lay4 = kvq.make_layout("int4", "channel", "token", 32, 8, 20000, 1024)
    assert kvq.plan_partition(lay4, lens) == kvq.PARTITION_PER_ROW
    # short rows (several rounds of per-row workgroups) stay per row
    lay2 = kvq.make_layout("int8", "token", "token", 32, 32, 512, 128)
    assert kvq.plan_partition(lay2, [2048] * 4) == kvq.PARTITION_PER_ROW
    assert kvq.plan_partition(lay2, []) == kvq.PARTITION_PER_ROW
