"""Read the device cache layout documented in include/kvq.h back into a
logical [token, head, channel] view (test helper; numpy only).

Written from the header's byte-offset formulas, independently of both the
HIP kernels and the oracle.
"""

import numpy as np

S_IDX = np.arange(16)[:, None]
C_IDX = np.arange(128)[None, :]

# INT8 / FP8 chunks (2048 bytes per (block, head))
K8_OFF = (1024 * ((C_IDX >> 4) & 1) + 256 * (C_IDX >> 5) + 16 * S_IDX + (C_IDX & 15))
V8_OFF = (1024 * (C_IDX >> 6) + 256 * (S_IDX >> 2) + 16 * (C_IDX & 15)
          + 4 * ((C_IDX >> 4) & 3) + (S_IDX & 3))

# INT4 chunks (1024 bytes per (block, head)): byte offset and nibble
K4_BYTE = 256 * (C_IDX >> 5) + 16 * S_IDX + ((C_IDX & 31) >> 1)
K4_NIB = np.broadcast_to(C_IDX & 1, (16, 128))
_J = C_IDX >> 4
_U = (C_IDX & 15) + 16 * (S_IDX >> 2)
_W = _J >> 1
_E = S_IDX & 3
_P = 2 * (_J & 1) + (_E >> 1) + 4 * (_E & 1)
V4_BYTE = 16 * _U + 4 * _W + (_P >> 1)
V4_NIB = _P & 1

# FP16 chunks (4096 bytes = 2048 fp16 per (block, head)): element offsets
K16_OFF = (1024 * ((C_IDX >> 3) & 3) + 256 * (C_IDX >> 5) + 16 * S_IDX + 2 * (C_IDX & 7)) // 2
V16_OFF = (1024 * (C_IDX >> 5) + 256 * (S_IDX >> 2) + 16 * (C_IDX & 15)
           + 8 * ((C_IDX >> 4) & 1) + 2 * (S_IDX & 3)) // 2

# 2-bit chunks (512 bytes per (block, head)): byte offset and bit position
K2_BYTE = 128 * (C_IDX >> 5) + 8 * S_IDX + ((C_IDX & 31) >> 2)
K2_BIT = np.broadcast_to(2 * (C_IDX & 3), (16, 128))
_J2 = C_IDX >> 4
V2_BYTE = (8 * ((C_IDX & 15) + 16 * (S_IDX >> 2)) + 4 * ((_J2 & 3) >> 1) + 2 * (_J2 & 1)
           + ((S_IDX & 3) >> 1))
V2_BIT = 2 * (_J2 >> 2) + 4 * (S_IDX & 1)
assert sorted((4 * K2_BYTE + K2_BIT // 2).ravel().tolist()) == list(range(2048))
assert sorted((4 * V2_BYTE + V2_BIT // 2).ravel().tolist()) == list(range(2048))

assert sorted(K16_OFF.ravel().tolist()) == list(range(2048))
assert sorted(V16_OFF.ravel().tolist()) == list(range(2048))
assert sorted(K8_OFF.ravel().tolist()) == list(range(2048))
assert sorted(V8_OFF.ravel().tolist()) == list(range(2048))
assert sorted((2 * K4_BYTE + K4_NIB).ravel().tolist()) == list(range(2048))
assert sorted((2 * V4_BYTE + V4_NIB).ravel().tolist()) == list(range(2048))


def chunk8(pool_chunk, which):
    """[2048] uint8 chunk -> [16 slots, 128 channels] uint8 codes."""
    off = K8_OFF if which == "k" else V8_OFF
    return np.asarray(pool_chunk)[off]


def chunk16(pool_chunk, which):
    """[2048] fp16 chunk -> [16 slots, 128 channels] fp16 values."""
    off = K16_OFF if which == "k" else V16_OFF
    return np.asarray(pool_chunk)[off]


def chunk2(pool_chunk, which):
    """[512] uint8 chunk -> [16, 128] uint8 2-bit codes in [0, 3]."""
    byte = K2_BYTE if which == "k" else V2_BYTE
    bit = K2_BIT if which == "k" else V2_BIT
    b = np.asarray(pool_chunk).astype(np.int64)[byte]
    return ((b >> bit) & 3).astype(np.uint8)


def chunk4(pool_chunk, which, signed=True):
    """[1024] uint8 chunk -> [16, 128] int8 codes in [-8, 7] (unsigned:
    uint8 codes in [0, 15])."""
    byte = K4_BYTE if which == "k" else V4_BYTE
    nib = K4_NIB if which == "k" else V4_NIB
    b = np.asarray(pool_chunk).astype(np.int64)[byte]
    v = np.where(nib == 1, (b >> 4) & 0xF, b & 0xF)
    if not signed:
        return v.astype(np.uint8)
    return np.where(v >= 8, v - 16, v).astype(np.int8)


def logical_codes(pool, table_row, n_tokens, which, dtype):
    """pool [NB, H, bytes] -> codes [n_tokens, H, 128] (uint8 for INT8/FP8
    bit patterns, int8 for INT4, the fp16 values for an FP16 pool, the
    float32 values of a BF16 pool read as float32)."""
    pool = np.asarray(pool)
    h = pool.shape[1]
    kind = {"int4": np.int8, "fp16": np.float16, "bf16": np.float32}.get(dtype, np.uint8)
    out = np.zeros((n_tokens, h, 128), kind)   # int4-affine: uint8 codes 0..15
    for j in range((n_tokens + 15) // 16):
        phys = int(table_row[j])
        n = min(16, n_tokens - 16 * j)
        for hh in range(h):
            if dtype == "int4":
                c = chunk4(pool[phys, hh], which)
            elif dtype == "int4-affine":
                c = chunk4(pool[phys, hh], which, signed=False)
            elif dtype == "int2-affine":
                c = chunk2(pool[phys, hh], which)
            elif dtype in ("fp16", "bf16"):
                c = chunk16(pool[phys, hh], which)
            else:
                c = chunk8(pool[phys, hh], which)
            out[16 * j:16 * j + n, hh] = c[:n]
    return out


def logical_token_scales(scales, table_row, n_tokens):
    """per-token scales [NB, H, 16] -> [n_tokens, H]."""
    scales = np.asarray(scales)
    out = np.zeros((n_tokens, scales.shape[1]), np.float32)
    for j in range((n_tokens + 15) // 16):
        n = min(16, n_tokens - 16 * j)
        out[16 * j:16 * j + n] = scales[int(table_row[j]), :, :n].T
    return out


def int4_k_scales(k_scales, table_row, n_groups):
    """INT4 K scales [NB, H, 32] (affine: [NB, H, 40], scales first) ->
    [n_groups, H, 128]: block 4g+u holds channels 32u..32u+31 of group g."""
    k_scales = np.asarray(k_scales)
    h = k_scales.shape[1]
    out = np.zeros((n_groups, h, 128), np.float32)
    for g in range(n_groups):
        for u in range(4):
            out[g, :, 32 * u:32 * u + 32] = k_scales[int(table_row[4 * g + u]), :, :32]
    return out


def int4_v_scales(v_scales, table_row, n_tokens):
    """INT4 V scales [NB, H, 16, 2] (affine: [NB, H, 40], scales first) ->
    [n_tokens, H, 2]."""
    v_scales = np.asarray(v_scales)
    v_scales = v_scales.reshape(v_scales.shape[0], v_scales.shape[1], -1)[:, :, :32]
    v_scales = v_scales.reshape(v_scales.shape[0], v_scales.shape[1], 16, 2)
    out = np.zeros((n_tokens, v_scales.shape[1], 2), np.float32)
    for j in range((n_tokens + 15) // 16):
        n = min(16, n_tokens - 16 * j)
        out[16 * j:16 * j + n] = v_scales[int(table_row[j]), :, :n].transpose(1, 0, 2)
    return out


def _zp_bytes(rows):
    """[NB, H, 40] fp32 affine rows -> [NB, H, 32] uint8 zero points."""
    rows = np.ascontiguousarray(np.asarray(rows, np.float32))
    return rows[:, :, 32:40].copy().view(np.uint8)


def int4_k_zero_points(k_scales, table_row, n_groups):
    """Affine K zero points -> [n_groups, H, 128] (same block order as the
    scales)."""
    z = _zp_bytes(k_scales)
    out = np.zeros((n_groups, z.shape[1], 128), np.int64)
    for g in range(n_groups):
        for u in range(4):
            out[g, :, 32 * u:32 * u + 32] = z[int(table_row[4 * g + u])]
    return out


def int4_v_zero_points(v_scales, table_row, n_tokens):
    """Affine V zero points -> [n_tokens, H, 2] (n_tokens a multiple of 64):
    token 16b + 4u + e of group G is byte 8b + 2e + g of the row of the
    group's block u (logical block 4G + u)."""
    z = _zp_bytes(v_scales)
    out = np.zeros((n_tokens, z.shape[1], 2), np.int64)
    for t in range(n_tokens):
        grp, r = divmod(t, 64)
        b, s16 = divmod(r, 16)
        u, e = divmod(s16, 4)
        row = z[int(table_row[4 * grp + u])]
        out[t] = row[:, 8 * b + 2 * e:8 * b + 2 * e + 2]
    return out


def ring_tokens(k_resid, v_resid, row, tokens, ring):
    """fp16 ring contents for absolute positions ``tokens`` of ``row``:
    (K [n, H, 128], V [n, H, 128])."""
    k_resid = np.asarray(k_resid)
    v_resid = np.asarray(v_resid)
    slots = np.asarray(tokens) % ring
    k = k_resid[row][:, slots, :].transpose(1, 0, 2)
    v = v_resid[row][:, slots >> 2, :, slots & 3]      # [n, H, 128] after advanced idx
    if v.shape[0] != len(slots):
        v = v.transpose(1, 0, 2)
    return k, v
