"""Algorithmic byte and flop counts of one decode step (host arithmetic only).

The decode step must read every cached code and scale of every attended
token, the fp16 residual tokens (INT4), the queries and the block-table
entries, and write the fp32 output.  Split-K workspace traffic and the
per-step quantize-on-write traffic are overhead and are not counted.

Each decode step streams the whole history ([oh-bug] "KV Cache
Quantization 生产实战", section "为什么长上下文更需要 KV Cache
Quantization"), so these bytes over the kernel time is the figure compared
with the HBM roofline.  Sizes follow the per-value byte counts of the
[oh-bug] section "KV Cache 的基本内存模型" (INT8/FP8 1 byte, INT4 half a
byte, FP16 2 bytes) plus the fp32 scales of each granularity (and the
one-byte zero points of the affine INT4 groups).
"""

from __future__ import annotations

HEAD_DIM = 128
BLOCK = 16
GROUP = 64


def kivi_quantized_len(s: int, residual: int) -> int:
    n = s - residual
    return (n // GROUP) * GROUP if n > 0 else 0


def _scale_bytes_uniform(gran: str, hkv: int) -> int:
    return {"tensor": 4, "head": 4 * hkv, "channel": 4 * hkv * HEAD_DIM}[gran]


def decode_bytes(dtype: str, k_gran: str, v_gran: str, lens, num_q_heads: int,
                 num_kv_heads: int, residual: int = 128) -> int:
    """Algorithmic bytes of one layer's decode over rows of lengths ``lens``."""
    hkv, hq, d = num_kv_heads, num_q_heads, HEAD_DIM
    b = len(lens)
    total = b * hq * d * 2 + b * hq * d * 4          # q fp16 (bf16) in, out fp32
    uniform_scales = 0
    for s in (int(x) for x in lens):
        if dtype in ("int4", "int4-affine", "int2-affine"):
            nq = kivi_quantized_len(s, residual)
            r = s - nq
            if dtype == "int2-affine":
                total += hkv * nq * d // 2            # K and V 2-bit codes: 2 x nq x d / 4
            else:
                total += hkv * nq * d                 # K and V nibbles: 2 x nq x d / 2
            total += hkv * (nq // GROUP) * d * 4      # K per-channel group scales
            total += hkv * nq * 2 * 4                 # V per-token scales, 2 groups
            if dtype != "int4":
                total += hkv * (nq // GROUP) * d      # K zero points, 1 byte each
                total += hkv * nq * 2                 # V zero points
            total += hkv * r * d * 2 * 2              # fp16 K and V residual
            total += (nq // BLOCK) * 4                # block-table entries
        elif dtype in ("fp16", "bf16"):
            total += 2 * hkv * s * d * 2              # K and V values, 2 bytes
            total += ((s + BLOCK - 1) // BLOCK) * 4
        else:
            total += 2 * hkv * s * d                  # K and V codes, 1 byte
            for gran in (k_gran, v_gran):
                if gran == "token":
                    total += hkv * s * 4
            total += ((s + BLOCK - 1) // BLOCK) * 4
    if dtype not in ("int4", "int4-affine", "int2-affine", "fp16", "bf16"):
        for gran in (k_gran, v_gran):
            if gran != "token":
                uniform_scales += _scale_bytes_uniform(gran, hkv)
    return total + uniform_scales


def decode_flops(lens, num_q_heads: int) -> int:
    """Multiply-adds of QK^T and PV counted as 2 flops each: 4 * D per
    (attended token, query head)."""
    return sum(4 * HEAD_DIM * num_q_heads * int(s) for s in lens)


def write_bytes(dtype: str, k_gran: str, v_gran: str, n_new: int, num_kv_heads: int) -> int:
    """Bytes of one INT8/FP8 quantize-on-write of ``n_new`` tokens: fp16 K/V
    read, codes (and per-token scales) written.  FP16 / BF16: K/V read and
    stored."""
    hkv, d = num_kv_heads, HEAD_DIM
    if dtype in ("fp16", "bf16"):
        return n_new * hkv * d * 2 * 2 * 2
    total = n_new * hkv * d * 2 * 2 + n_new * hkv * d * 2
    for gran in (k_gran, v_gran):
        if gran == "token":
            total += n_new * hkv * 4
    return total


def kivi_write_bytes(dtype: str, lens, num_kv_heads: int, residual: int = 128) -> int:
    """Bytes of a KIVI kvq_write that grows empty rows to lengths ``lens``:
    every new token's fp16 K and V read once; the INT4 (2-bit) codes, scales
    and zero points of the groups the write flushes (those below nq(S + 1):
    groups leave the window one token early) and the fp16 ring tokens
    written."""
    hkv, d = num_kv_heads, HEAD_DIM
    total = 0
    for s in (int(x) for x in lens):
        nq = kivi_quantized_len(s + 1, residual)
        total += s * hkv * d * 2 * 2                      # K and V read
        total += hkv * nq * d // (2 if dtype == "int2-affine" else 1)   # codes
        total += hkv * (nq // GROUP) * d * 4 + hkv * nq * 2 * 4         # scales
        if dtype != "int4":
            total += hkv * (nq // GROUP) * d + hkv * nq * 2             # zero points
        total += hkv * (s - kivi_quantized_len(s, residual)) * d * 2 * 2  # ring
    return total
