"""Plain, slow, obviously-correct reference for quantized paged-KV decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the bench's CPU-baseline leg may use it.

Page tags used in citations:
  [yunthe]  "KV Cache量化压缩技术与vLLM推理引擎显存优化实战"
  [oh-bug]  "KV Cache Quantization 生产实战：用低精度缓存降低长上下文推理显存"
  [intelli] "大模型KV Cache显存优化与量化技术实践"

Conventions (readings of points the pages leave open are listed with the
function that takes them):
  * fp16 inputs are widened to fp32 exactly; scales are fp32.
  * quantization arithmetic is fp32: ``scale = amax / qmax`` and ``x / scale``
    are single IEEE fp32 divisions, rounding is half-to-even (``np.rint``).
  * attention is fp64 over ``code * scale`` (exact in fp64) or fp16 values.
  * query head ``hq`` reads KV head ``hq // (Hq // Hkv)``.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, printed page values, invariants or an independent
library routine.  None is "parity unpinned".
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "BLOCK_SIZE", "INT8_QMIN", "INT8_QMAX", "INT4_QMIN", "INT4_QMAX",
    "E4M3_MAX", "E5M2_MAX", "KIVI_GROUP", "KIVI_RESIDUAL", "BYTES_PER_VALUE",
    "e5m2_value", "e5m2_decode_table", "e5m2_encode", "quantize_e5m2",
    "calibrate_scales", "quant_divisor",
    "kv_cache_bytes", "absmax_scale", "quantize_int", "e4m3_value",
    "e4m3_decode_table", "e4m3_encode", "quantize_e4m3", "dequantize",
    "quantize_per_token", "quantize_static", "kivi_quantized_len",
    "kivi_quantize_k_group", "kivi_quantize_v_tokens", "pack_int4",
    "unpack_int4", "kivi_quantize", "kivi_dequantize", "INT4_UMAX",
    "affine_params", "quantize_affine", "kivi_affine_quantize_k_group",
    "kivi_affine_quantize_v_tokens", "decode_attention",
    "decode_attention_partials", "merge_partials", "paged_gather",
    "multi_query_attention",
    "paged_scatter",
]

# Paged KV blocks hold 16 tokens each ([yunthe], section
# "PagedAttention与KV Cache量化协同工作原理").
BLOCK_SIZE = 16

# Symmetric INT8 range and divisor ([intelli] §3.1 对称量化算法; [yunthe]
# section "KV Cache量化策略：INT8与FP8精度对比与选择").
INT8_QMAX = 127
INT8_QMIN = -128
# 4-bit codes by the same symmetric rule with 2**(4-1)-1 = 7 as divisor and a
# two's-complement nibble range ([oh-bug] bytes-per-value table, INT4 row;
# the symmetric rule is the INT8 one carried to 4 bits).
INT4_QMAX = 7
INT4_QMIN = -8
# Largest finite OCP E4M3 magnitude (1.75 * 2**8).
E4M3_MAX = 448.0
# Largest finite OCP E5M2 magnitude (1.75 * 2**15).
E5M2_MAX = 57344.0
# KIVI-style INT4 cache parameters ([oh-bug] section "Transformers：适合实验和
# 小规模验证": 4 bits, group 64, residual 128).
KIVI_GROUP = 64
KIVI_RESIDUAL = 128

# Bytes per cached value ([oh-bug] section "KV Cache 的基本内存模型", table).
BYTES_PER_VALUE = {
    "fp16": Fraction(2), "bf16": Fraction(2), "fp8": Fraction(1),
    "int8": Fraction(1), "int4": Fraction(1, 2), "int2": Fraction(1, 4),
}


# ---------------------------------------------------------------------------
# Sizes
# ---------------------------------------------------------------------------

def kv_cache_bytes(num_layers, num_kv_heads, head_dim, seq_len,
                   bytes_per_value, batch=1):
    """Bytes of a KV cache: 2 (K and V) x batch x layers x KV heads x head_dim
    x tokens x bytes per value.

    [intelli] §2.1 基础计算公式 (batch inside the product, KV heads under GQA);
    [oh-bug] section "KV Cache 的基本内存模型" (per request, times sequences).
    Returned as an exact ``Fraction`` so sub-byte formats stay exact.
    """
    return (2 * batch * num_layers * num_kv_heads * head_dim * seq_len
            * Fraction(bytes_per_value))


# ---------------------------------------------------------------------------
# Symmetric integer quantization
# ---------------------------------------------------------------------------

def absmax_scale(x, divisor, axis=None):
    """``scale = max|x| / divisor`` in IEEE fp32.

    [intelli] §3.1 对称量化算法 (max of |x| over the tensor, divided by 127);
    [yunthe] INT8/FP8 section (same formula).  Reading: the division is one
    correctly rounded fp32 division (the page's code divides in the input's
    precision; fp32 is the precision the scales are stored in).  ``axis``
    selects the extent (tensor, head, token, channel) the max runs over.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.size == 0:
        return np.float32(0.0)
    amax = np.max(np.abs(x), axis=axis)
    return (np.asarray(amax, np.float32) / np.float32(divisor)).astype(np.float32)


def quantize_int(x, scale, qmin, qmax):
    """``q = clamp(round(x / scale), qmin, qmax)`` with fp32 division and
    round-half-to-even.

    [intelli] §3.1 对称量化算法 (``torch.round`` then clamp to [-128, 127]);
    [yunthe] INT8/FP8 section (``q = round(x / scale)``).
    Reading for a zero scale (an all-zero vector under dynamic scaling, which
    the pages do not address): every code is 0.
    ``scale`` broadcasts against ``x``.
    """
    x = np.asarray(x, dtype=np.float32)
    scale = np.asarray(scale, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = x / scale
    q = np.clip(np.rint(y), qmin, qmax)
    q = np.where(np.broadcast_to(scale, q.shape) == 0, 0.0, q)
    return q.astype(np.int8)


# ---------------------------------------------------------------------------
# OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; the
# all-ones exponent with all-ones mantissa is NaN, there is no infinity).
# FP8 cache storage with a runtime scale: [yunthe] INT8/FP8 section; FP8 with
# a scale and no zero point: [oh-bug] section "量化不是简单'截断精度'".
# ---------------------------------------------------------------------------

def e4m3_value(code):
    """Real value of one E4M3 byte, from the format definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = man * 2.0 ** -9          # subnormal: man/8 * 2**(1-7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


def e4m3_decode_table():
    """All 256 E4M3 codes as float64 (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y):
    """Round fp32 values in [-448, 448] to the nearest E4M3 code, ties to the
    even mantissa, keeping the sign of zero.

    Written from the format: in the normal range [2**-6, 448] the spacing of
    representable values in [2**e, 2**(e+1)) is 2**(e-3); below 2**-6 it is
    2**-9 (subnormals).  Rounding |y| to a multiple of that spacing with
    half-to-even gives the nearest value; an even multiple is an even
    mantissa.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.abs(y) > E4M3_MAX) or np.any(np.isnan(y)):
        raise ValueError("e4m3_encode expects finite values clamped to +-448")
    a = np.abs(y).astype(np.float64)
    neg = np.signbit(y)
    _, k = np.frexp(a)                         # a = f * 2**k, f in [0.5, 1)
    e = np.maximum(k - 1, -6)                  # floor(log2 a), floored at -6
    quantum = np.ldexp(1.0, e - 3)
    n = np.rint(a / quantum)                   # exact scaling, RNE
    v = n * quantum                            # representable magnitude
    # bits of v
    _, kv = np.frexp(v)
    ev = kv - 1
    normal = v >= 2.0 ** -6
    man_norm = np.where(normal, v / np.ldexp(1.0, np.where(normal, ev, 0)) * 8 - 8, 0)
    code_norm = ((ev + 7) << 3) | man_norm.astype(np.int64)
    code_sub = (v / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_norm, code_sub).astype(np.int64)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def e5m2_value(code):
    """Real value of one OCP E5M2 byte (1 sign, 5 exponent bits with bias 15,
    2 mantissa bits; exponent 31 is infinity or NaN), from the format
    definition.  [yunthe] section "KV Cache量化策略：INT8与FP8精度对比与选择"
    names E4M3 and E5M2 as the two FP8 formats."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 2) & 0x1F
    man = code & 0x3
    if exp == 0x1F:
        return sign * float("inf") if man == 0 else float("nan")
    if exp == 0:
        mag = man * 2.0 ** -16         # subnormal: man/4 * 2**(1-15)
    else:
        mag = (1.0 + man / 4.0) * 2.0 ** (exp - 15)
    return sign * mag


def e5m2_decode_table():
    """All 256 E5M2 codes as float64 (+-inf and NaN where the format has them)."""
    return np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)


def e5m2_encode(y):
    """Round fp32 values in [-57344, 57344] to the nearest E5M2 code, ties to
    the even mantissa, keeping the sign of zero.

    Normal values in [2**e, 2**(e+1)), e >= -14, are spaced 2**(e-2); below
    2**-14 the spacing is 2**-16.  Rounding |y| to a multiple of the spacing
    with half-to-even gives the nearest representable value.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.abs(y) > E5M2_MAX) or np.any(np.isnan(y)):
        raise ValueError("e5m2_encode expects finite values clamped to +-57344")
    a = np.abs(y).astype(np.float64)
    neg = np.signbit(y)
    _, k = np.frexp(a)
    e = np.maximum(k - 1, -14)                 # floor(log2 a), floored at -14
    quantum = np.ldexp(1.0, e - 2)
    v = np.rint(a / quantum) * quantum         # representable magnitude
    _, kv = np.frexp(v)
    ev = kv - 1
    normal = v >= 2.0 ** -14
    man_norm = np.where(normal, v / np.ldexp(1.0, np.where(normal, ev, 0)) * 4 - 4, 0)
    code_norm = ((ev + 15) << 2) | man_norm.astype(np.int64)
    code_sub = (v / 2.0 ** -16).astype(np.int64)
    code = np.where(normal, code_norm, code_sub).astype(np.int64)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def quantize_e5m2(x, scale):
    """E5M2 code of ``clamp(x / scale, -57344, 57344)`` (fp32 division); the
    E4M3 rule with E5M2's range (dynamic scale = amax / 57344); a zero scale
    gives +0 codes."""
    x = np.asarray(x, dtype=np.float32)
    scale = np.asarray(scale, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = x / scale
    zero = np.broadcast_to(scale, y.shape) == 0
    y = np.where(zero, np.float32(0.0), y)
    y = np.clip(y, np.float32(-E5M2_MAX), np.float32(E5M2_MAX)).astype(np.float32)
    return e5m2_encode(y)


def quantize_e4m3(x, scale):
    """E4M3 code of ``clamp(x / scale, -448, 448)`` (fp32 division).

    Reading of the pages' "FP8 with runtime scaling": the scale maps the
    tensor's range onto E4M3's (dynamic scale = amax / 448), values beyond
    the range saturate to +-448 and a zero scale gives +0 codes.
    """
    x = np.asarray(x, dtype=np.float32)
    scale = np.asarray(scale, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = x / scale
    zero = np.broadcast_to(scale, y.shape) == 0
    y = np.where(zero, np.float32(0.0), y)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode(y)


def dequantize(codes, scale, dtype):
    """``x_hat = code * scale`` in fp64 (exact).  [intelli] §3.1
    (``q_x.float() * scale``).  ``dtype`` is "int8", "int4", "fp8" (E4M3) or
    "fp8e5m2"."""
    scale = np.asarray(scale, dtype=np.float64)
    if dtype == "fp8":
        vals = e4m3_decode_table()[np.asarray(codes, np.uint8)]
    elif dtype == "fp8e5m2":
        vals = e5m2_decode_table()[np.asarray(codes, np.uint8)]
    else:
        vals = np.asarray(codes).astype(np.float64)
    return vals * scale


# ---------------------------------------------------------------------------
# Granularities for INT8 / FP8 caches
# ---------------------------------------------------------------------------

def quant_divisor(dtype):
    """The code range a scale maps max|x| onto: 127 (INT8), 448 (E4M3),
    57344 (E5M2)."""
    return {"int8": INT8_QMAX, "fp8": E4M3_MAX, "fp8e5m2": E5M2_MAX}[dtype]


_qdivisor = quant_divisor


def _quant(x, scale, dtype):
    if dtype == "int8":
        return quantize_int(x, scale, INT8_QMIN, INT8_QMAX)
    if dtype == "fp8":
        return quantize_e4m3(x, scale)
    if dtype == "fp8e5m2":
        return quantize_e5m2(x, scale)
    raise ValueError(dtype)


def calibrate_scales(x, gran, dtype, previous=None):
    """Static scales from calibration tokens ``x`` [T, Hkv, D] (fp16): the
    maximum of |x| over the tokens and, per granularity, over the channels
    ("head", shape [Hkv]) or over heads and channels too ("tensor", [1]);
    "channel" keeps [Hkv, D].  Scale = amax / divisor in fp32.

    [yunthe] sections "KV Cache量化策略" (scale = max(abs(x)) / 127) and
    "配置与启动参数" (per-layer K and V scales computed offline from
    calibration data); [oh-bug] vLLM section (per-tensor and per-head FP8
    scales from a random-token warmup or calibration data).  Reading: with
    ``previous`` (scales of earlier calibration batches) the result is the
    elementwise maximum, i.e. the scale of all batches together.
    """
    a = np.abs(np.asarray(x, dtype=np.float32))
    if gran == "channel":
        amax = a.max(axis=0)
    elif gran == "head":
        amax = a.max(axis=(0, 2))
    elif gran == "tensor":
        amax = np.array([a.max()], np.float32)
    else:
        raise ValueError(gran)
    s = (amax.astype(np.float32) / np.float32(quant_divisor(dtype))).astype(np.float32)
    if previous is not None:
        s = np.maximum(s, np.asarray(previous, np.float32).reshape(s.shape))
    return s


def quantize_per_token(x, dtype):
    """Dynamic per-token quantization of ``x`` [..., D]: one fp32 scale per
    token's vector (per KV head), ``scale = amax / 127`` (INT8) or
    ``amax / 448`` (E4M3).

    [intelli] §3.2 动态量化策略 (a scale for each token's K/V vector);
    [oh-bug] section "量化不是简单'截断精度'" (per-token granularity).
    Reading: the vector is one KV head's D values of one token, K and V
    separately.  Returns (codes [..., D], scales [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    s = absmax_scale(x, _qdivisor(dtype), axis=-1)
    return _quant(x, s[..., None], dtype), s


def quantize_static(x, scale, gran, dtype):
    """Quantize ``x`` [S, Hkv, D] with caller-given static fp32 scales.

    ``gran``: "tensor" (scale shape [1]), "head" ([Hkv]) or "channel"
    ([Hkv, D]).  [oh-bug] section "量化不是简单'截断精度'" (tensor, head,
    channel granularity); [intelli] §3.2 (static: one fixed scale).
    """
    x = np.asarray(x, dtype=np.float32)
    scale = np.asarray(scale, dtype=np.float32)
    if gran == "tensor":
        sb = scale.reshape(1, 1, 1)
    elif gran == "head":
        sb = scale.reshape(1, -1, 1)
    elif gran == "channel":
        sb = scale.reshape(1, scale.shape[0], scale.shape[1])
    else:
        raise ValueError(gran)
    return _quant(x, sb, dtype)


# ---------------------------------------------------------------------------
# KIVI-style INT4 cache ([oh-bug] sections "Key 和 Value 的分布不一定相同"
# and "Transformers：适合实验和小规模验证")
# ---------------------------------------------------------------------------

def kivi_quantized_len(seq_len, residual=KIVI_RESIDUAL, group=KIVI_GROUP):
    """Number of leading tokens held as INT4 for a sequence of ``seq_len``.

    Reading of "keep the most recent tokens in high precision with a fixed
    residual length" together with 64-token groups: whole groups are
    quantized while at least ``residual`` newer tokens remain, i.e.
    ``max(0, floor((S - R) / G)) * G``; the rest stay fp16 (between R and
    R + G - 1 of them once S >= R).
    """
    return max(0, (int(seq_len) - residual) // group) * group


def kivi_quantize_k_group(k_group):
    """K of one 64-token group and one KV head, [64, D] fp16 -> (codes [64, D]
    int8 in [-8, 7], scales [D] fp32): per-channel scale = max over the
    group's tokens of |K[:, c]| / 7.  [oh-bug] "Key 和 Value 的分布不一定相同"
    (keys per channel)."""
    k = np.asarray(k_group, np.float32)
    s = absmax_scale(k, INT4_QMAX, axis=0)
    return quantize_int(k, s[None, :], INT4_QMIN, INT4_QMAX), s


def kivi_quantize_v_tokens(v_tokens, group=KIVI_GROUP):
    """V rows [T, D] -> (codes [T, D], scales [T, D // group]): per-token
    scales over consecutive channel groups of ``group``.  [oh-bug] "Key 和
    Value 的分布不一定相同" (values per token) with the cache's group size."""
    v = np.asarray(v_tokens, np.float32)
    t, d = v.shape
    vg = v.reshape(t, d // group, group)
    s = absmax_scale(vg, INT4_QMAX, axis=-1)
    q = quantize_int(vg, s[..., None], INT4_QMIN, INT4_QMAX)
    return q.reshape(t, d), s


def pack_int4(codes):
    """Pack int4 codes along the last axis two per byte: element 2i in the low
    nibble, 2i+1 in the high nibble, two's complement ([oh-bug] table: 0.5
    byte per INT4 value).  The nibble order is this oracle's convention."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed):
    """Inverse of :func:`pack_int4`."""
    p = np.asarray(packed, np.uint8).astype(np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def kivi_quantize(k, v, residual=KIVI_RESIDUAL, group=KIVI_GROUP, affine=False, bits=4):
    """Quantize a whole sequence's K and V [S, Hkv, D] (fp16) KIVI-style.

    Returns a dict with
      nq        number of INT4 tokens,
      k_codes   [nq, Hkv, D] int8,  k_scales [nq // group, Hkv, D] fp32,
      v_codes   [nq, Hkv, D] int8,  v_scales [nq, Hkv, D // group] fp32,
      k_resid, v_resid  [S - nq, Hkv, D] fp16 (unchanged inputs).
    With ``affine`` the groups are quantized asymmetrically: codes are uint8
    in [0, 2**bits - 1] (``bits`` 4 or 2) and ``k_zp`` / ``v_zp`` (int64,
    shaped like the scales) hold the zero points.
    Each group depends only on its own 64 tokens, so quantizing the final
    state equals quantizing group by group as the sequence grows.
    """
    k = np.asarray(k, np.float16)
    v = np.asarray(v, np.float16)
    s_len, hkv, d = k.shape
    nq = kivi_quantized_len(s_len, residual, group)
    code_t = np.uint8 if affine else np.int8
    k_codes = np.zeros((nq, hkv, d), code_t)
    k_scales = np.zeros((nq // group, hkv, d), np.float32)
    k_zp = np.zeros((nq // group, hkv, d), np.int64)
    for gi in range(nq // group):
        for h in range(hkv):
            kg = k[gi * group:(gi + 1) * group, h, :]
            if affine:
                c, s, z = kivi_affine_quantize_k_group(kg, qmax=(1 << bits) - 1)
                k_zp[gi, h, :] = z
            else:
                c, s = kivi_quantize_k_group(kg)
            k_codes[gi * group:(gi + 1) * group, h, :] = c
            k_scales[gi, h, :] = s
    v_codes = np.zeros((nq, hkv, d), code_t)
    v_scales = np.zeros((nq, hkv, d // group), np.float32)
    v_zp = np.zeros((nq, hkv, d // group), np.int64)
    for h in range(hkv):
        if affine:
            c, s, z = kivi_affine_quantize_v_tokens(v[:nq, h, :], group, qmax=(1 << bits) - 1)
            v_zp[:, h, :] = z
        else:
            c, s = kivi_quantize_v_tokens(v[:nq, h, :], group)
        v_codes[:, h, :] = c
        v_scales[:, h, :] = s
    out = {"nq": nq, "k_codes": k_codes, "k_scales": k_scales,
           "v_codes": v_codes, "v_scales": v_scales,
           "k_resid": k[nq:].copy(), "v_resid": v[nq:].copy()}
    if affine:
        out["k_zp"] = k_zp
        out["v_zp"] = v_zp
    return out


# ---------------------------------------------------------------------------
# Asymmetric (affine) INT4 KIVI groups ([oh-bug] section "量化不是简单'截断精度'":
# the affine form X_q = round(X / scale) + zero_point, dequantized as
# (X_q - zero_point) * scale; the page's references name KIVI as an
# asymmetric scheme).  Same groups as the symmetric cache: K per channel over
# 64 tokens, V per token over 64 channels.
# ---------------------------------------------------------------------------

# unsigned 4-bit codes 0 .. 15
INT4_UMAX = 15


def affine_params(x, qmax, axis):
    """Scale and integer zero point of the groups of ``x`` reduced over
    ``axis``.

    The page gives the affine form but not how its two parameters are
    chosen.  Reading: the group's range is widened to contain zero (so zero
    is a code and the zero point an integer), ``lo = min(min x, 0)``,
    ``hi = max(max x, 0)``; ``scale = (hi - lo) / qmax`` and
    ``zero_point = clamp(round(-lo / scale), 0, qmax)``, fp32 arithmetic,
    round half to even.  A group of zeros has scale 0 and zero point 0.
    Returns (scale fp32, zero_point int64).
    """
    x = np.asarray(x, np.float32)
    lo = np.minimum(x.min(axis=axis), np.float32(0)).astype(np.float32)
    hi = np.maximum(x.max(axis=axis), np.float32(0)).astype(np.float32)
    scale = ((hi - lo).astype(np.float32) / np.float32(qmax)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    zp = np.rint((-lo).astype(np.float32) / safe)
    zp = np.where(scale > 0, np.clip(zp, 0, qmax), 0)
    return scale, zp.astype(np.int64)


def quantize_affine(x, scale, zero_point, qmax):
    """``q = clamp(round(x / scale) + zero_point, 0, qmax)`` (fp32 division,
    round half to even); a zero scale gives code 0.  ``scale`` and
    ``zero_point`` broadcast against ``x``.  Returns uint8 codes."""
    x = np.asarray(x, np.float32)
    s = np.asarray(scale, np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    q = np.rint(x / safe) + np.asarray(zero_point, np.float64)
    q = np.where(s > 0, np.clip(q, 0, qmax), 0)
    return q.astype(np.uint8)


def kivi_affine_quantize_k_group(k_group, qmax=INT4_UMAX):
    """K of one 64-token group and one KV head, [64, D] fp16 -> (codes [64,
    D] uint8 in [0, qmax], scales [D] fp32, zero points [D] int64), one
    (scale, zero point) per channel over the group's tokens.  qmax 15: 4-bit
    codes; 3: 2-bit ([oh-bug] table: 2-bit caches at 0.25 byte per value;
    KIVI's scheme, named in its references, is asymmetric 2-bit)."""
    k = np.asarray(k_group, np.float32)
    s, z = affine_params(k, qmax, axis=0)
    return quantize_affine(k, s[None, :], z[None, :], qmax), s, z


def kivi_affine_quantize_v_tokens(v_tokens, group=KIVI_GROUP, qmax=INT4_UMAX):
    """V rows [T, D] -> (codes [T, D] uint8, scales [T, D // group] fp32, zero
    points [T, D // group]): one (scale, zero point) per token and channel
    group."""
    v = np.asarray(v_tokens, np.float32)
    t, d = v.shape
    vg = v.reshape(t, d // group, group)
    s, z = affine_params(vg, qmax, axis=-1)
    q = quantize_affine(vg, s[..., None], z[..., None], qmax)
    return q.reshape(t, d), s, z


def kivi_dequantize(kv, group=KIVI_GROUP):
    """K_hat, V_hat [S, Hkv, D] fp64 from :func:`kivi_quantize` output: INT4
    tokens as code * scale (affine: (code - zero_point) * scale), residual
    tokens as their fp16 values."""
    nq = kv["nq"]
    hkv, d = kv["k_codes"].shape[1], kv["k_codes"].shape[2]
    # K: token t of group t // group uses that group's per-channel scales
    kc = kv["k_codes"].astype(np.float64).reshape(nq // group, group, hkv, d)
    if "k_zp" in kv:
        kc = kc - kv["k_zp"].astype(np.float64)[:, None, :, :]
    ks = kv["k_scales"].astype(np.float64)[:, None, :, :]
    k_hat_q = (kc * ks).reshape(nq, hkv, d)
    # V: channel c of a token uses the token's scale of channel group c // group
    vc = kv["v_codes"].astype(np.float64).reshape(nq, hkv, d // group, group)
    if "v_zp" in kv:
        vc = vc - kv["v_zp"].astype(np.float64)[..., None]
    vs = kv["v_scales"].astype(np.float64)[..., None]
    v_hat_q = (vc * vs).reshape(nq, hkv, d)
    k_hat = np.concatenate([k_hat_q, kv["k_resid"].astype(np.float64)], axis=0)
    v_hat = np.concatenate([v_hat_q, kv["v_resid"].astype(np.float64)], axis=0)
    assert k_hat.shape[0] == nq + kv["k_resid"].shape[0]
    return k_hat, v_hat


# ---------------------------------------------------------------------------
# Paging ([yunthe] "PagedAttention与KV Cache量化协同工作原理": fixed blocks of
# 16 tokens managed independently).  Token t of sequence b lives in physical
# block block_table[b][t // 16], slot t % 16.
# ---------------------------------------------------------------------------

def paged_scatter(pool, logical, block_table_row, seq_len):
    """Write ``logical`` [S, ...] into ``pool`` [NB, 16, ...] through one
    sequence's block table."""
    for t in range(seq_len):
        pool[block_table_row[t // BLOCK_SIZE], t % BLOCK_SIZE] = logical[t]
    return pool


def paged_gather(pool, block_table_row, seq_len):
    """Read a sequence's [S, ...] view out of ``pool`` [NB, 16, ...]."""
    out = np.empty((seq_len,) + pool.shape[2:], pool.dtype)
    for t in range(seq_len):
        out[t] = pool[block_table_row[t // BLOCK_SIZE], t % BLOCK_SIZE]
    return out


# ---------------------------------------------------------------------------
# Decode attention in fp64
# ---------------------------------------------------------------------------

def decode_attention(q, k_hat, v_hat, softmax_scale):
    """One decode step: ``out[hq] = softmax(k_hat[:, h] @ q[hq] * scale) @
    v_hat[:, h]`` with ``h = hq // (Hq // Hkv)``.

    [intelli] §6 Q1 (``softmax(q k^T / sqrt(head_dim))``; its "+0.01" is a
    constant shift that softmax ignores and is not applied); [oh-bug] section
    "为什么长上下文更需要 KV Cache Quantization" (every decode step reads the
    whole history).  q [Hq, D], k_hat/v_hat [S, Hkv, D]; every token
    0..S-1 is visible.  S == 0 gives zeros.
    """
    q = np.asarray(q, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    hq_n, d = q.shape
    s_len, hkv, _ = k_hat.shape
    g = hq_n // hkv
    out = np.zeros((hq_n, d), np.float64)
    if s_len == 0:
        return out
    for hq in range(hq_n):
        h = hq // g
        s = (k_hat[:, h, :] @ q[hq]) * softmax_scale
        s = s - s.max()
        p = np.exp(s)
        p = p / p.sum()
        out[hq] = p @ v_hat[:, h, :]
    return out


def multi_query_attention(q, k_hat, v_hat, softmax_scale):
    """Several new query tokens of one sequence over its cache: q [Nq, Hq,
    D] are the queries of the last Nq positions S - Nq .. S - 1 (their K/V
    already cached), and query j attends to tokens 0 .. S - Nq + j
    (causal).  Returns [Nq, Hq, D] in fp64; a query with no visible token
    (S - Nq + j < 0) gives zeros.

    The step beside decode that [oh-bug] sections "为什么长上下文更需要 KV
    Cache Quantization" and "常见误区" describe reading the whole cached
    history: speculative verification or chunked prefill over the quantized
    cache.  Reading: every query sees the full prefix up to and including
    its own position, as in causal self-attention.
    """
    q = np.asarray(q, np.float64)
    nq = q.shape[0]
    s_len = k_hat.shape[0]
    out = np.zeros(q.shape, np.float64)
    for j in range(nq):
        vis = s_len - nq + j + 1
        if vis > 0:
            out[j] = decode_attention(q[j], k_hat[:vis], v_hat[:vis], softmax_scale)
    return out


def decode_attention_partials(q, k_hat, v_hat, softmax_scale, bounds):
    """Split the token axis at ``bounds`` (list of (start, end)) and return
    per-partition (m [Hq], l [Hq], o [Hq, D]) with o unnormalised:
    m = max score, l = sum exp(s - m), o = sum exp(s - m) v."""
    q = np.asarray(q, np.float64)
    hq_n, d = q.shape
    hkv = k_hat.shape[1]
    g = hq_n // hkv
    parts = []
    for (a, b) in bounds:
        m = np.full(hq_n, -np.inf)
        l = np.zeros(hq_n)
        o = np.zeros((hq_n, d))
        for hq in range(hq_n):
            if b <= a:
                continue
            h = hq // g
            s = (k_hat[a:b, h, :] @ q[hq]) * softmax_scale
            m[hq] = s.max()
            p = np.exp(s - m[hq])
            l[hq] = p.sum()
            o[hq] = p @ v_hat[a:b, h, :]
        parts.append((m, l, o))
    return parts


def merge_partials(parts):
    """Log-sum-exp merge of partition partials into the normalised output:
    M = max m_p, w_p = exp(m_p - M), out = sum w_p o_p / sum w_p l_p."""
    ms = np.stack([p[0] for p in parts])          # [P, Hq]
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])         # [P, Hq, D]
    big = np.max(ms, axis=0)
    out = np.zeros(os_.shape[1:])
    for hq in range(ms.shape[1]):
        if not np.isfinite(big[hq]):
            continue
        w = np.where(np.isfinite(ms[:, hq]), np.exp(ms[:, hq] - big[hq]), 0.0)
        out[hq] = (w[:, None] * os_[:, hq, :]).sum(0) / (w * ls[:, hq]).sum()
    return out
