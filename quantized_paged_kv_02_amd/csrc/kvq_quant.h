// INT8 / FP8 quantize-on-write of one token vector, shared by the write
// kernel and the decode kernel's fused append.  Symmetric rule from
// [intelli] "大模型KV Cache显存优化与量化技术实践" §3.1 对称量化算法 and
// [yunthe] "KV Cache量化压缩技术与vLLM推理引擎显存优化实战", section
// "KV Cache量化策略：INT8与FP8精度对比与选择": scale = max|x| / 127 (448 for
// E4M3, 57344 for E5M2, the page's two FP8 formats), code = clamp(round(x /
// scale)); dynamic per-token scales follow
// [intelli] §3.2 动态量化策略.  fp32 division is the correctly rounded IEEE
// one (the library is built without fast-math); rounding is rintf
// (half-to-even).
#pragma once

#include "kvq_args.h"
#include "kvq_device.h"

namespace kvq {

constexpr int kPerTensor = 0, kPerHead = 1, kPerChannel = 2, kPerToken = 3;

// Byte offset of (slot s, channel c) inside an INT8/FP8 (block, head) chunk.
__device__ __forceinline__ int k8_offset(int s, int c) {
  return 1024 * ((c >> 4) & 1) + 256 * (c >> 5) + 16 * s + (c & 15);
}
__device__ __forceinline__ int v8_offset(int s, int c) {
  return 1024 * (c >> 6) + 256 * (s >> 2) + 16 * (c & 15) + 4 * ((c >> 4) & 3) +
         (s & 3);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(f16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t quant_int(float x, float s, float lo, float hi) {
  if (s == 0.0f) return 0u;
  float y = rintf(x / s);
  y = fminf(fmaxf(y, lo), hi);
  return (uint32_t)(int)y;
}

// KIVI group codes: round half to even of the IEEE fp32 quotient x / s, as
// the oracle computes it, from r = 1 / s (correctly rounded) without a
// division per value.  zm = M + z with M = 1.5 * 2^23 and z the affine zero
// point (0 for symmetric codes; M + z is exact).  t = fma(x, r, zm) rounds
// the product x * r to an integer n and adds it to zm, all in t's low
// mantissa bits (half to even: t's unit in the last place is 1);
// rem = fma(x, r, -n) is the product's distance to n.  For |x / s| <= 16
// the product x * r is within |x / s| 2^-23 <= 2^-19 of the quotient and
// the quotient's own rounding is at most 2^-20, so the two round to the same
// integer unless the product lies within 2^-18 of a half-integer; the test
// |rem| < 1/2 - 2^-17 leaves a margin for rem's own rounding.  If any lane
// of the wavefront fails it (or is not finite), the wavefront divides
// instead.  The codes are the low bits of t's bits (returned as `bits`):
// symmetric, the two's-complement low bits of n (a group's own scale keeps
// |n| <= qmax); affine, n + z clamped to [0, qmax], so the low byte is the
// code itself.  A zero scale (r = 0) gives n = 0, and its group's z is 0.
constexpr float kRoundAddend = 12582912.0f;  // 1.5 * 2^23
template <int N, bool AFF>
__device__ __forceinline__ void kivi_codes(uint32_t (&bits)[N], const float (&x)[N],
                                           const float (&s)[N], const float (&r)[N],
                                           const float (&zm)[N], float qmax) {
  constexpr float M = kRoundAddend;
  float t[N];
  bool near = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    t[i] = __builtin_fmaf(x[i], r[i], zm[i]);
    const float n = t[i] - zm[i];
    const float rem = __builtin_fmaf(x[i], r[i], -n);
    near |= !(fabsf(rem) < 0.5f - 0x1p-17f);
  }
  if (__any(near)) {
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = (s[i] != 0.0f ? rintf(x[i] / s[i]) : 0.0f) + zm[i];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float v = t[i];
    if constexpr (AFF) v = fminf(fmaxf(v, M), M + qmax);
    bits[i] = __builtin_bit_cast(uint32_t, v);
  }
}

// Byte gathers for packing codes (byte_pair<B>: the low bytes of a and b as
// bytes B and B + 1 of the result, zeros elsewhere; byte_spread<B>: as
// bytes B and B + 2).
template <int B>
__device__ __forceinline__ uint32_t byte_pair(uint32_t a, uint32_t b) {
  constexpr uint32_t z = 0x0C0C0C0Cu;  // selector 0x0C: a zero byte
  constexpr uint32_t sel = (z & ~(0xFFFFu << (8 * B))) | (0x0400u << (8 * B));
  return __builtin_amdgcn_perm(b, a, sel);
}
template <int B>
__device__ __forceinline__ uint32_t byte_spread(uint32_t a, uint32_t b) {
  constexpr uint32_t z = 0x0C0C0C0Cu;
  constexpr uint32_t sel = (z & ~((0xFFu << (8 * B)) | (0xFFu << (8 * B + 16)))) |
                           (0x00u << (8 * B)) | (0x04u << (8 * B + 16));
  return __builtin_amdgcn_perm(b, a, sel);
}
// Eight 4-bit codes (low nibbles of the bytes of lo, low nibbles of the
// bytes of hi; other bits ignored) as one dword: byte k = lo's byte k in
// its low nibble, hi's byte k in its high nibble.
__device__ __forceinline__ uint32_t nibbles_of(uint32_t lo, uint32_t hi) {
  return (lo & 0x0F0F0F0Fu) | ((hi << 4) & 0xF0F0F0F0u);
}

// x / s clamped to the format's finite range (448 E4M3, 57344 E5M2).
__device__ __forceinline__ float fp8_prescale(float x, float s, float top) {
  if (s == 0.0f) return 0.0f;
  const float y = x / s;
  return fminf(fmaxf(y, -top), top);
}

// max|x| divisor of a dynamic scale ([yunthe] section "KV Cache量化策略"):
// the largest code magnitude of the format
template <int DT>
constexpr float code_top() {
  return DT == kFp8 ? 448.0f : (DT == kFp8E5M2 ? 57344.0f : 127.0f);
}

// Codes of channels 2 lane, 2 lane + 1 of one tensor (K or V) of one
// (token, KV head), and the token's scale.
struct CodePair {
  uint32_t q0, q1;
  float scale;
};

// Scale of channels c0, c0 + 1 for the static granularities.
__device__ __forceinline__ float2 static_scales(const float *scales, int gran, int h, int c0) {
  if (gran == kPerTensor) return float2{scales[0], scales[0]};
  if (gran == kPerHead) return float2{scales[h], scales[h]};
  return float2{scales[h * kHeadDim + c0], scales[h * kHeadDim + c0 + 1]};
}

template <int DT>
__device__ __forceinline__ CodePair quantize_pair(uint32_t raw, int gran, float2 st) {
  const float x0 = half_bits_to_float(raw & 0xFFFFu);
  const float x1 = half_bits_to_float(raw >> 16);
  float s0 = st.x, s1 = st.y;
  if (gran == kPerToken) {
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    s0 = s1 = amax / code_top<DT>();
  }
  CodePair r;
  r.scale = s0;
  if (DT == kFp8) {
    const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        fp8_prescale(x0, s0, 448.0f), fp8_prescale(x1, s1, 448.0f), 0, false);
    r.q0 = pk & 0xFFu;
    r.q1 = (pk >> 8) & 0xFFu;
  } else if (DT == kFp8E5M2) {
    // OCP E5M2, round to nearest even (the hardware conversion)
    const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(
        fp8_prescale(x0, s0, 57344.0f), fp8_prescale(x1, s1, 57344.0f), 0, false);
    r.q0 = pk & 0xFFu;
    r.q1 = (pk >> 8) & 0xFFu;
  } else {
    r.q0 = quant_int(x0, s0, -128.0f, 127.0f) & 0xFFu;
    r.q1 = quant_int(x1, s1, -128.0f, 127.0f) & 0xFFu;
  }
  return r;
}

// Store codes of channels 2 lane, 2 lane + 1 at `slot` of a (block, head)
// chunk.  K: the two channels are adjacent bytes of one 16-byte run.
__device__ __forceinline__ void store_k_codes(uint8_t *chunk, int slot, int lane,
                                              const CodePair &q) {
  *reinterpret_cast<uint16_t *>(chunk + k8_offset(slot, 2 * lane)) = (uint16_t)(q.q0 | (q.q1 << 8));
}
__device__ __forceinline__ void store_v_codes(uint8_t *chunk, int slot, int lane,
                                              const CodePair &q) {
  chunk[v8_offset(slot, 2 * lane)] = (uint8_t)q.q0;
  chunk[v8_offset(slot, 2 * lane + 1)] = (uint8_t)q.q1;
}

// FP16 (unquantized) cache: byte offset of (slot s, channel c) inside a
// (block, head) chunk of 16 tokens x 128 channels x 2 bytes.
//   K: 1024*((c>>3)&3) + 256*(c>>5) + 16*s + 2*(c&7)
//   V: 1024*(c>>5) + 256*(s>>2) + 16*(c&15) + 8*((c>>4)&1) + 2*(s&3)
// Lane l of a wavefront then reads, with one 16-byte load per 1 KiB quarter,
// channels 32qd+8j..+7 of token l%16 (K, quarter j) and tokens 4qd..4qd+3
// of channels 32j+l%16 and 32j+16+l%16 (V, quarter j), qd = l/16: its
// matrix-core operands, as for the 8-bit layouts.
__device__ __forceinline__ int k16_offset(int s, int c) {
  return 1024 * ((c >> 3) & 3) + 256 * (c >> 5) + 16 * s + 2 * (c & 7);
}
__device__ __forceinline__ int v16_offset(int s, int c) {
  return 1024 * (c >> 5) + 256 * (s >> 2) + 16 * (c & 15) + 8 * ((c >> 4) & 1) + 2 * (s & 3);
}

// Store fp16 values of channels 2 lane, 2 lane + 1 (one dword of K; two
// halves of V) at `slot` of a 4 KiB (block, head) chunk.
__device__ __forceinline__ void store_k_f16(uint8_t *chunk, int slot, int lane, uint32_t pair) {
  *reinterpret_cast<uint32_t *>(chunk + k16_offset(slot, 2 * lane)) = pair;
}
__device__ __forceinline__ void store_v_f16(uint8_t *chunk, int slot, int lane, uint32_t pair) {
  *reinterpret_cast<uint16_t *>(chunk + v16_offset(slot, 2 * lane)) = (uint16_t)(pair & 0xFFFFu);
  *reinterpret_cast<uint16_t *>(chunk + v16_offset(slot, 2 * lane + 1)) = (uint16_t)(pair >> 16);
}

}  // namespace kvq
