// Device-side helpers shared by the libkvq kernels (gfx950 only).
//
// Vector types for matrix-core operands, exact code -> fp16 conversions and
// wavefront reductions.  Conversions are written so that every code becomes
// the exact fp16 value of the integer (or E4M3 number) it encodes; scales are
// never applied per element here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kBlock = 16;
constexpr int kGroup = 64;        // INT4 group (tokens for K, channels for V)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t as_u32(f16x2 v) {
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) {
  return __builtin_bit_cast(f16x2, v);
}
// Two fp32 -> packed fp16 pair, rounding toward zero (v_cvt_pkrtz_f16_f32).
__device__ __forceinline__ uint32_t pack_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// --- INT8: 4 two's-complement codes in a dword -> 4 exact fp16 -------------
// Bias each byte to code+128 (xor 0x80), splice it under the fp16 exponent of
// 1024 (0x64 high byte: 1024 + u exactly) and subtract 1152.
__device__ __forceinline__ f16x4 int8x4_to_f16(uint32_t x) {
  const uint32_t u = x ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const f16x2 bias = {(f16)-1152.0f, (f16)-1152.0f};
  const f16x2 a = as_f16x2(lo) + bias;
  const f16x2 b = as_f16x2(hi) + bias;
  return f16x4{a.x, a.y, b.x, b.y};
}

// --- FP8 E4M3: 4 codes in a dword -> 4 exact fp16 (hardware OCP convert) ---
__device__ __forceinline__ f16x4 fp8x4_to_f16(uint32_t x) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  return f16x4{a.x, a.y, b.x, b.y};
}

// --- INT4: 8 nibbles in a dword -> 4 fp16 pairs (nibble s, nibble s+4) ------
// Bitwise select m ? (x ^ c) : c, one v_bitop3_b32: under the mask it biases
// the nibble to code+8 (xor of its top bit, carried in c); elsewhere it
// writes the fp16 exponent of 1024.  Low nibbles become 1024 + code + 8
// (subtract 1032); nibbles in the upper half of a byte become
// 1024 + 16 (code + 8) (times 1/16, minus 72).  All steps are exact.
__device__ __forceinline__ uint32_t bsel(uint32_t x, uint32_t m, uint32_t c) {
  return ((x ^ c) & m) | (c & ~m);
}

// (x & m) | c as one three-input bit operation (gfx950 v_bitop3_b32: bit i
// of the table is the result for inputs (x, m, c) = bits 2, 1, 0 of i).
// Written out, the compiler emits an AND and an OR with literal operands.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  return (uint32_t)__builtin_amdgcn_bitop3_b32(x, m, c, 0xEA);
}

__device__ __forceinline__ void int4x8_to_f16_pairs(uint32_t x, uint32_t out[4]) {
  const f16x2 sub = {(f16)-1032.0f, (f16)-1032.0f};
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 sub_hi = {(f16)-72.0f, (f16)-72.0f};
  const uint32_t y = x >> 8;
  out[0] = as_u32(as_f16x2(bsel(x, 0x000F000Fu, 0x64086408u)) + sub);
  out[1] = as_u32(as_f16x2(bsel(x, 0x00F000F0u, 0x64806480u)) * sixteenth + sub_hi);
  out[2] = as_u32(as_f16x2(bsel(y, 0x000F000Fu, 0x64086408u)) + sub);
  out[3] = as_u32(as_f16x2(bsel(y, 0x00F000F0u, 0x64806480u)) * sixteenth + sub_hi);
}

__device__ __forceinline__ f16x8 pairs_to_f16x8(const uint32_t p[4]) {
  const f16x2 a = as_f16x2(p[0]), b = as_f16x2(p[1]), c = as_f16x2(p[2]),
              d = as_f16x2(p[3]);
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// --- cross-lane helpers (wave64) --------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int m) {
  return __shfl_xor(v, m, 64);
}

// Reductions over the four lanes l, l^16, l^32, l^48 with the gfx950 row
// swaps (v_permlane16_swap / v_permlane32_swap exchange 16-lane rows and
// 32-lane halves between two registers; passing the value twice yields the
// value and its partner).
__device__ __forceinline__ float max_over_quads(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}
__device__ __forceinline__ float sum_over_quads(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

// DPP moves within 16-lane rows.  Row shift left by k: lane i reads lane
// i + k; right: lane i reads lane i - k; rotate right: lane i reads lane
// (i - k) mod 16.  Lanes whose source falls outside the row read zero.
// Bank b of a row is its lanes 4b .. 4b+3; lanes outside `bank_mask` keep
// `old`.
constexpr int kRowShl = 0x100, kRowShr = 0x110, kRowRor = 0x120;
template <int Ctrl, int BankMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src) {
  if constexpr ((Ctrl & 0xF) == 0) {
    return src;  // shift by zero
  } else {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, Ctrl, 0xF, BankMask, true);
  }
}
template <int Ctrl, int BankMask = 0xF>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return __builtin_bit_cast(
      float, dpp_u32<Ctrl, BankMask>(__builtin_bit_cast(uint32_t, old), __builtin_bit_cast(uint32_t, src)));
}
// max / sum over the four banks of a row (lanes i, i^4, i^8, i^12 share the
// result)
__device__ __forceinline__ float bank_max(float v) {
  v = fmaxf(v, dpp_f32<kRowRor + 4>(0.0f, v));
  return fmaxf(v, dpp_f32<kRowRor + 8>(0.0f, v));
}
__device__ __forceinline__ float bank_sum(float v) {
  v += dpp_f32<kRowRor + 4>(0.0f, v);
  return v + dpp_f32<kRowRor + 8>(0.0f, v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// --- matrix cores -----------------------------------------------------------
// D(16x16) += A(16x32) * B(32x16): lane l supplies row l%16 of A and column
// l%16 of B for k-slots 8*(l/16) .. +7; D row 4*(l/16)+i, column l%16 is
// element i of the result.
__device__ __forceinline__ f32x4 mfma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Raw buffer resource over `bytes` bytes at `base` (a wave-uniform address);
// bytes == 0 makes every load through it return zeros without touching
// memory, which lets a pipeline issue a fixed number of loads per step.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
// Buffer loads carry the non-temporal hint (cache policy bit nt): a decode
// launch reads each cache byte once, so its stream should not displace
// other lines from L2 (measured: 4-8 % faster launches, same results).
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}
__device__ __forceinline__ f32x4 bld16f(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}

// 16-byte global load (one dwordx4 per lane).
__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
// The same for data read once (non-temporal hint).
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ f32x4 ld16f(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}

__device__ __forceinline__ int kivi_quantized_len(int s, int residual) {
  const int n = s - residual;
  return n > 0 ? (n / kGroup) * kGroup : 0;
}

}  // namespace kvq
