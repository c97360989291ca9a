// Quantize-on-write kernels (and the plain scatter of an FP16 cache):
// INT8 / FP8 (E4M3, E5M2) per token vector, KIVI groups (INT4 symmetric,
// INT4 and 2-bit affine).
//
// INT8 / FP8: one wavefront per (new token, KV head) quantizes the token's K
// and V vectors (128 values each, two per lane; the rule is in kvq_quant.h)
// and scatters the codes into the block slot given by the block table.
//
// INT4 (KIVI-style, [oh-bug] "KV Cache Quantization 生产实战", sections
// "Key 和 Value 的分布不一定相同" and "Transformers：适合实验和小规模验证"):
// a 256-thread workgroup per (row, flushed 64-token group, KV head) gathers
// the group from the fp16 ring or from the new tokens, computes per-channel K
// scales over the 64 tokens and per-token V scales over 64-channel groups,
// and writes packed nibbles; a second kernel appends the remaining new tokens
// to the fp16 ring.
#include "kvq_args.h"
#include "kvq_device.h"
#include "kvq_kivi_write.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

template <int DT>
__global__ __launch_bounds__(64) void kvq_write_q8_kernel(WriteArgs a) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  int c_begin, n_new;
  new_tokens(a, b, c_begin, n_new);
  if (i >= n_new) return;
  const int pos = a.seq_lens[b] - n_new + i;
  const int c0 = 2 * lane;
  // every load first (block id, both input vectors, static scales): the
  // code stores below are byte stores, which may alias any of them
  const size_t src = ((size_t)(c_begin + i) * a.num_kv_heads + h) * kHeadDim;
  const uint32_t rk = reinterpret_cast<const uint32_t *>(a.k_new + src)[lane];
  const uint32_t rv = reinterpret_cast<const uint32_t *>(a.v_new + src)[lane];
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + pos / kBlock];
  float2 sk = {0.f, 0.f}, sv = {0.f, 0.f};
  if (a.k_gran != kPerToken) sk = static_scales(a.k_scales, a.k_gran, h, c0);
  if (a.v_gran != kPerToken) sv = static_scales(a.v_scales, a.v_gran, h, c0);
  const CodePair qk = quantize_pair<DT>(rk, a.k_gran, sk);
  const CodePair qv = quantize_pair<DT>(rv, a.v_gran, sv);

  const int slot = pos % kBlock;
  const size_t chunk = (size_t)phys * a.num_kv_heads + h;
  uint8_t *kc = a.k_codes + chunk * 2048;
  uint8_t *vc = a.v_codes + chunk * 2048;
  store_k_codes(kc, slot, lane, qk);
  store_v_codes(vc, slot, lane, qv);
  if (lane == 0) {
    const size_t tsi = chunk * kBlock + slot;
    if (a.k_gran == kPerToken) a.k_scales[tsi] = qk.scale;
    if (a.v_gran == kPerToken) a.v_scales[tsi] = qv.scale;
  }
}

// Codes of 8 values under their scales (the rule of quantize_pair: round
// half to even of the IEEE quotient x / s, INT8 clamped to [-128, 127]; FP8
// clamped to the format's range then converted by the hardware, round to
// nearest even), byte i = value i, from r = 1 / s (correctly rounded; 0 for
// a zero scale) instead of a division per value.  The product p = x * r is
// within 2^-23 |x / s| of the quotient, whose own rounding is at most
// 2^-24 |x / s|.
// INT8: p clamped to [-128, 127] and rounded half to even by adding
// M = 1.5 * 2^23 (the integer lands in the low mantissa bits, whose byte is
// the two's-complement code).  For |x / s| <= 129 the two quotients differ
// by less than 2^-16, so they round alike unless p lies within 2^-14 of a
// half-integer; beyond that range both clamp to the same end code.
// FP8: the codes of p (1 - 2^-20) and p (1 + 2^-20), clamped, bracket both
// quotients, and rounding is monotonic: when the two codes agree, both
// quotients take that code.
// A wavefront with a value outside these windows, or with a scale whose
// reciprocal is not finite (FP8: or zero), divides instead.
template <int DT>
__device__ __forceinline__ u32x2 quantize8(const float (&x)[8], const float (&s)[8],
                                           const float (&r)[8]) {
  u32x2 w;
  bool near = false;
  if constexpr (DT == kInt8) {
    constexpr float M = 12582912.0f;  // 1.5 * 2^23
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = fminf(fmaxf(x[i] * r[i], -128.0f), 127.0f);
      t[i] = p + M;
      near |= !(fabsf(p - (t[i] - M)) < 0.5f - 0x1p-14f) || !(fabsf(r[i]) < 0x1p127f);
    }
    if (__any(near)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        t[i] = (s[i] != 0.0f ? fminf(fmaxf(rintf(x[i] / s[i]), -128.0f), 127.0f) : 0.0f) + M;
    }
#pragma unroll
    for (int hw = 0; hw < 2; ++hw) {
      const uint32_t *b = reinterpret_cast<const uint32_t *>(t + 4 * hw);
      const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);  // bytes n0, n1
      const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);  // bytes n2, n3
      w[hw] = lo | hi;
    }
  } else {
    constexpr float top = code_top<DT>();
    auto clamp = [](float v) { return fminf(fmaxf(v, -top), top); };
    auto cvt4 = [](const float (&v)[4]) {
      int pk;
      if constexpr (DT == kFp8) {
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
      } else {
        pk = __builtin_amdgcn_cvt_pk_bf8_f32(v[0], v[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_bf8_f32(v[2], v[3], pk, true);
      }
      return (uint32_t)pk;
    };
#pragma unroll
    for (int hw = 0; hw < 2; ++hw) {
      float lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * hw + e;
        const float p = x[i] * r[i];
        lo[e] = clamp(p * (1.0f - 0x1p-20f));
        hi[e] = clamp(p * (1.0f + 0x1p-20f));
        // a zero scale codes +0, which -0 * 0 would not give
        near |= !(fabsf(r[i]) < 0x1p127f) || r[i] == 0.0f;
      }
      w[hw] = cvt4(lo);
      near |= w[hw] != cvt4(hi);
    }
    if (__any(near)) {
#pragma unroll
      for (int hw = 0; hw < 2; ++hw) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fp8_prescale(x[4 * hw + e], s[4 * hw + e], top);
        w[hw] = cvt4(y);
      }
    }
  }
  return w;
}

// Maximum over the 16 lanes of a row (every lane gets it): quad swaps, then
// rotations by 4 and 8 within the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(0.0f, v));  // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f32<0x4E>(0.0f, v));  // quad_perm [2, 3, 0, 1]
  return bank_max(v);
}

// 1 / s, correctly rounded, and 0 for a zero scale
__device__ __forceinline__ float recip_or_zero(float s) { return s != 0.0f ? 1.0f / s : 0.0f; }

// INT8 / FP8 bulk write (prefill): one 256-thread workgroup per run of
// kWriteBlocks 16-token blocks of a row and one KV head, for the blocks'
// new tokens.  Thread t takes channels 8 (t % 16) .. + 7 of token slot
// t / 16 of every block (one 16-byte load of K and one of V per block, all
// issued first); a per-token scale is the maximum over the 16 threads of
// the slot (DPP within the 16-lane row); static scales and their
// reciprocals are taken once per workgroup.  Block by block, the codes go to
// LDS in the cache's byte order, then every thread stores one 16-byte unit
// of the (block, head) chunk (threads 0..127 K, 128..255 V): a K unit is 16
// channels of one token, a V unit 4 channels of 4 tokens, stored whole when
// all its tokens are new and byte by byte otherwise (the tokens already in
// the block keep their codes).
constexpr int kWriteBlocks = 4;

template <int DT>
__global__ __launch_bounds__(256) void kvq_write_q8_block_kernel(WriteArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[2][2048];  // K, V chunks
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  int c_begin, n_new;
  new_tokens(a, b, c_begin, n_new);
  const int s_new = a.seq_lens[b];
  const int s_old = s_new - n_new;
  const int lb0 = s_old / kBlock + (int)blockIdx.x * kWriteBlocks;  // first logical block
  if (n_new <= 0 || lb0 * kBlock >= s_new) return;
  const int slot = tid >> 4, k8 = tid & 15;
  // loads of every block first (tokens past the write read nothing)
  u32x4 rk[kWriteBlocks], rv[kWriteBlocks];
  int phys[kWriteBlocks];
#pragma unroll
  for (int j = 0; j < kWriteBlocks; ++j) {
    const int lb = lb0 + j;
    const int pos = lb * kBlock + slot;
    rk[j] = rv[j] = u32x4{0u, 0u, 0u, 0u};
    phys[j] = 0;
    if (lb * kBlock < s_new) {
      phys[j] = a.block_tables[(size_t)b * a.max_blocks_per_seq + lb];
      if (pos >= s_old && pos < s_new) {
        const size_t src =
            ((size_t)(c_begin + pos - s_old) * a.num_kv_heads + h) * kHeadDim + 8 * k8;
        rk[j] = ld16(a.k_new + src);
        rv[j] = ld16(a.v_new + src);
      }
    }
  }
  // static scales of this thread's channels and their reciprocals (per
  // token: set per block below)
  float ss[2][8], sr[2][8];
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const int gran = which ? a.v_gran : a.k_gran;
    const float *scales = which ? a.v_scales : a.k_scales;
    if (gran == kPerChannel) {
      const f32x4 s0 = ld16f(scales + h * kHeadDim + 8 * k8);
      const f32x4 s1 = ld16f(scales + h * kHeadDim + 8 * k8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss[which][e] = s0[e];
        ss[which][4 + e] = s1[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sr[which][e] = recip_or_zero(ss[which][e]);
    } else {
      const float st = gran == kPerToken ? 0.0f : scales[gran == kPerHead ? h : 0];
      const float rt = recip_or_zero(st);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss[which][e] = st;
        sr[which][e] = rt;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kWriteBlocks; ++j) {
    const int lb = lb0 + j;
    if (lb * kBlock >= s_new) break;  // uniform
    const int t_lo = max(lb * kBlock, s_old), t_hi = min(lb * kBlock + kBlock, s_new);
    const bool live = lb * kBlock + slot >= t_lo && lb * kBlock + slot < t_hi;
    const size_t chunk = (size_t)phys[j] * a.num_kv_heads + h;
    if (j > 0) __syncthreads();  // the previous block's units are stored
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const u32x4 raw = which ? rv[j] : rk[j];
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = half_bits_to_float(raw[e] & 0xFFFFu);
        x[2 * e + 1] = half_bits_to_float(raw[e] >> 16);
      }
      u32x2 q;
      if ((which ? a.v_gran : a.k_gran) == kPerToken) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
        m = row16_max(m);
        const float st = m / code_top<DT>();
        const float rt = recip_or_zero(st);
        const float sc[8] = {st, st, st, st, st, st, st, st};
        const float rc[8] = {rt, rt, rt, rt, rt, rt, rt, rt};
        q = quantize8<DT>(x, sc, rc);
        if (live && k8 == 0)
          (which ? a.v_scales : a.k_scales)[chunk * kBlock + slot] = st;
      } else {
        q = quantize8<DT>(x, ss[which], sr[which]);
      }
      if (which == 0) {
        // K: channels 8 k8 .. + 7 of the slot are 8 consecutive bytes
        *reinterpret_cast<u32x2 *>(&codes[0][1024 * ((k8 >> 1) & 1) + 256 * (k8 >> 2) +
                                             16 * slot + 8 * (k8 & 1)]) = q;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          codes[1][v8_offset(slot, 8 * k8 + e)] = (uint8_t)(q[e >> 2] >> (8 * (e & 3)));
      }
    }
    __syncthreads();
    const int u = tid & 127;
    if (tid < 128) {
      // K unit u: token slot u % 16
      const int upos = lb * kBlock + (u & 15);
      if (upos >= t_lo && upos < t_hi)
        *reinterpret_cast<u32x4 *>(a.k_codes + chunk * 2048 + 16 * u) =
            *reinterpret_cast<const u32x4 *>(&codes[0][16 * u]);
    } else {
      // V unit u: slots 4 ((u / 16) % 4) .. + 3, byte 4 i + e = slot e
      const int q0 = lb * kBlock + 4 * ((u >> 4) & 3);
      uint8_t *dst = a.v_codes + chunk * 2048 + 16 * u;
      if (q0 >= t_lo && q0 + 3 < t_hi) {
        *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(&codes[1][16 * u]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (q0 + e >= t_lo && q0 + e < t_hi) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[4 * i + e] = codes[1][16 * u + 4 * i + e];
          }
        }
      }
    }
  }
}

// FP16 (unquantized) cache: the same scatter with the values stored as they
// are, in the 4 KiB-per-(block, head) operand layout of kvq_quant.h.
__global__ __launch_bounds__(64) void kvq_write_f16_kernel(WriteArgs a) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  int c_begin, n_new;
  new_tokens(a, b, c_begin, n_new);
  if (i >= n_new) return;
  const int pos = a.seq_lens[b] - n_new + i;
  const size_t src = ((size_t)(c_begin + i) * a.num_kv_heads + h) * kHeadDim;
  const uint32_t rk = reinterpret_cast<const uint32_t *>(a.k_new + src)[lane];
  const uint32_t rv = reinterpret_cast<const uint32_t *>(a.v_new + src)[lane];
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + pos / kBlock];
  const size_t chunk = (size_t)phys * a.num_kv_heads + h;
  store_k_f16(a.k_codes + chunk * 4096, pos % kBlock, lane, rk);
  store_v_f16(a.v_codes + chunk * 4096, pos % kBlock, lane, rv);
}

// FP16 bulk write (prefill): one 256-thread workgroup per run of
// kWriteBlocks 16-token blocks of a row and one KV head, as the INT8/FP8
// block write.  Thread t holds channels 8 (t % 16) .. + 7 of token slot
// t / 16 of every block (one 16-byte load of K and one of V per block, all
// issued first).  K: those 8 channels are one 16-byte run of the chunk,
// stored directly when the token is new.  V: a 16-byte unit holds channels
// m and m + 16 of the four tokens of a slot quad; each block's V goes
// through LDS in the chunk's byte order, then every thread stores one unit
// (by halves for units whose tokens are not all new).
__global__ __launch_bounds__(256) void kvq_write_f16_block_kernel(WriteArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vlds[2048];  // one V chunk
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  int c_begin, n_new;
  new_tokens(a, b, c_begin, n_new);
  const int s_new = a.seq_lens[b];
  const int s_old = s_new - n_new;
  const int lb0 = s_old / kBlock + (int)blockIdx.x * kWriteBlocks;  // first logical block
  if (n_new <= 0 || lb0 * kBlock >= s_new) return;
  const int slot = tid >> 4, k8 = tid & 15;
  u32x4 rk[kWriteBlocks], rv[kWriteBlocks];
  int phys[kWriteBlocks];
#pragma unroll
  for (int j = 0; j < kWriteBlocks; ++j) {
    const int lb = lb0 + j;
    const int pos = lb * kBlock + slot;
    rk[j] = rv[j] = u32x4{0u, 0u, 0u, 0u};
    phys[j] = 0;
    if (lb * kBlock < s_new) {
      phys[j] = a.block_tables[(size_t)b * a.max_blocks_per_seq + lb];
      if (pos >= s_old && pos < s_new) {
        const size_t src =
            ((size_t)(c_begin + pos - s_old) * a.num_kv_heads + h) * kHeadDim + 8 * k8;
        rk[j] = ld16(a.k_new + src);
        rv[j] = ld16(a.v_new + src);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kWriteBlocks; ++j) {
    const int lb = lb0 + j;
    if (lb * kBlock >= s_new) break;  // uniform
    const int t_lo = max(lb * kBlock, s_old), t_hi = min(lb * kBlock + kBlock, s_new);
    const bool live = lb * kBlock + slot >= t_lo && lb * kBlock + slot < t_hi;
    const size_t chunk = (size_t)phys[j] * a.num_kv_heads + h;
    if (live)
      *reinterpret_cast<u32x4 *>(a.k_codes + chunk * 4096 + k16_offset(slot, 8 * k8)) = rk[j];
    if (j > 0) __syncthreads();  // the previous block's V units are stored
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vlds[v16_offset(slot, 8 * k8 + e) >> 1] =
          (uint16_t)((e & 1) ? (rv[j][e >> 1] >> 16) : (rv[j][e >> 1] & 0xFFFFu));
    __syncthreads();
    // unit tid: channels m, m + 16 (bytes 0..7, 8..15) of slots 4q .. 4q + 3
    const int q0 = lb * kBlock + 4 * ((tid >> 4) & 3);
    uint8_t *dst = a.v_codes + chunk * 4096 + 16 * tid;
    if (q0 >= t_lo && q0 + 3 < t_hi) {
      *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(&vlds[8 * tid]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (q0 + e >= t_lo && q0 + e < t_hi) {
          reinterpret_cast<uint16_t *>(dst)[e] = vlds[8 * tid + e];
          reinterpret_cast<uint16_t *>(dst)[4 + e] = vlds[8 * tid + 4 + e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// INT4 KIVI
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(256) void kvq_int4_flush_kernel(WriteArgs a) {
  __shared__ __attribute__((aligned(16))) FlushLds<DT != kInt4> lds;
  int4_flush<DT>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// Workgroup x stores the row's new fp16-window tokens in the x-th position
// quad they occupy (append_quad): a row keeps at most ring - 1 tokens in
// fp16 (S - nq(S) < R + G), so at most min(n_new, ring - 1) new tokens, in
// at most (min(n_new, ring) + 3) / 4 + 1 quads, land in the ring.
__global__ __launch_bounds__(64) void kvq_int4_append_kernel(WriteArgs a) {
  append_quad(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

// Flush and append in one launch: workgroups x < 2*groups flush, the rest
// append.  Only for calls that add at most one token per row: the appended
// token is then fewer than R + G positions after any token the flush reads
// from the ring, so its ring slot is never one of them.
template <int DT>
__global__ __launch_bounds__(256) void kvq_int4_flush_append_kernel(WriteArgs a, int groups) {
  __shared__ __attribute__((aligned(16))) FlushLds<DT != kInt4> lds;
  if ((int)blockIdx.x < 2 * groups) {
    int4_flush<DT>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
  } else if (threadIdx.x < 64) {
    append_token(a, blockIdx.x - 2 * groups, blockIdx.y, blockIdx.z, threadIdx.x);
  }
}

}  // namespace

hipError_t launch_write_q8(const WriteArgs &a, int dtype, int batch, int max_new,
                           hipStream_t stream) {
  if (max_new > 1) {
    // blocks a run of n tokens can touch: floor((n + 14) / 16) + 1
    const int blocks = (max_new + 14) / kBlock + 1;
    const dim3 grid((blocks + kWriteBlocks - 1) / kWriteBlocks, a.num_kv_heads, batch);
    if (dtype == kFp8) {
      hipLaunchKernelGGL(kvq_write_q8_block_kernel<kFp8>, grid, dim3(256), 0, stream, a);
    } else if (dtype == kFp8E5M2) {
      hipLaunchKernelGGL(kvq_write_q8_block_kernel<kFp8E5M2>, grid, dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL(kvq_write_q8_block_kernel<kInt8>, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
  }
  // one token per row (a decode step written apart from its decode)
  const dim3 grid(max_new, a.num_kv_heads, batch);
  if (dtype == kFp8) {
    hipLaunchKernelGGL(kvq_write_q8_kernel<kFp8>, grid, dim3(64), 0, stream, a);
  } else if (dtype == kFp8E5M2) {
    hipLaunchKernelGGL(kvq_write_q8_kernel<kFp8E5M2>, grid, dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(kvq_write_q8_kernel<kInt8>, grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_write_f16(const WriteArgs &a, int batch, int max_new, hipStream_t stream) {
  if (max_new > 1) {
    const int blocks = (max_new + 14) / kBlock + 1;  // blocks a run of max_new tokens can touch
    const dim3 grid((blocks + kWriteBlocks - 1) / kWriteBlocks, a.num_kv_heads, batch);
    hipLaunchKernelGGL(kvq_write_f16_block_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kvq_write_f16_kernel, dim3(max_new, a.num_kv_heads, batch), dim3(64), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_write_int4(const WriteArgs &a, int dtype, int batch, int max_new,
                             int max_flush_groups, hipStream_t stream) {
  if (max_new == 1 && max_flush_groups > 0) {
    const dim3 grid(2 * max_flush_groups + 1, a.num_kv_heads, batch);
    if (dtype == kInt2Affine) {
      hipLaunchKernelGGL(kvq_int4_flush_append_kernel<kInt2Affine>, grid, dim3(256), 0, stream,
                         a, max_flush_groups);
    } else if (dtype == kInt4Affine) {
      hipLaunchKernelGGL(kvq_int4_flush_append_kernel<kInt4Affine>, grid, dim3(256), 0, stream,
                         a, max_flush_groups);
    } else {
      hipLaunchKernelGGL(kvq_int4_flush_append_kernel<kInt4>, grid, dim3(256), 0, stream, a,
                         max_flush_groups);
    }
    return hipGetLastError();
  }
  if (max_flush_groups > 0) {
    const dim3 grid(2 * max_flush_groups, a.num_kv_heads, batch);
    if (dtype == kInt2Affine) {
      hipLaunchKernelGGL(kvq_int4_flush_kernel<kInt2Affine>, grid, dim3(256), 0, stream, a);
    } else if (dtype == kInt4Affine) {
      hipLaunchKernelGGL(kvq_int4_flush_kernel<kInt4Affine>, grid, dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL(kvq_int4_flush_kernel<kInt4>, grid, dim3(256), 0, stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kvq_int4_append_kernel,
                     dim3(((max_new < a.ring ? max_new : a.ring) + 3) / 4 + 1, a.num_kv_heads,
                          batch),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
