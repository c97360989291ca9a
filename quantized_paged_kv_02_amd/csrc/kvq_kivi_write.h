// KIVI-grouped quantize-on-write steps shared by the write kernels and the
// decode kernel's one-step path (kvq_write_decode): the flush of a 64-token
// group out of the fp16 window into packed codes and scales (one 256-thread
// workgroup per (row, group, KV head, K or V)) and the append of a new token
// to the fp16 ring (one wavefront).
//
// Groups follow [oh-bug] "KV Cache Quantization 生产实战", sections "Key 和
// Value 的分布不一定相同" (K per channel, V per token) and "Transformers：适合
// 实验和小规模验证" (group 64, residual 128); the affine form is that page's
// "量化不是简单'截断精度'".
#pragma once

#include "kvq_args.h"
#include "kvq_device.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

// New tokens of row b: entries [c_begin, c_begin + n_new) of k_new / v_new.
// Without cu_new every row owns entry b and holds one new token unless the
// row is empty.
__device__ __forceinline__ void new_tokens(const WriteArgs &a, int b, int &c_begin, int &n_new) {
  if (a.cu_new != nullptr) {
    c_begin = a.cu_new[b];
    n_new = a.cu_new[b + 1] - c_begin;
  } else {
    c_begin = b;
    n_new = a.seq_lens[b] > 0 ? 1 : 0;
  }
}

__device__ __forceinline__ int kivi_len(int s, int residual) {
  return kivi_quantized_len(s, residual);
}

// Flush of one 64-token group leaving the fp16 window, for one (row, KV
// head) and one of K or V: 256 threads.  The group's fp16 values are
// gathered into LDS (from the ring for tokens already cached, else from the
// call's new tokens), the scales are reduced across threads, and every
// thread then quantizes exactly the 32 nibbles of one 16-byte unit of the
// block layout and writes it with one store.
//
// AFF: asymmetric groups ([oh-bug] "量化不是简单'截断精度'", the affine
// form): over the group's range widened to contain zero, scale = (hi - lo)
// / 15 and zero point = clamp(round(-lo / scale), 0, 15); codes are
// clamp(round(x / scale) + zero point, 0, 15), unsigned.  Scale rows are 40
// floats per (block, head), the last 32 bytes holding the zero points.
constexpr int kFlushRow = kHeadDim + 8;  // padded LDS row (fp16)

// A flush workgroup's LDS (AFF: affine, with the channel minima).  The
// decode kernel's flush workgroups lay it over the LDS the decode
// workgroups use for streaming and merging.
template <bool AFF>
struct alignas(16) FlushLds {
  f16 x[kGroup][kFlushRow];
  float part[4][kHeadDim];              // K: channel maxima of four 16-token slices
  float partn[AFF ? 4 : 1][kHeadDim];   // K affine: channel minima
  int phys[4];
};

// Affine parameters of a group with minimum lo <= 0 <= maximum hi, codes
// 0 .. qmax.
__device__ __forceinline__ float2 affine_params(float lo, float hi, float qmax) {
  const float s = (hi - lo) / qmax;
  const float z = s > 0.0f ? fminf(fmaxf(rintf(-lo / s), 0.0f), qmax) : 0.0f;
  return float2{s, z};
}
// The reciprocal a flush quantizes with (see rint_quotients; 0 for a zero
// scale, whose codes are 0 whatever the quotient).
__device__ __forceinline__ float recip(float s) { return s > 0.0f ? 1.0f / s : 0.0f; }

// DT: kInt4 (symmetric), kInt4Affine or kInt2Affine (2-bit codes: 512-byte
// chunks, the code layouts of kvq.h).  bx = 2 x (the call's g-th group of
// row b) + (0: K, 1: V); h: KV head.
template <int DT>
__device__ void int4_flush(const WriteArgs &a, int bx, int h, int b,
                           FlushLds<DT != kInt4> &lds) {
  constexpr bool AFF = DT != kInt4;
  constexpr bool TWO = DT == kInt2Affine;
  constexpr float kQmax = TWO ? 3.0f : 15.0f;
  constexpr int kChunk = kivi_chunk_bytes(DT);
  constexpr int kRow = AFF ? 40 : 32;   // floats per (block, head) scale row
  auto &x = lds.x;
  auto &part = lds.part;
  auto &partn = lds.partn;
  int *const phys_s = lds.phys;
  // Scales, their reciprocals and (affine) kRoundAddend + zero points, K:
  // [128] per channel, V: [64][2] per token and channel group.  They reuse
  // part's rows: a K thread writes its channel's entries after reading that
  // channel's partial maxima, and no other thread reads them before the
  // next barrier (the smaller footprint keeps 7 affine workgroups per CU).
  float *const sc = part[0];
  float *const rc = part[1];
  float *const zs = part[2];

  const int gs = bx >> 1;
  const bool is_v = (bx & 1) != 0;
  const int tid = threadIdx.x;
  const int H = a.num_kv_heads;
  int c_begin, n_new;
  new_tokens(a, b, c_begin, n_new);
  const int s_new = a.seq_lens[b];
  const int s_old = s_new - n_new;
  // A row of length S keeps groups [0, nq(S + 1)) quantized: the group
  // that leaves the window at the next length is flushed one write early
  // (its tokens are all at least R positions old, already in the ring, and
  // no decode at length S reads its codes), so a one-token decode step can
  // flush concurrently with its own attention.  A write that grows a row
  // from S_old to S_new flushes [nq(S_old + 1), nq(S_new + 1)).
  const int nq_old = kivi_len(s_old + 1, a.residual);
  const int nq_new = kivi_len(s_new + 1, a.residual);
  const int t0 = nq_old + kGroup * gs;
  if (t0 >= nq_new) return;

  const size_t ring_row = (size_t)b * H + h;
  const uint16_t *fresh = is_v ? a.v_new : a.k_new;
  if (t0 >= s_old) {
    // every token of the group is new (a prefill write): K and V alike in
    // 16-byte units (token, 8 channels), all four loads of a thread first
    u32x4 g[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = tid + 256 * k;
      g[k] = ld16(fresh + ((size_t)(c_begin + t0 + (e >> 4) - s_old) * H + h) * kHeadDim +
                  (e & 15) * 8);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = tid + 256 * k;
      *reinterpret_cast<u32x4 *>(&x[e >> 4][(e & 15) * 8]) = g[k];
    }
  } else if (!is_v) {
    // K: 16-byte units (token, 8 channels); ring rows are contiguous
    for (int e = tid; e < kGroup * 16; e += 256) {
      const int tt = e >> 4, c8 = (e & 15) * 8;
      const int t = t0 + tt;
      const uint16_t *src =
          t < s_old ? a.k_resid + (ring_row * a.ring + t % a.ring) * kHeadDim + c8
                    : fresh + ((size_t)(c_begin + t - s_old) * H + h) * kHeadDim + c8;
      *reinterpret_cast<u32x4 *>(&x[tt][c8]) = ld16(src);
    }
  } else {
    // V: the ring is token-minor in quads ([slot/4][channel][slot%4]); a
    // 16-byte unit is 2 channels x 4 tokens of one quad
    for (int e = tid; e < (kGroup / 4) * (kHeadDim / 2); e += 256) {
      const int q = e >> 6, cp = e & 63;
      const int tq = t0 + 4 * q;
      if (tq + 3 < s_old) {
        const int slot = tq % a.ring;  // multiple of 4: the quad is contiguous
        const u32x4 w = ld16(a.v_resid + ((ring_row * (a.ring / 4) + slot / 4) * kHeadDim +
                                          2 * cp) * 4);
        // w = [c0 t0..t3][c1 t0..t3] as fp16 pairs
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
          const uint32_t hi = (i & 1) ? (w[2 + (i >> 1)] >> 16) : (w[2 + (i >> 1)] & 0xFFFFu);
          *reinterpret_cast<uint32_t *>(&x[4 * q + i][2 * cp]) = lo | (hi << 16);
        }
      } else {
        for (int i = 0; i < 4; ++i) {
          const int t = tq + i;
          uint32_t pr;
          if (t < s_old) {
            const int slot = t % a.ring;
            const uint16_t *vb = a.v_resid +
                                 ((ring_row * (a.ring / 4) + slot / 4) * kHeadDim + 2 * cp) * 4 +
                                 (slot & 3);
            pr = (uint32_t)vb[0] | ((uint32_t)vb[4] << 16);
          } else {
            pr = *reinterpret_cast<const uint32_t *>(
                fresh + ((size_t)(c_begin + t - s_old) * H + h) * kHeadDim + 2 * cp);
          }
          *reinterpret_cast<uint32_t *>(&x[4 * q + i][2 * cp]) = pr;
        }
      }
    }
  }
  if (tid < 4) {
    phys_s[tid] = a.block_tables[(size_t)b * a.max_blocks_per_seq + t0 / kBlock + tid];
  }
  __syncthreads();

  if (!is_v) {
    // K scales: max over the group's 64 tokens of |K[:, c]| / 7 (affine: the
    // channel's minimum and maximum, each starting from 0)
    {
      // maxima and minima of fp16 values are exact in packed fp16
      const int cp = tid & 63, qq = tid >> 6;
      f16x2 m = {(f16)0.0f, (f16)0.0f}, n = m;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const f16x2 v = *reinterpret_cast<const f16x2 *>(&x[16 * qq + i][2 * cp]);
        if constexpr (AFF) {
          m = __builtin_elementwise_max(m, v);
          n = __builtin_elementwise_min(n, v);
        } else {
          m = __builtin_elementwise_max(m, __builtin_elementwise_abs(v));
        }
      }
      part[qq][2 * cp] = (float)m.x;
      part[qq][2 * cp + 1] = (float)m.y;
      if constexpr (AFF) {
        partn[qq][2 * cp] = (float)n.x;
        partn[qq][2 * cp + 1] = (float)n.y;
      }
    }
    __syncthreads();
    if (tid < kHeadDim) {
      const float mx = fmaxf(fmaxf(part[0][tid], part[1][tid]), fmaxf(part[2][tid], part[3][tid]));
      float *row = a.k_scales + ((size_t)phys_s[tid >> 5] * H + h) * kRow;
      if constexpr (AFF) {
        const float mn =
            fminf(fminf(partn[0][tid], partn[1][tid]), fminf(partn[2][tid], partn[3][tid]));
        const float2 sz = affine_params(mn, mx, kQmax);
        sc[tid] = sz.x;
        rc[tid] = recip(sz.x);
        zs[tid] = kRoundAddend + sz.y;
        row[tid & 31] = sz.x;
        reinterpret_cast<uint8_t *>(row + 32)[tid & 31] = (uint8_t)(int)sz.y;
      } else {
        sc[tid] = mx / 7.0f;
        rc[tid] = recip(mx / 7.0f);
        row[tid & 31] = mx / 7.0f;
      }
    }
    __syncthreads();
    // one unit: channels 32cb .. 32cb+31 of token tt; INT4: nibble e of dword
    // d is channel 32cb + 8d + e; 2-bit: bits 2e of dword d are channel
    // 32cb + 16d + e
    const int tt = tid >> 2, cb = tid & 3;
    uint8_t *chunk = a.k_codes + ((size_t)phys_s[tt >> 4] * H + h) * kChunk;
    if constexpr (TWO) {
      u32x2 out;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        float xv[16], sv[16], rv[16], zv[16];
        uint32_t qv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = 32 * cb + 16 * d + e;
          xv[e] = (float)x[tt][c];
          sv[e] = sc[c];
          rv[e] = rc[c];
          zv[e] = zs[c];
        }
        kivi_codes<16, true>(qv, xv, sv, rv, zv, kQmax);
        // byte k of a_f: the code of channel 4k + f (affine codes fill
        // their bytes' low bits exactly)
        uint32_t af[4];
#pragma unroll
        for (int f = 0; f < 4; ++f)
          af[f] = byte_pair<0>(qv[f], qv[4 + f]) | byte_pair<2>(qv[8 + f], qv[12 + f]);
        out[d] = af[0] | (af[1] << 2) | (af[2] << 4) | (af[3] << 6);
      }
      *reinterpret_cast<u32x2 *>(chunk + 128 * cb + 8 * (tt & 15)) = out;
    } else {
      u32x4 out;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const f16x8 v = *reinterpret_cast<const f16x8 *>(&x[tt][32 * cb + 8 * d]);
        float xv[8], sv[8], rv[8], zv[8];
        uint32_t qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 32 * cb + 8 * d + e;
          xv[e] = (float)v[e];
          sv[e] = sc[c];
          rv[e] = rc[c];
          zv[e] = AFF ? zs[c] : kRoundAddend;
        }
        kivi_codes<8, AFF>(qv, xv, sv, rv, zv, kQmax);
        // byte k: channel 2k in the low nibble, 2k + 1 in the high one
        const uint32_t lo = byte_pair<0>(qv[0], qv[2]) | byte_pair<2>(qv[4], qv[6]);
        const uint32_t hi = byte_pair<0>(qv[1], qv[3]) | byte_pair<2>(qv[5], qv[7]);
        out[d] = AFF ? lo | (hi << 4) : nibbles_of(lo, hi);
      }
      *reinterpret_cast<u32x4 *>(chunk + 256 * cb + 16 * (tt & 15)) = out;
    }
  } else {
    // V scales: per token, max over each 64-channel half of |V| / 7
    // (affine: the half's minimum and maximum, each starting from 0)
    {
      const int tt = tid >> 2, qq = tid & 3;
      f16x2 m2 = {(f16)0.0f, (f16)0.0f}, n2 = m2;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const f16x8 v = *reinterpret_cast<const f16x8 *>(&x[tt][32 * qq + 8 * d]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f16x2 w = {v[e], v[e + 1]};
          if constexpr (AFF) {
            m2 = __builtin_elementwise_max(m2, w);
            n2 = __builtin_elementwise_min(n2, w);
          } else {
            m2 = __builtin_elementwise_max(m2, __builtin_elementwise_abs(w));
          }
        }
      }
      float m = fmaxf((float)m2.x, (float)m2.y), mn = fminf((float)n2.x, (float)n2.y);
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      if constexpr (AFF) mn = fminf(mn, __shfl_xor(mn, 1, 64));
      if ((qq & 1) == 0) {
        const int k = 2 * (tt & 15) + (qq >> 1);  // [slot][channel group]
        float *row = a.v_scales + ((size_t)phys_s[tt >> 4] * H + h) * kRow;
        if constexpr (AFF) {
          const float2 sz = affine_params(mn, m, kQmax);
          sc[2 * tt + (qq >> 1)] = sz.x;
          rc[2 * tt + (qq >> 1)] = recip(sz.x);
          zs[2 * tt + (qq >> 1)] = kRoundAddend + sz.y;
          row[k] = sz.x;
          // zero points group-transposed: token 16b + 4u + e of the group
          // goes to the row of the group's block u, byte 8b + 2e + g
          const int s16 = tt & 15;
          float *zrow = a.v_scales + ((size_t)phys_s[s16 >> 2] * H + h) * kRow;
          reinterpret_cast<uint8_t *>(zrow + 32)[8 * (tt >> 4) + 2 * (s16 & 3) + (qq >> 1)] =
              (uint8_t)(int)sz.y;
        } else {
          const float s = m / 7.0f;
          sc[2 * tt + (qq >> 1)] = s;
          rc[2 * tt + (qq >> 1)] = recip(s);
          row[k] = s;
        }
      }
    }
    __syncthreads();
    // one unit u of block ub: channels 16j + m (j = 0..7) of the quad's four
    // tokens; dword w holds tiles 2w and 2w+1, token e of tile j at nibble
    // 2(j&1) + (e>>1) + 4(e&1)
    const int ub = tid >> 6, u = tid & 63;
    const int m = u & 15, quad = u >> 4;
    uint8_t *chunk = a.v_codes + ((size_t)phys_s[ub] * H + h) * kChunk;
    if constexpr (TWO) {
      // 2-bit: tile j, token e at dword (j % 4) / 2, byte 2 (j % 2) + e / 2,
      // bits 2 (j / 4) + 4 (e % 2).  pf[w][g][h]: the codes of dword w with
      // j / 4 = g and e % 2 = h, each in the low bits of its byte
      uint32_t pf[2][2][2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tt = 16 * ub + 4 * quad + e;
        float xv[8], sv[8], rv[8], zv[8];
        uint32_t qv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int g = j >> 2;
          xv[j] = (float)x[tt][16 * j + m];
          sv[j] = sc[2 * tt + g];
          rv[j] = rc[2 * tt + g];
          zv[j] = zs[2 * tt + g];
        }
        kivi_codes<8, true>(qv, xv, sv, rv, zv, kQmax);
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            // tiles 4g + 2w (bytes e / 2) and 4g + 2w + 1 (bytes 2 + e / 2)
            const uint32_t v = (e >> 1) ? byte_spread<1>(qv[4 * g + 2 * w], qv[4 * g + 2 * w + 1])
                                        : byte_spread<0>(qv[4 * g + 2 * w], qv[4 * g + 2 * w + 1]);
            if (e < 2) {
              pf[w][g][e & 1] = v;
            } else {
              pf[w][g][e & 1] |= v;
            }
          }
      }
      u32x2 out;
#pragma unroll
      for (int w = 0; w < 2; ++w)
        out[w] = pf[w][0][0] | (pf[w][1][0] << 2) | (pf[w][0][1] << 4) | (pf[w][1][1] << 6);
      *reinterpret_cast<u32x2 *>(chunk + 8 * u) = out;
    } else {
      // dword w (tiles 2w, 2w + 1): byte k low nibble = tile 2w + k % 2 of
      // token k / 2, high nibble = the same tile of token 2 + k / 2
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tt = 16 * ub + 4 * quad + e;
        const float s0 = sc[2 * tt], s1 = sc[2 * tt + 1];
        const float r0 = rc[2 * tt], r1 = rc[2 * tt + 1];
        const float z0 = AFF ? zs[2 * tt] : kRoundAddend;
        const float z1 = AFF ? zs[2 * tt + 1] : kRoundAddend;
        float xv[8], sv[8], rv[8], zv[8];
        uint32_t qv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xv[j] = (float)x[tt][16 * j + m];
          sv[j] = j < 4 ? s0 : s1;
          rv[j] = j < 4 ? r0 : r1;
          zv[j] = j < 4 ? z0 : z1;
        }
        kivi_codes<8, AFF>(qv, xv, sv, rv, zv, kQmax);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t v = (e & 1) ? byte_pair<2>(qv[2 * w], qv[2 * w + 1])
                                     : byte_pair<0>(qv[2 * w], qv[2 * w + 1]);
          uint32_t &dst = (e >> 1) ? hi[w] : lo[w];
          if (e & 1) {
            dst |= v;
          } else {
            dst = v;
          }
        }
      }
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) out[w] = AFF ? lo[w] | (hi[w] << 4) : nibbles_of(lo[w], hi[w]);
      *reinterpret_cast<u32x4 *>(chunk + 16 * u) = out;
    }
  }
}

// Store new token i of row b, head h in the fp16 ring (first wave of the
// workgroup) unless it is already part of a quantized group.
__device__ __forceinline__ void append_token(const WriteArgs &a, int i, int h, int b, int lane) {
  const int H = a.num_kv_heads;
  int c_begin, n_new;
  new_tokens(a, b, c_begin, n_new);
  if (i >= n_new) return;
  const int s_new = a.seq_lens[b];
  const int pos = s_new - n_new + i;
  if (pos < kivi_len(s_new, a.residual)) return;  // already quantized
  const int slot = pos % a.ring;
  const size_t ring_row = (size_t)b * H + h;
  const size_t src = ((size_t)(c_begin + i) * H + h) * kHeadDim + 2 * lane;
  const uint32_t kp = *reinterpret_cast<const uint32_t *>(a.k_new + src);
  const uint32_t vp = *reinterpret_cast<const uint32_t *>(a.v_new + src);
  *reinterpret_cast<uint32_t *>(a.k_resid + (ring_row * a.ring + slot) * kHeadDim +
                                2 * lane) = kp;
  uint16_t *vb = a.v_resid + ((ring_row * (a.ring / 4) + slot / 4) * kHeadDim + 2 * lane) * 4 +
                 (slot & 3);
  vb[0] = (uint16_t)(vp & 0xFFFFu);
  vb[4] = (uint16_t)(vp >> 16);
}

// Store the new tokens of row b, head h that stay in the fp16 window and
// fall in its x-th position quad (positions 4q .. 4q+3, q counted from the
// quad of the first such token; ring slots 4q % RING .. +3, contiguous as
// RING is a multiple of 4).  One wavefront, lane l: channels 2l and 2l + 1.
// A V ring row holds a quad's four tokens per channel, so each lane writes
// its two channels' four tokens as one 16-byte unit, merged with the
// slots' current contents where the quad is only partly new.  One
// workgroup per quad: no other workgroup of the launch touches its slots.
__device__ __forceinline__ void append_quad(const WriteArgs &a, int x, int h, int b, int lane) {
  const int H = a.num_kv_heads;
  int c_begin, n_new;
  new_tokens(a, b, c_begin, n_new);
  if (n_new <= 0) return;
  const int s_new = a.seq_lens[b];
  const int s_old = s_new - n_new;
  const int lo = max(s_old, kivi_len(s_new, a.residual));  // first position kept in fp16
  if (lo >= s_new) return;
  const int p0 = 4 * (lo / 4 + x);
  if (p0 >= s_new) return;
  const size_t ring_row = (size_t)b * H + h;
  const int slot0 = p0 % a.ring;
  uint16_t *vq = a.v_resid + ((ring_row * (a.ring / 4) + slot0 / 4) * kHeadDim + 2 * lane) * 4;
  // dwords: channel 2l tokens (0, 1), (2, 3); channel 2l + 1 tokens (0, 1), (2, 3)
  u32x4 vw = {0u, 0u, 0u, 0u};
  if (p0 < lo || p0 + 3 >= s_new) vw = ld16(vq);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pos = p0 + e;
    if (pos < lo || pos >= s_new) continue;
    const size_t src = ((size_t)(c_begin + pos - s_old) * H + h) * kHeadDim + 2 * lane;
    const uint32_t kp = *reinterpret_cast<const uint32_t *>(a.k_new + src);
    const uint32_t vp = *reinterpret_cast<const uint32_t *>(a.v_new + src);
    *reinterpret_cast<uint32_t *>(a.k_resid + (ring_row * a.ring + slot0 + e) * kHeadDim +
                                  2 * lane) = kp;
    const int sh = 16 * (e & 1);
    const uint32_t keep = ~(0xFFFFu << sh);
    vw[e >> 1] = (vw[e >> 1] & keep) | ((vp & 0xFFFFu) << sh);
    vw[2 + (e >> 1)] = (vw[2 + (e >> 1)] & keep) | ((vp >> 16) << sh);
  }
  *reinterpret_cast<u32x4 *>(vq) = vw;
}

}  // namespace
}  // namespace kvq
