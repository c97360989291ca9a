// Split-K paged decode attention over a quantized KV cache (gfx950).
//
// What is computed: for every batch row b and query head hq,
//   out = sum_t softmax_t(scale * q.k_hat_t) * v_hat_t   over t < seq_lens[b],
// with k_hat/v_hat = code * scale dequantized inside the kernel
// ([yunthe] "KV Cache量化压缩技术与vLLM推理引擎显存优化实战", section
// "PagedAttention与KV Cache量化协同工作原理": 16-token blocks, dequantization
// fused into the attention kernel; [intelli] "大模型KV Cache显存优化与量化技术
// 实践" §6 Q1 for the softmax(q k^T / sqrt(d)) form; [oh-bug] "KV Cache
// Quantization 生产实战", section "为什么长上下文更需要 KV Cache Quantization":
// each decode step streams the whole history, so the kernel is bound by HBM).
//
// Work decomposition: one wavefront (workgroup of 64) per (partition p, KV
// head h, row b).  A partition is `part_blocks` consecutive 16-token blocks
// (INT4: whole 64-token groups); INT4 adds one partition for the fp16
// residual ring.  Each wavefront keeps an online softmax (running max m in
// the log2 domain, running sum l, unnormalised output o) for the g query
// heads that share h, writes it as a partial, and the last partition of
// (b, h) to arrive merges all partials in partition order (log-sum-exp) and
// writes out.  Rows with a single partition write out directly.
//
// Matrix cores: scores S^T[token][head] = K[token][:] . Q^T[:][head] use
// v_mfma_f32_16x16x32_f16 (16 tokens x 16 head slots, g of them live); the
// value product O^T[channel][head] = V^T[channel][token] . P^T[token][head]
// uses v_mfma_f32_16x16x16_f16.  Both leave lane (head n = l%16, quad
// qd = l/16) owning tokens 4qd..4qd+3 of head n (scores) and channels
// 16j+4qd..+3 of head n (output), so softmax state, rescaling and the V-scale
// folding are lane-local.  The cache layout (kvq.h) gives every lane its
// operand bytes as one 16-byte run, loaded straight into registers.
//
// Scales are factored out of the contraction: per-token K scales multiply
// the 16 scores, uniform K scales fold into one multiplier, per-channel K
// scales (and INT4 group scales) fold into q, kept exact as an fp16 hi/lo
// pair; per-token V scales fold into p, uniform and per-channel V scales are
// applied to o once per partition.
#include "kvq_args.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();
// The running max is only moved when a score exceeds it by more than this
// (log2 units), so p <= 2^8 and rescaling of o is rare.
constexpr float kRescaleSlack = 8.0f;

struct Softmax {
  float m;       // running max (log2 domain), same on the 4 lanes of a head
  float l;       // this lane's share of the running sum
  f32x4 o[8];    // o^T rows 16j + 4qd + i for head n
};

__device__ __forceinline__ void softmax_init(Softmax &st) {
  st.m = kNegInf;
  st.l = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Fold one tile of 16 scores (4 per lane, log2 domain, masked = -inf) into
// the running state; returns p (relative to the updated max).
__device__ __forceinline__ f32x4 softmax_update(Softmax &st, f32x4 sc) {
  float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  bm = max_over_quads(bm);
  const bool need = bm > st.m + kRescaleSlack;
  if (__any(need)) {
    const float mn = need ? bm : st.m;
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - mn) : 1.0f;
    st.l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= alpha;
    st.m = mn;
  }
  f32x4 p;
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - st.m);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  return p;
}

__device__ __forceinline__ f16x4 to_f16x4(f32x4 v) {
  const f16x2 a = as_f16x2(pack_rtz(v[0], v[1]));
  const f16x2 b = as_f16x2(pack_rtz(v[2], v[3]));
  return f16x4{a.x, a.y, b.x, b.y};
}

// Split fp32 x into hi + lo fp16 parts (hi rounded toward zero, lo the
// rounded remainder): |x - hi - lo| <= 2^-22 |x|.
__device__ __forceinline__ void split_hi_lo(float x0, float x1, uint32_t &hi,
                                            uint32_t &lo) {
  hi = pack_rtz(x0, x1);
  const f16x2 h = as_f16x2(hi);
  const float r0 = x0 - (float)h.x;
  const float r1 = x1 - (float)h.y;
  lo = pack_rtz(r0, r1);
}

__device__ __forceinline__ f16x8 u4_to_f16x8(u32x4 v) {
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ f16x4 u2_to_f16x4(u32x2 v) {
  return __builtin_bit_cast(f16x4, v);
}

template <int DT>
__device__ __forceinline__ f16x4 codes4_to_f16(uint32_t w) {
  if constexpr (DT == kFp8) {
    return fp8x4_to_f16(w);
  } else {
    return int8x4_to_f16(w);
  }
}

// keep the first `n` bytes (0..4) of w
__device__ __forceinline__ uint32_t keep_bytes(uint32_t w, int n) {
  return n >= 4 ? w : (n <= 0 ? 0u : (w & ((1u << (8 * n)) - 1u)));
}

// Physical block ids of a partition, read 64 at a time into one vector
// register and handed out with readlane (uniform index), so the tile loads
// never wait on a dependent block-table load.
struct BlockIds {
  const int32_t *bt;
  int end, base, vec;
  // requires begin < stop; lanes past the end re-read the last entry
  __device__ BlockIds(const int32_t *table, int begin, int stop, int lane)
      : bt(table), end(stop), base(begin) {
    vec = table[min(begin + lane, stop - 1)];
  }
  __device__ __forceinline__ int get(int jb, int lane) {
    if (jb - base >= 64) {
      base = jb;
      vec = bt[min(base + lane, end - 1)];
    }
    return __builtin_amdgcn_readlane(vec, jb - base);
  }
};

// ---------------------------------------------------------------------------
// INT8 / FP8 block tile
// ---------------------------------------------------------------------------
struct Tile8 {
  u32x4 k0, k1;   // K bytes: channels 32qd+0..15 / +16..31 of token l%16
  u32x4 v0, v1;   // V bytes: 4 tokens x channels 16j + l%16, j = 0..3 / 4..7
  f32x4 ks, vs;   // per-token scales of tokens 4qd..4qd+3
};

template <int KS, int VS>
__device__ __forceinline__ void load_tile8(Tile8 &t, const DecodeArgs &a, int phys,
                                           int h, int lane, int qd) {
  const size_t chunk = (size_t)phys * a.num_kv_heads + h;
  const uint8_t *kc = a.k_codes + chunk * 2048 + 16 * lane;
  const uint8_t *vc = a.v_codes + chunk * 2048 + 16 * lane;
  t.k0 = ld16(kc);
  t.k1 = ld16(kc + 1024);
  t.v0 = ld16(vc);
  t.v1 = ld16(vc + 1024);
  if constexpr (KS == kToken) t.ks = ld16f(a.k_scales + chunk * kBlock + 4 * qd);
  if constexpr (VS == kToken) t.vs = ld16f(a.v_scales + chunk * kBlock + 4 * qd);
}

template <int DT, int KS, int VS, bool TAIL>
__device__ __forceinline__ void compute_tile8(Softmax &st, const Tile8 &t,
                                              const f16x8 (&bq)[4],
                                              const f16x8 (&bq_lo)[4], float kmul,
                                              int tok0, int seq_len, int qd) {
  // scores: MFMA j covers channels 32qd + 8j .. +7 (j = 2i + jj uses dwords
  // 2jj, 2jj+1 of load i)
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 &src = (j < 2) ? t.k0 : t.k1;
    const int jj = j & 1;
    const f16x4 a0 = codes4_to_f16<DT>(src[2 * jj]);
    const f16x4 a1 = codes4_to_f16<DT>(src[2 * jj + 1]);
    const f16x8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    s = mfma32(av, bq[j], s);
    if constexpr (KS == kChannel) s = mfma32(av, bq_lo[j], s);
  }
  f32x4 sc;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = s[r];
    if constexpr (KS == kToken) v *= t.ks[r] * kmul;
    else if constexpr (KS == kUniform) v *= kmul;
    if (TAIL && tok0 + 4 * qd + r >= seq_len) v = kNegInf;
    sc[r] = v;
  }
  f32x4 p = softmax_update(st, sc);
  if constexpr (VS == kToken) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] *= t.vs[r];
      if (TAIL && tok0 + 4 * qd + r >= seq_len) p[r] = 0.0f;
    }
  }
  const f16x4 pb = to_f16x4(p);
  int valid = 4;
  if (TAIL) valid = seq_len - (tok0 + 4 * qd);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w = (j < 4) ? t.v0[j] : t.v1[j - 4];
    if (TAIL) w = keep_bytes(w, valid);
    st.o[j] = mfma16(codes4_to_f16<DT>(w), pb, st.o[j]);
  }
}

// ---------------------------------------------------------------------------
// INT4 group tile (4 blocks = 64 tokens)
// ---------------------------------------------------------------------------
struct Tile4 {
  u32x4 k[4];      // per block: channels 32qd..32qd+31 of token l%16 (nibbles)
  u32x4 v[4];      // per block: 4 tokens x 8 channels (nibbles)
  f32x4 vs[4][2];  // per block: V scales of tokens 4qd..4qd+3, both groups
  f32x4 ks[8];     // K scales of channels 32qd .. 32qd+31 for the group
};

__device__ __forceinline__ void load_tile4(Tile4 &t, const DecodeArgs &a,
                                           const int (&phys)[4], int h, int lane,
                                           int qd) {
  const int H = a.num_kv_heads;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t chunk = (size_t)phys[u] * H + h;
    t.k[u] = ld16(a.k_codes + chunk * 1024 + 16 * lane);
    t.v[u] = ld16(a.v_codes + chunk * 1024 + 16 * lane);
    const float *vsp = a.v_scales + (chunk * kBlock + 4 * qd) * 2;
    t.vs[u][0] = ld16f(vsp);
    t.vs[u][1] = ld16f(vsp + 4);
  }
  // block u of the group holds the scales of channels 32u..32u+31
  const int pq = qd == 0 ? phys[0] : qd == 1 ? phys[1] : qd == 2 ? phys[2] : phys[3];
  const float *ksp = a.k_scales + ((size_t)pq * H + h) * 32;
#pragma unroll
  for (int m = 0; m < 8; ++m) t.ks[m] = ld16f(ksp + 4 * m);
}

// k-slot order produced by int4x8_to_f16_pairs: (0,4,1,5,2,6,3,7)
__device__ __forceinline__ int int4_kslot(int e) { return (e >> 1) + 4 * (e & 1); }

__device__ __forceinline__ void compute_tile4(Softmax &st, const Tile4 &t,
                                              const float (&qf)[32], int qd) {
  // q' = q * scale_c * qk_scale for this lane's 32 channels, as hi/lo fp16
  f16x8 bhi[4], blo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int k0 = int4_kslot(2 * e2), k1 = int4_kslot(2 * e2 + 1);
      const int c0 = 8 * j + k0, c1 = 8 * j + k1;
      const float x0 = qf[c0] * t.ks[c0 >> 2][c0 & 3];
      const float x1 = qf[c1] * t.ks[c1 >> 2][c1 & 3];
      split_hi_lo(x0, x1, hi[e2], lo[e2]);
    }
    bhi[j] = pairs_to_f16x8(hi);
    blo[j] = pairs_to_f16x8(lo);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pr[4];
      int4x8_to_f16_pairs(t.k[u][j], pr);
      const f16x8 av = pairs_to_f16x8(pr);
      s = mfma32(av, bhi[j], s);
      s = mfma32(av, blo[j], s);
    }
    const f32x4 p = softmax_update(st, s);
    f32x4 p0, p1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p0[r] = p[r] * t.vs[u][r >> 1][2 * (r & 1)];
      p1[r] = p[r] * t.vs[u][r >> 1][2 * (r & 1) + 1];
    }
    const f16x4 pb0 = to_f16x4(p0), pb1 = to_f16x4(p1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t pr[4];
      int4x8_to_f16_pairs(t.v[u][w], pr);
      const f16x2 a0 = as_f16x2(pr[0]), a1 = as_f16x2(pr[1]);
      const f16x2 b0 = as_f16x2(pr[2]), b1 = as_f16x2(pr[3]);
      const f16x4 va = {a0.x, a0.y, a1.x, a1.y};
      const f16x4 vb = {b0.x, b0.y, b1.x, b1.y};
      const f16x4 &pb = (w < 2) ? pb0 : pb1;
      st.o[2 * w] = mfma16(va, pb, st.o[2 * w]);
      st.o[2 * w + 1] = mfma16(vb, pb, st.o[2 * w + 1]);
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 residual ring tile (INT4 caches)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void compute_ring_tile(Softmax &st, const DecodeArgs &a,
                                                  const uint16_t *kr, const uint16_t *vr,
                                                  const f16x8 (&bq)[4], int slot0,
                                                  int tok0, int seq_len, int n, int qd) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 kv = ld16(kr + (size_t)(slot0 + n) * kHeadDim + 32 * qd + 8 * j);
    s = mfma32(u4_to_f16x8(kv), bq[j], s);
  }
  const int valid = seq_len - (tok0 + 4 * qd);
  f32x4 sc;
#pragma unroll
  for (int r = 0; r < 4; ++r) sc[r] = r < valid ? s[r] * a.qk_scale : kNegInf;
  f32x4 p = softmax_update(st, sc);
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = r < valid ? p[r] : 0.0f;
  const f16x4 pb = to_f16x4(p);
  const uint16_t *vq = vr + ((size_t)(slot0 / 4 + qd) * kHeadDim + n) * 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x2 w = *reinterpret_cast<const u32x2 *>(vq + 16 * j * 4);
    if (valid < 4) {
      // zero the halves of tokens past the end (the ring may hold stale data)
      if (valid <= 0) w = u32x2{0u, 0u};
      else if (valid == 1) w = u32x2{w[0] & 0xFFFFu, 0u};
      else if (valid == 2) w = u32x2{w[0], 0u};
      else w = u32x2{w[0], w[1] & 0xFFFFu};
    }
    st.o[j] = mfma16(u2_to_f16x4(w), pb, st.o[j]);
  }
}

// ---------------------------------------------------------------------------
// epilogue: partial write + last-arrival merge
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_out(float *dst, const f32x4 (&o)[8], float inv,
                                          int qd) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    *reinterpret_cast<f32x4 *>(dst + 16 * j + 4 * qd) = o[j] * inv;
  }
}

__device__ void finish(const DecodeArgs &a, Softmax &st, int b, int h, int p,
                       int n_main, bool has_ring, int lane) {
  const int n = lane & 15, qd = lane >> 4;
  const bool live = n < a.group;
  const int hq = h * a.group + n;
  const float lsum = sum_over_quads(st.l);
  const int total = n_main + (has_ring ? 1 : 0);
  float *out = a.out + ((size_t)b * a.num_q_heads + hq) * kHeadDim;
  if (total == 1) {
    if (live) store_out(out, st.o, 1.0f / lsum, qd);
    return;
  }
  const size_t row = (size_t)b * a.num_q_heads + hq;
  if (live) {
    const size_t idx = row * a.slots + p;
    store_out(a.ws_o + idx * kHeadDim, st.o, 1.0f, qd);
    if (qd == 0) {
      a.ws_m[idx] = st.m;
      a.ws_l[idx] = lsum;
    }
  }
  __threadfence();
  int prev = 0;
  if (lane == 0) {
    prev = __hip_atomic_fetch_add(a.ws_cnt + (size_t)b * a.num_kv_heads + h, 1,
                                  __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  }
  prev = __shfl(prev, 0, 64);
  if (prev != total - 1) return;
  __threadfence();
  if (live) {
    const size_t base = row * a.slots;
    float big = kNegInf;
    for (int pp = 0; pp < total; ++pp) {
      const int slot = pp < n_main ? pp : a.num_parts;
      big = fmaxf(big, a.ws_m[base + slot]);
    }
    float lt = 0.0f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int pp = 0; pp < total; ++pp) {
      const int slot = pp < n_main ? pp : a.num_parts;
      const float w = __builtin_amdgcn_exp2f(a.ws_m[base + slot] - big);
      lt += w * a.ws_l[base + slot];
      const float *src = a.ws_o + (base + slot) * kHeadDim;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j] += w * *reinterpret_cast<const f32x4 *>(src + 16 * j + 4 * qd);
      }
    }
    store_out(out, acc, 1.0f / lt, qd);
  }
  if (lane == 0) {
    __hip_atomic_store(a.ws_cnt + (size_t)b * a.num_kv_heads + h, 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// per-channel / uniform V scale applied to o before it leaves the wavefront
template <int VS>
__device__ __forceinline__ void apply_v_scale(Softmax &st, const DecodeArgs &a, int h,
                                              int qd) {
  if constexpr (VS == kUniform) {
    const float s = a.v_scales[h * a.v_head_stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= s;
  } else if constexpr (VS == kChannel) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 s = ld16f(a.v_scales + h * kHeadDim + 16 * j + 4 * qd);
      st.o[j] *= s;
    }
  }
}

// Load this lane's 32 query channels 32qd .. 32qd+31 (as 4 x 8 fp16).
__device__ __forceinline__ void load_q(u32x4 (&qr)[4], const DecodeArgs &a, int b, int h,
                                       int hq, bool live, int qd) {
  // lanes past the group read the group's first head and discard it
  const int hq_safe = live ? hq : h * a.group;
  const uint16_t *qp = a.q + ((size_t)b * a.num_q_heads + hq_safe) * kHeadDim + 32 * qd;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = ld16(qp + 8 * j);
    qr[j] = live ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int DT, int KS, int VS>
__global__ __launch_bounds__(64) void kvq_paged_decode_kernel(DecodeArgs a) {
  const int p = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int n = lane & 15, qd = lane >> 4;
  const int seq_len = a.seq_lens[b];
  const bool live = n < a.group;
  const int hq = h * a.group + n;

  if (seq_len <= 0) {
    if (p == 0 && live) {
      float *out = a.out + ((size_t)b * a.num_q_heads + hq) * kHeadDim;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4 *>(out + 16 * j + 4 * qd) = z;
    }
    return;
  }

  int n_blocks, nq = 0;
  bool has_ring = false;
  if constexpr (DT == kInt4) {
    nq = kivi_quantized_len(seq_len, a.residual);
    n_blocks = nq / kBlock;
    has_ring = seq_len > nq;
  } else {
    n_blocks = (seq_len + kBlock - 1) / kBlock;
  }
  const int n_main = (n_blocks + a.part_blocks - 1) / a.part_blocks;
  const bool ring_part = (DT == kInt4) && p == a.num_parts;
  if (!ring_part && p >= n_main) return;
  if (ring_part && !has_ring) return;

  u32x4 qr[4];
  load_q(qr, a, b, h, hq, live, qd);

  Softmax st;
  softmax_init(st);
  const int32_t *bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;

  if constexpr (DT == kInt4) {
    if (ring_part) {
      f16x8 bq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[j] = u4_to_f16x8(qr[j]);
      const size_t row = (size_t)b * a.num_kv_heads + h;
      const uint16_t *kr = a.k_resid + row * a.ring * kHeadDim;
      const uint16_t *vr = a.v_resid + row * (a.ring / 4) * kHeadDim * 4;
      for (int t0 = nq; t0 < seq_len; t0 += kBlock) {
        compute_ring_tile(st, a, kr, vr, bq, t0 % a.ring, t0, seq_len, n, qd);
      }
    } else {
      // q * qk_scale in fp32 for the lane's 32 channels (natural order)
      float qf[32];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 hv = u4_to_f16x8(qr[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[8 * j + e] = (float)hv[e] * a.qk_scale;
      }
      const int g0 = (p * a.part_blocks) / 4;
      const int g1 = min(n_blocks, (p + 1) * a.part_blocks) / 4;
      BlockIds ids(bt, 4 * g0, 4 * g1, lane);
      Tile4 cur, nxt;
      int ph[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ph[u] = ids.get(4 * g0 + u, lane);
      load_tile4(cur, a, ph, h, lane, qd);
      for (int gi = g0; gi < g1; gi += 2) {
        if (gi + 1 < g1) {
#pragma unroll
          for (int u = 0; u < 4; ++u) ph[u] = ids.get(4 * (gi + 1) + u, lane);
          load_tile4(nxt, a, ph, h, lane, qd);
        }
        compute_tile4(st, cur, qf, qd);
        if (gi + 1 >= g1) break;
        if (gi + 2 < g1) {
#pragma unroll
          for (int u = 0; u < 4; ++u) ph[u] = ids.get(4 * (gi + 2) + u, lane);
          load_tile4(cur, a, ph, h, lane, qd);
        }
        compute_tile4(st, nxt, qf, qd);
      }
    }
  } else {
    // INT8 / FP8 paged blocks
    f16x8 bq[4], bq_lo[4];
    float kmul = a.qk_scale;
    if constexpr (KS == kChannel) {
      const float *ksc = a.k_scales + h * kHeadDim + 32 * qd;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 hv = u4_to_f16x8(qr[j]);
        const f32x4 s0 = ld16f(ksc + 8 * j), s1 = ld16f(ksc + 8 * j + 4);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 2 * e2;
          const float x0 = (float)hv[e] * a.qk_scale * (e < 4 ? s0[e] : s1[e - 4]);
          const float x1 = (float)hv[e + 1] * a.qk_scale * (e + 1 < 4 ? s0[e + 1] : s1[e - 3]);
          split_hi_lo(x0, x1, hi[e2], lo[e2]);
        }
        bq[j] = pairs_to_f16x8(hi);
        bq_lo[j] = pairs_to_f16x8(lo);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bq[j] = u4_to_f16x8(qr[j]);
        bq_lo[j] = bq[j];
      }
      if constexpr (KS == kUniform) kmul *= a.k_scales[h * a.k_head_stride];
    }
    const int blk0 = p * a.part_blocks;
    const int blk1 = min(n_blocks, blk0 + a.part_blocks);
    const int last = n_blocks - 1;
    const bool partial_last = (seq_len % kBlock) != 0;
    BlockIds ids(bt, blk0, blk1, lane);
    Tile8 cur, nxt;
    load_tile8<KS, VS>(cur, a, ids.get(blk0, lane), h, lane, qd);
    for (int jb = blk0; jb < blk1; jb += 2) {
      if (jb + 1 < blk1) load_tile8<KS, VS>(nxt, a, ids.get(jb + 1, lane), h, lane, qd);
      if (jb == last && partial_last) {
        compute_tile8<DT, KS, VS, true>(st, cur, bq, bq_lo, kmul, jb * kBlock, seq_len, qd);
      } else {
        compute_tile8<DT, KS, VS, false>(st, cur, bq, bq_lo, kmul, jb * kBlock, seq_len, qd);
      }
      if (jb + 1 >= blk1) break;
      if (jb + 2 < blk1) load_tile8<KS, VS>(cur, a, ids.get(jb + 2, lane), h, lane, qd);
      if (jb + 1 == last && partial_last) {
        compute_tile8<DT, KS, VS, true>(st, nxt, bq, bq_lo, kmul, (jb + 1) * kBlock, seq_len, qd);
      } else {
        compute_tile8<DT, KS, VS, false>(st, nxt, bq, bq_lo, kmul, (jb + 1) * kBlock, seq_len, qd);
      }
    }
    apply_v_scale<VS>(st, a, h, qd);
  }
  finish(a, st, b, h, ring_part ? a.num_parts : p, n_main, has_ring, lane);
}

template <int DT, int KS>
hipError_t launch_v(const DecodeArgs &a, int v_kind, dim3 grid, hipStream_t s) {
  switch (v_kind) {
    case kUniform:
      hipLaunchKernelGGL((kvq_paged_decode_kernel<DT, KS, kUniform>), grid, dim3(64), 0, s, a);
      break;
    case kChannel:
      hipLaunchKernelGGL((kvq_paged_decode_kernel<DT, KS, kChannel>), grid, dim3(64), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((kvq_paged_decode_kernel<DT, KS, kToken>), grid, dim3(64), 0, s, a);
      break;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_k(const DecodeArgs &a, int k_kind, int v_kind, dim3 grid, hipStream_t s) {
  switch (k_kind) {
    case kUniform: return launch_v<DT, kUniform>(a, v_kind, grid, s);
    case kChannel: return launch_v<DT, kChannel>(a, v_kind, grid, s);
    default: return launch_v<DT, kToken>(a, v_kind, grid, s);
  }
}

}  // namespace

int decode_scale_kind(int granularity) {
  // kvq_granularity: 0 tensor, 1 head, 2 channel, 3 token
  if (granularity == 2) return kChannel;
  if (granularity == 3) return kToken;
  return kUniform;
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int k_kind, int v_kind, int batch,
                         hipStream_t stream) {
  const int parts = a.num_parts + (dtype == kInt4 ? 1 : 0);
  const dim3 grid(parts, a.num_kv_heads, batch);
  if (dtype == kInt4) {
    hipLaunchKernelGGL((kvq_paged_decode_kernel<kInt4, kChannel, kToken>), grid, dim3(64), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (dtype == kFp8) return launch_k<kFp8>(a, k_kind, v_kind, grid, stream);
  return launch_k<kInt8>(a, k_kind, v_kind, grid, stream);
}

}  // namespace kvq
