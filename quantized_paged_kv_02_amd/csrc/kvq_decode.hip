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
// Work decomposition.  A workgroup of four wavefronts handles one partition
// p of one (row b, KV head h): `part_blocks` consecutive 16-token blocks
// (INT4: whole 64-token groups; the row's last partition also takes the fp16
// residual ring).  The workgroup stages the partition's physical block
// ids in LDS; wave w takes units w, w+4, w+8, ... (a unit is a pair of
// blocks for INT8/FP8, a 64-token group for INT4) and keeps an online
// softmax (running max m in the log2 domain, running sum l, unnormalised
// output o) for the g query heads that share h.  The four wave states are
// merged in LDS; the result is the final output when the launch has a
// single partition per row, else one partial (m, l, o) per (b, hq, p) that
// kvq_partition_reduce merges (log-sum-exp, fixed order) in a second
// launch.  Stream order is the only synchronisation between the two: no
// atomics, no cross-workgroup fences.
//
// Pipelining: unit loads are issued unconditionally one unit ahead of the
// compute (the loop is unrolled by two and the last unit is peeled), so the
// compiler waits only for the unit about to be used while the next one is
// in flight.
//
// Matrix cores: scores S^T[token][head] = K[token][:] . Q^T[:][head] use
// v_mfma_f32_16x16x32_f16 per 16-token block (16 head slots, g of them
// live).  The value product O^T[channel][head] = V^T[channel][token] .
// P^T[token][head] uses v_mfma_f32_16x16x32_f16 over a pair of blocks: lane
// (n = l%16, qd = l/16) holds scores of tokens 4qd..4qd+3 of both blocks,
// which are exactly its eight k-slots of P^T, and the cache layout gives it
// the matching eight V codes of channel 16j + n.  Output lane layout: o[j]
// element i is channel 16j + 4qd + i of head n.
//
// Scales are factored out of the contraction: per-token K scales multiply
// the scores, uniform K scales fold into one multiplier, per-channel K
// scales (and INT4 group scales) fold into q, kept exact as an fp16 hi/lo
// pair; per-token V scales fold into p, uniform and per-channel V scales are
// applied to o once per wave.
//
// An unquantized FP16 cache ([intelli] §5, the baseline of the INT8 memory
// and latency comparison) runs through the same skeleton: its layout puts
// each lane's fp16 operands in 16-byte runs, so a pair of blocks is sixteen
// loads and the matrix-core products with no conversion and no scales.
//
// Further formats on the same skeleton: FP8 E5M2 (codes are the upper byte
// of an fp16; scale-derived fp16 operands carry an exact 2^7), affine INT4
// and 2-bit KIVI groups ([oh-bug] "量化不是简单'截断精度'": the zero points
// enter through offset and bias operands of the matrix products).  Several
// query tokens per row use the score product's columns for (query, head)
// pairs and mask the last block pairs per column.
#include <type_traits>

#include "kvq_args.h"
#include "kvq_device.h"
#include "kvq_kivi_write.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kQRow = 128 + 8;  // LDS row of a staged query (fp16)
constexpr int kQbRow = 64 + 4;  // LDS row of q' (dwords of fp16 pairs)
constexpr int kThreads = 64 * kWaves;
// Block ids staged in LDS per pass (one id per thread; 512-id passes
// measured no faster).
constexpr int kIdChunk = kThreads;
constexpr float kNegInf = -__builtin_inff();
// The running max is only moved when a score exceeds it by more than this
// (log2 units), so p <= 2^8 and rescaling of o is rare.
constexpr float kRescaleSlack = 8.0f;
// Where the weights are multiplied by a per-token V scale sigma before the
// fp16 operand is formed, the lag is bounded so that 2^slack * sigma stays
// below 65504 for every scale finite fp16 values can give: INT8 per token
// sigma <= 65504 / 127 (slack 6), INT4 <= 65504 / 7 and affine INT4
// <= 2 * 65504 / 15 (slack 2), 2-bit <= 2 * 65504 / 3 (slack 0.5).  E4M3
// (<= 65504 / 448) and E5M2 (times 2^7, <= 65504 / 448 as well) fit under
// kRescaleSlack.  Measured on the KIVI shape: the 2-bit launch ~1 % slower
// with the tight bound (more frequent rescales), INT4 within noise.
constexpr float kSlackInt8Token = 6.0f;
constexpr float kSlackInt4 = 2.0f;
constexpr float kSlackInt2 = 0.5f;

struct Softmax {
  float m;     // running max (log2 domain), same on the 4 lanes of a head
  float l;     // this lane's share of the running sum
  f32x4 o[8];  // o^T rows 16j + 4qd + i for head n
};

// Workgroup LDS: block ids and per-wave INT4 scale staging while streaming,
// then the four wave states for the merge.
struct StreamLds {
  int ids[kIdChunk];
  // INT4: K scales [128 channels], V scales [64 tok][2]; affine INT4 also
  // the zero points, laid out the same way from float 256 on
  float scl[kWaves][512];
  // INT4: the group's queries, zero past the group; rows padded by 16 bytes
  // so the 16 head rows of one read start in different banks
  f16 q[16][kQRow];
  // INT4 with a query group of at most 4: per wave, q' = q * s_c of the
  // four heads as fp16 hi and lo rows (channels in the k-slot order of the
  // key conversion)
  uint32_t qb[kWaves][2][4][kQbRow];
};
// o rows padded by 4 floats so the 16 head rows of one store or load fall
// in different banks
constexpr int kMergeRow = kHeadDim + 4;
struct MergeLds {
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][16][kMergeRow];
};
union alignas(16) SharedLds {
  StreamLds s;
  MergeLds g;
  FlushLds<true> f;  // a KIVI step's flush workgroups (FlushLds<false> is smaller)
};

__device__ __forceinline__ void softmax_init(Softmax &st) {
  st.m = kNegInf;
  st.l = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Fold the scores of two blocks (4 tokens each per lane, log2 domain,
// masked = -inf) into the running state; returns p relative to the new max.
__device__ __forceinline__ void softmax_update(Softmax &st, const f32x4 &s0, const f32x4 &s1,
                                               f32x4 &p0, f32x4 &p1,
                                               float slack = kRescaleSlack) {
  float bm = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                   fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
  bm = max_over_quads(bm);
  const bool need = bm > st.m + slack;
  if (__any(need)) {
    const float mn = need ? bm : st.m;
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - mn) : 1.0f;
    st.l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= alpha;
    st.m = mn;
  }
  // a column that has seen only masked scores keeps m = -inf: its weights
  // are exp2(-inf) = 0, not exp2(-inf - -inf)
  const float mref = st.m == kNegInf ? 0.0f : st.m;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p0[r] = __builtin_amdgcn_exp2f(s0[r] - mref);
    p1[r] = __builtin_amdgcn_exp2f(s1[r] - mref);
  }
  st.l += ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
}

// The same for four blocks at once (one max and one rescale decision).
__device__ __forceinline__ void softmax_update4(Softmax &st, f32x4 (&vb)[2],
                                                const f32x4 (&s)[4], f32x4 (&p)[4],
                                                float slack) {
  float bm = kNegInf;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    bm = fmaxf(bm, fmaxf(fmaxf(s[u][0], s[u][1]), fmaxf(s[u][2], s[u][3])));
  bm = max_over_quads(bm);
  const bool need = bm > st.m + slack;
  if (__any(need)) {
    const float mn = need ? bm : st.m;
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - mn) : 1.0f;
    st.l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= alpha;
    vb[0] *= alpha;
    vb[1] *= alpha;
    st.m = mn;
  }
  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int r = 0; r < 4; ++r) p[u][r] = __builtin_amdgcn_exp2f(s[u][r] - st.m);
    sum += (p[u][0] + p[u][1]) + (p[u][2] + p[u][3]);
  }
  st.l += sum;
}

// P^T operand of the value product: tokens 4qd..4qd+3 of block 0, then of
// block 1, rounded to nearest even fp16 (no bias against the fp32 sum).
__device__ __forceinline__ f16x8 p_operand(const f32x4 &p0, const f32x4 &p1) {
  return f16x8{(f16)p0[0], (f16)p0[1], (f16)p0[2], (f16)p0[3],
               (f16)p1[0], (f16)p1[1], (f16)p1[2], (f16)p1[3]};
}

// The same weights as two fp16 terms, hi = fp16(p) and lo = fp16(p - hi)
// (p - hi is exact in fp32): about 22 significant bits where one term keeps
// 11, for a second value product per tile.
__device__ __forceinline__ void p_operand_hilo(const f32x4 &p0, const f32x4 &p1, f16x8 &hi,
                                               f16x8 &lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = i < 4 ? p0[i] : p1[i - 4];
    hi[i] = (f16)p;
    lo[i] = (f16)(p - (float)hi[i]);
  }
}

// BF16 caches: 16-bit operands carried in f16x8 containers hold bf16 bits.
// bf16 keeps 8 significant bits, fp16 11: the weights go to the value
// product as two bf16 terms, hi = bf16(p) and lo = bf16(p - hi) (p - hi is
// exact in fp32), about 16 significant bits together, at the cost of a
// second value MFMA per tile.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void p_operand_bf16(const f32x4 &p0, const f32x4 &p1, f16x8 &hi,
                                               f16x8 &lo) {
  bf16x8 h, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = i < 4 ? p0[i] : p1[i - 4];
    h[i] = (__bf16)p;
    l[i] = (__bf16)(p - (float)h[i]);
  }
  hi = __builtin_bit_cast(f16x8, h);
  lo = __builtin_bit_cast(f16x8, l);
}
__device__ __forceinline__ f32x4 mfma32_bf16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 cat(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f16x8 u4_to_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ f16x4 u2_to_f16x4(u32x2 v) { return __builtin_bit_cast(f16x4, v); }

// E5M2 codes reach 57344 and their scales are max|x| / 57344: scale-derived
// fp16 operands (q' = q s_c, p s_v) would fall into fp16 subnormals.  They
// carry an exact factor 2^7 (so their range is E4M3's, 57344 / 128 = 448),
// removed again in fp32.
template <int DT>
constexpr float operand_boost() { return DT == kFp8E5M2 ? 128.0f : 1.0f; }

template <int DT>
__device__ __forceinline__ f16x4 codes4_to_f16(uint32_t w) {
  if constexpr (DT == kFp8) {
    return fp8x4_to_f16(w);
  } else if constexpr (DT == kFp8E5M2) {
    // an E5M2 byte is the upper byte of the fp16 with the same value
    const uint32_t lo = __builtin_amdgcn_perm(w, w, 0x010C000Cu);  // bytes 0, 1
    const uint32_t hi = __builtin_amdgcn_perm(w, w, 0x030C020Cu);  // bytes 2, 3
    const f16x2 a = as_f16x2(lo), b = as_f16x2(hi);
    return f16x4{a.x, a.y, b.x, b.y};
  } else {
    return int8x4_to_f16(w);
  }
}

// keep the first `n` bytes (0..4) of w
__device__ __forceinline__ uint32_t keep_bytes(uint32_t w, int n) {
  return n >= 4 ? w : (n <= 0 ? 0u : (w & ((1u << (8 * n)) - 1u)));
}

// q' = x rounded toward zero to fp16 (hi) plus the fp16 remainder (lo):
// |x - hi - lo| <= 2^-22 |x|.
__device__ __forceinline__ void split_hi_lo(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = pack_rtz(x0, x1);
  const f16x2 hh = as_f16x2(hi);
  lo = pack_rtz(x0 - (float)hh.x, x1 - (float)hh.y);
}

// A wave-uniform value (a block id read from LDS) moved to a scalar register,
// so tile addresses are a scalar base plus one shared per-lane offset.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Stage physical block ids [c0, c1) of a row in LDS (whole workgroup).  The
// partition's first chunk arrives prefetched (`pre`, one id per thread).
static_assert(kIdChunk == kThreads, "one prefetched block id per thread");
__device__ __forceinline__ void stage_ids(SharedLds &sh, const int32_t *bt, int c0, int c1,
                                          int tid, int pre, bool use_pre) {
  __syncthreads();
  if (use_pre) {
    if (tid < c1 - c0) sh.s.ids[tid] = pre;
  } else if (tid < c1 - c0) {
    sh.s.ids[tid] = bt[c0 + tid];
  }
  __syncthreads();
}

// The scheduler may not move instructions across a pipeline stage boundary:
// otherwise it sinks the next unit's loads below the current unit's first
// use, and the wait for the current unit then also waits for the next one.
__device__ __forceinline__ void stage_fence() { __builtin_amdgcn_sched_barrier(0); }

// Run `cnt` units through a one-ahead software pipeline.  load(T&, k)
// issues unit k's loads, compute(T&, k) consumes them.
template <typename T, typename Load, typename Compute>
__device__ __forceinline__ void pipeline(int cnt, Load &&load, Compute &&compute) {
  if (cnt <= 0) return;
  T a(0), b(1);
  load(a, 0);
  int k = 0;
  for (; k + 2 < cnt; k += 2) {
    load(b, k + 1);
    stage_fence();
    compute(a, k);
    stage_fence();
    load(a, k + 2);
    stage_fence();
    compute(b, k + 1);
    stage_fence();
  }
  if (k + 1 < cnt) {
    load(b, k + 1);
    stage_fence();
    compute(a, k);
    stage_fence();
    compute(b, k + 1);
  } else {
    compute(a, k);
  }
}

// ---------------------------------------------------------------------------
// INT8 / FP8: a unit is a pair of 16-token blocks
// ---------------------------------------------------------------------------
struct Pair8 {
  u32x4 k[2][2];  // block u: K bytes of channels 32qd+0..15 / +16..31, token l%16
  u32x4 v[2][2];  // block u: V bytes, 4 tokens x channels 16j + l%16 (j 0..3 / 4..7)
  f32x4 ks[2];    // per-token K scales of tokens 4qd..4qd+3
  f32x4 vs[2];
  __device__ explicit Pair8(int = 0) {}
};

template <int KS, int VS>
__device__ __forceinline__ void load_pair8(Pair8 &t, const DecodeArgs &a, int ph0, int ph1,
                                           int h, int lane, int qd) {
  const int ph[2] = {ph0, ph1};
  constexpr uint32_t cb = 2048, sb = 64;  // bytes of a code chunk / a scale row
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const size_t chunk = (size_t)ph[u] * a.num_kv_heads + h;
    const rsrc_t kr = make_rsrc(a.k_codes + chunk * 2048, cb);
    const rsrc_t vr = make_rsrc(a.v_codes + chunk * 2048, cb);
    t.k[u][0] = bld16(kr, 16 * lane);
    t.k[u][1] = bld16(kr, 16 * lane + 1024);
    t.v[u][0] = bld16(vr, 16 * lane);
    t.v[u][1] = bld16(vr, 16 * lane + 1024);
    if constexpr (KS == kToken)
      t.ks[u] = bld16f(make_rsrc(a.k_scales + chunk * kBlock, sb), 16 * qd);
    if constexpr (VS == kToken)
      t.vs[u] = bld16f(make_rsrc(a.v_scales + chunk * kBlock, sb), 16 * qd);
  }
}

// Scores of one block: 4 x v_mfma_f32_16x16x32_f16 over channels 32qd+8j..+7.
template <int DT, int KS>
__device__ __forceinline__ f32x4 block_scores8(const u32x4 (&k)[2], const f16x8 (&bq)[4],
                                               const f16x8 (&bq_lo)[4]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 &src = k[j >> 1];
    const int jj = j & 1;
    const f16x8 av = cat(codes4_to_f16<DT>(src[2 * jj]), codes4_to_f16<DT>(src[2 * jj + 1]));
    s = mfma32(av, bq[j], s);
    if constexpr (KS == kChannel) s = mfma32(av, bq_lo[j], s);
  }
  return s;
}

// TAIL only: valid_s = tokens of the pair this lane's column attends to
// (may be <= 0), valid_v = tokens of the pair that exist (1..32, the same
// for every lane; values past it are zeroed).
template <int DT, int KS, int VS, bool TAIL>
__device__ __forceinline__ void compute_pair8(Softmax &st, Pair8 &t, const f16x8 (&bq)[4],
                                              const f16x8 (&bq_lo)[4], float kmul, int valid_s,
                                              int valid_v, int qd) {
  f32x4 s[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    s[u] = block_scores8<DT, KS>(t.k[u], bq, bq_lo);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = s[u][r];
      if constexpr (KS == kToken) v *= t.ks[u][r] * kmul;
      else v *= kmul;
      if (TAIL && 16 * u + 4 * qd + r >= valid_s) v = kNegInf;
      s[u][r] = v;
    }
  }
  f32x4 p0, p1;
  softmax_update(st, s[0], s[1], p0, p1,
                 VS == kToken && DT == kInt8 ? kSlackInt8Token : kRescaleSlack);
  if constexpr (VS == kToken) {
    constexpr float boost = operand_boost<DT>();  // removed from o at the end
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p0[r] *= t.vs[0][r] * boost;
      p1[r] *= t.vs[1][r] * boost;
      if (TAIL && 4 * qd + r >= valid_s) p0[r] = 0.0f;
      if (TAIL && 16 + 4 * qd + r >= valid_s) p1[r] = 0.0f;
    }
  }
  // per-token V scales: the weights as a hi + lo pair (a second value
  // product per tile); otherwise one fp16 term
  f16x8 pb, pl;
  if constexpr (VS == kToken) p_operand_hilo(p0, p1, pb, pl);
  else pb = p_operand(p0, p1);
  if (TAIL) {
    // zero the codes of tokens past the end (their bytes may be stale or NaN)
    const int v0 = valid_v - 4 * qd, v1 = valid_v - 16 - 4 * qd;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        t.v[0][i][w] = keep_bytes(t.v[0][i][w], v0);
        t.v[1][i][w] = keep_bytes(t.v[1][i][w], v1);
      }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f16x8 av = cat(codes4_to_f16<DT>(t.v[0][j >> 2][j & 3]),
                         codes4_to_f16<DT>(t.v[1][j >> 2][j & 3]));
    st.o[j] = mfma32(av, pb, st.o[j]);
    if constexpr (VS == kToken) st.o[j] = mfma32(av, pl, st.o[j]);
  }
}

// ---------------------------------------------------------------------------
// FP16 (unquantized): a unit is a pair of 16-token blocks whose 16-byte
// loads are the matrix-core operands as they stand
// ---------------------------------------------------------------------------
struct Pair16 {
  u32x4 k[2][4];  // block u, quarter j: channels 32qd+8j..+7 of token l%16
  u32x4 v[2][4];  // block u, quarter j: tokens 4qd..4qd+3 of channel 32j+l%16,
                  // then of channel 32j+16+l%16
  __device__ explicit Pair16(int = 0) {}
};

__device__ __forceinline__ void load_pair16(Pair16 &t, const DecodeArgs &a, int ph0, int ph1,
                                            int h, int lane) {
  constexpr uint32_t cb = 4096;  // bytes of a (block, head) chunk
  const size_t c0 = ((size_t)ph0 * a.num_kv_heads + h) * cb;
  const size_t c1 = ((size_t)ph1 * a.num_kv_heads + h) * cb;
  const rsrc_t k0 = make_rsrc(a.k_codes + c0, cb), k1 = make_rsrc(a.k_codes + c1, cb);
  const rsrc_t v0 = make_rsrc(a.v_codes + c0, cb), v1 = make_rsrc(a.v_codes + c1, cb);
#pragma unroll
  for (int j = 0; j < 4; ++j) t.k[0][j] = bld16(k0, 16 * lane + 1024 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) t.k[1][j] = bld16(k1, 16 * lane + 1024 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) t.v[0][j] = bld16(v0, 16 * lane + 1024 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) t.v[1][j] = bld16(v1, 16 * lane + 1024 * j);
}

// V operand of output tile j (channels 16j + l%16): the lane's 4 tokens of
// block 0, then of block 1
__device__ __forceinline__ f16x8 value_operand16(const Pair16 &t, int j) {
  const int w = 2 * (j & 1);
  return cat(u2_to_f16x4(u32x2{t.v[0][j >> 1][w], t.v[0][j >> 1][w + 1]}),
             u2_to_f16x4(u32x2{t.v[1][j >> 1][w], t.v[1][j >> 1][w + 1]}));
}

// valid_s, valid_v as for compute_pair8.  BF: a BF16 cache (bf16 operands).
template <bool TAIL, bool BF>
__device__ __forceinline__ void compute_pair16(Softmax &st, Pair16 &t, const f16x8 (&bq)[4],
                                               float kmul, int valid_s, int valid_v, int qd) {
  auto mma = [](f16x8 a, f16x8 b, f32x4 c) { return BF ? mfma32_bf16(a, b, c) : mfma32(a, b, c); };
  f32x4 s[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) s[u] = mma(u4_to_f16x8(t.k[u][j]), bq[j], s[u]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = s[u][r] * kmul;
      s[u][r] = (TAIL && 16 * u + 4 * qd + r >= valid_s) ? kNegInf : v;
    }
  }
  f32x4 p0, p1;
  softmax_update(st, s[0], s[1], p0, p1);
  f16x8 pb, pl;
  if constexpr (BF) p_operand_bf16(p0, p1, pb, pl);
  else p_operand_hilo(p0, p1, pb, pl);
  if (TAIL) {
    // zero the values of unattended tokens (stale, possibly NaN): dword w
    // of a quarter holds tokens 2(w&1), 2(w&1)+1 of the lane's four
    const int v0 = valid_v - 4 * qd, v1 = valid_v - 16 - 4 * qd;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        t.v[0][j][w] = keep_bytes(t.v[0][j][w], 2 * (v0 - 2 * (w & 1)));
        t.v[1][j][w] = keep_bytes(t.v[1][j][w], 2 * (v1 - 2 * (w & 1)));
      }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f16x8 v = value_operand16(t, j);
    st.o[j] = mma(v, pb, st.o[j]);
    st.o[j] = mma(v, pl, st.o[j]);
  }
}

template <int DT> struct UnitOf { using T = Pair8; };
template <> struct UnitOf<kFp16> { using T = Pair16; };
template <> struct UnitOf<kBf16> { using T = Pair16; };

// Query operand of the score product for this lane's channels 32qd..32qd+31
// (as 4 x 8 fp16), zero for the 16 - cols padding columns.  Column n is
// query token n / g, head h*g + n % g.
__device__ __forceinline__ void load_q(u32x4 (&qr)[4], const DecodeArgs &a, int b, int h, int n,
                                       int qd) {
  const bool live = n < a.cols;
  const int qt = live ? n / a.group : 0;
  const int hq = h * a.group + (live ? n - qt * a.group : 0);
  const uint16_t *qp =
      a.q + (((size_t)b * a.n_query + qt) * a.num_q_heads + hq) * kHeadDim + 32 * qd;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = ld16(qp + 8 * j);
    qr[j] = live ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

// Blocks [blk0, blk1) of row b (a partition, or a balanced launch's segment
// of the row).  use_pre: the first 256 block ids arrive prefetched (pre_id).
template <int DT, int KS, int VS>
__device__ void stream_q8(Softmax &st, const DecodeArgs &a, SharedLds &sh, int b, int h,
                          int blk0, int blk1, int seq_len, int wave, int lane, int tid,
                          int pre_id, bool use_pre) {
  const int n = lane & 15, qd = lane >> 4;
  u32x4 qr[4];
  load_q(qr, a, b, h, n, qd);
  f16x8 bq[4], bq_lo[4];
  float kmul = a.qk_scale;
  if constexpr (is_f16_cache(DT)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bq[j] = bq_lo[j] = u4_to_f16x8(qr[j]);
  } else if constexpr (KS == kChannel) {
    const float *ksc = a.k_scales + h * kHeadDim + 32 * qd;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x8 hv = u4_to_f16x8(qr[j]);
      const f32x4 s0 = ld16f(ksc + 8 * j), s1 = ld16f(ksc + 8 * j + 4);
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e = 2 * e2;
        constexpr float boost = operand_boost<DT>();
        const float x0 = (float)hv[e] * a.qk_scale * (e < 4 ? s0[e] : s1[e - 4]) * boost;
        const float x1 =
            (float)hv[e + 1] * a.qk_scale * (e + 1 < 4 ? s0[e + 1] : s1[e - 3]) * boost;
        split_hi_lo(x0, x1, hi[e2], lo[e2]);
      }
      bq[j] = pairs_to_f16x8(hi);
      bq_lo[j] = pairs_to_f16x8(lo);
    }
    kmul = 1.0f / operand_boost<DT>();
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bq[j] = u4_to_f16x8(qr[j]);
      bq_lo[j] = bq[j];
    }
    if constexpr (KS == kUniform) kmul *= a.k_scales[h * a.k_head_stride];
  }

  const int32_t *bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  for (int c0 = blk0; c0 < blk1; c0 += kIdChunk) {
    const int c1 = min(blk1, c0 + kIdChunk);
    stage_ids(sh, bt, c0, c1, tid, pre_id, use_pre && c0 == blk0);
    const int npairs = (c1 - c0 + 1) / 2;
    // Pairs wholly visible to every column run unmasked.  The rest are
    // masked per column: the row's partial block, a chunk's odd last block
    // and, with several query tokens, the last positions that only the
    // later queries see (at most two pairs in all).
    const int end_tok = min(seq_len, c1 * kBlock);
    const int all_end = min(seq_len - a.n_query + 1, end_tok);
    const int nfull = max(0, min(npairs, (all_end - c0 * kBlock) / (2 * kBlock)));
    const int cnt = wave < nfull ? (nfull - wave + kWaves - 1) / kWaves : 0;
    using Unit = typename UnitOf<DT>::T;
    auto load_unit = [&](Unit &t, int ph0, int ph1) {
      if constexpr (is_f16_cache(DT)) {
        load_pair16(t, a, ph0, ph1, h, lane);
      } else {
        load_pair8<KS, VS>(t, a, ph0, ph1, h, lane, qd);
      }
    };
    auto load = [&](Unit &t, int k) {
      const int j0 = 2 * (wave + kWaves * k);
      load_unit(t, uniform(sh.s.ids[j0]), uniform(sh.s.ids[j0 + 1]));
    };
    auto compute = [&](Unit &t, int) {
      if constexpr (is_f16_cache(DT)) {
        compute_pair16<false, DT == kBf16>(st, t, bq, kmul, 32, 32, qd);
      } else {
        compute_pair8<DT, KS, VS, false>(st, t, bq, bq_lo, kmul, 32, 32, qd);
      }
    };
    pipeline<Unit>(cnt, load, compute);
    // masked pairs (at most two: no wave owns more than one), each by the
    // wave the round-robin gives it
    const int i = nfull + (wave - nfull % kWaves + kWaves) % kWaves;
    if (i < npairs) {
      const int j0 = 2 * i;
      const int start = (c0 + j0) * kBlock;
      const int valid_v = end_tok - start;  // 1..32
      // position of this lane's column's query token (padding columns: the
      // last); computed here so it is not live across the pipeline
      const int last_pos = seq_len - a.n_query + (n < a.cols ? n / a.group : a.n_query - 1);
      const int valid_s = min(valid_v, last_pos + 1 - start);
      const int ph0 = uniform(sh.s.ids[j0]);
      const int ph1 = c0 + j0 + 1 < c1 ? uniform(sh.s.ids[j0 + 1]) : ph0;
      Unit t;
      load_unit(t, ph0, ph1);
      if constexpr (is_f16_cache(DT)) {
        compute_pair16<true, DT == kBf16>(st, t, bq, kmul, valid_s, valid_v, qd);
      } else {
        compute_pair8<DT, KS, VS, true>(st, t, bq, bq_lo, kmul, valid_s, valid_v, qd);
      }
    }
  }
  if constexpr (is_f16_cache(DT)) return;  // no scales
  // uniform and per-channel V scales multiply o once (per-token ones rode
  // on the weights, with the operand boost to remove)
  if constexpr (VS == kToken && operand_boost<DT>() != 1.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= 1.0f / operand_boost<DT>();
  }
  if constexpr (VS == kUniform) {
    const float s = a.v_scales[h * a.v_head_stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= s;
  } else if constexpr (VS == kChannel) {
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= ld16f(a.v_scales + h * kHeadDim + 16 * j + 4 * qd);
  }
}

// ---------------------------------------------------------------------------
// INT4 KIVI: a unit is a 64-token group (4 blocks)
// ---------------------------------------------------------------------------
// Key nibbles -> 8 fp16 with offsets, in six operations: the low nibble of
// each byte, biased to code + 8, is the OCP E4M3 byte 0000nnnn = (code + 8)
// / 512 exactly (subnormal below 8), which the hardware conversion with
// scale 512 turns into code + 8; high nibbles take the exponent splice
// (1152 + 16 code).  Slot e holds nibble kperm(e) = 0, 2, 1, 5, 4, 6, 3, 7;
// slots 2, 3, 6, 7 are the high nibbles.  The offsets (8 per low slot, 1152
// per high slot) add a per-(head, group) constant to every score of the
// group, removed after the product.
__device__ __forceinline__ f16x8 int4x8_to_f16_koff(uint32_t x) {
  const uint32_t lo = bsel(x, 0x0F0F0F0Fu, 0x08080808u);
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);  // nibbles 0, 2
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);   // nibbles 4, 6
  const f16x2 b = as_f16x2(bsel(x, 0x00F000F0u, 0x64806480u));                  // nibbles 1, 5
  const f16x2 d = as_f16x2(bsel(x >> 8, 0x00F000F0u, 0x64806480u));             // nibbles 3, 7
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Affine (unsigned) key nibbles in the same slot order: low nibbles read as
// E4M3 bytes 0000nnnn give u, high nibbles under the exponent of 1024 give
// 1024 + 16 u; the offsets (the zero points) are removed after the product.
__device__ __forceinline__ f16x8 uint4x8_to_f16_koff(uint32_t x) {
  const uint32_t lo = x & 0x0F0F0F0Fu;
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);  // nibbles 0, 2
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);   // nibbles 4, 6
  const f16x2 b = as_f16x2(and_or(x, 0x00F000F0u, 0x64006400u));               // nibbles 1, 5
  const f16x2 d = as_f16x2(and_or(x >> 8, 0x00F000F0u, 0x64006400u));          // nibbles 3, 7
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Lane k of this lane's 16-lane row (DPP row broadcast).
template <int K>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
  static_assert(K >= 0 && K < 16, "lane within a row");
  // every lane's source is valid: no old value to merge
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + K, 0xF, 0xF, true);
}

// Offset operand of the affine key conversion for the channels 8j..8j+7 of
// a lane's 32 (zero-point bytes d0 = channels 0..3, d1 = 4..7): z for the
// low-nibble slots, 1024 + 16 z for the high ones, in the slot order
// 0, 2, 1, 5, 4, 6, 3, 7.
__device__ __forceinline__ f16x8 zp_key_offsets(uint32_t d0, uint32_t d1) {
  const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
      __builtin_amdgcn_perm(d0, d0, 0x0C0C0200u), 512.0f, false);                       // z0, z2
  const uint32_t s23 = (__builtin_amdgcn_perm(d1, d0, 0x0C050C01u) << 4) | 0x64006400u;  // z1, z5
  const f16x2 s45 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
      __builtin_amdgcn_perm(d1, d1, 0x0C0C0200u), 512.0f, false);                       // z4, z6
  const uint32_t s67 = (__builtin_amdgcn_perm(d1, d0, 0x0C070C03u) << 4) | 0x64006400u;  // z3, z7
  return u4_to_f16x8(u32x4{as_u32(s01), s23, as_u32(s45), s67});
}

// Value bias operand of an affine block pair for channel group g from the
// pair's 16 zero-point bytes (byte 8b + 2e + g: block b of the pair, token
// 4qd + e): -(1024 + z) for tokens 0, 1 (low nibbles), -(1024 + 16 z) for
// tokens 2, 3, block 0 then block 1.
template <int G>
__device__ __forceinline__ f16x8 zp_value_bias(const u32x4 &w) {
  constexpr uint32_t sel = G ? 0x0C030C01u : 0x0C020C00u;  // bytes g, 2 + g -> halves
  constexpr uint32_t neg1024 = 0xE400E400u;
  const u32x4 r = {__builtin_amdgcn_perm(w[0], w[0], sel) | neg1024,
                   (__builtin_amdgcn_perm(w[1], w[1], sel) << 4) | neg1024,
                   __builtin_amdgcn_perm(w[2], w[2], sel) | neg1024,
                   (__builtin_amdgcn_perm(w[3], w[3], sel) << 4) | neg1024};
  return u4_to_f16x8(r);
}

// The two channels (within a k-slot chunk of 8) of lane l's slot pair
// 2(l%4), 2(l%4)+1 in the offset conversion's order: (0,2) (1,5) (4,6) (3,7).
__device__ __forceinline__ int2 koff_pair(int lane) {
  const int i = lane & 3;
  return int2{(0x3410 >> (4 * i)) & 0xF, (0x7652 >> (4 * i)) & 0xF};
}

struct Group4 {
  u32x4 k[4];   // block u: nibbles of channels 32qd..32qd+31, token l%16
  u32x4 v[4];   // block u: nibbles of 4 tokens x 8 channel tiles
  float ks[2];  // K scales of channels 8(l/4) + koff_pair(l) (block l/16)
  float vs[2];  // V scales (channel groups 0, 1) of token l of the group
  uint32_t kz;  // affine: zero points of those K channels (bytes 0, 1)
  uint32_t vz;  // affine: zero points of those V scales (bytes 0, 1)
  __device__ explicit Group4(int = 0) {}
};

// pm: physical block of this lane's K-scale row (block lane/16 of the group).
// AFF: scale rows of 40 floats, the zero points in the last 32 bytes; pz:
// physical block (lane%16)/4 of the group, whose V row holds this lane's
// token's zero points (group-transposed).
template <bool AFF>
__device__ __forceinline__ void load_group4(Group4 &t, const DecodeArgs &a, const int (&ph)[4],
                                            int pm, int pz, int h, int lane) {
  constexpr int kRow = AFF ? 40 : 32;  // floats per (block, head) scale row
  const int H = a.num_kv_heads;
  constexpr uint32_t bytes = 1024;  // one (block, head) code chunk
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t chunk = (size_t)ph[u] * H + h;
    t.k[u] = bld16(make_rsrc(a.k_codes + chunk * 1024, bytes), 16 * lane);
    t.v[u] = bld16(make_rsrc(a.v_codes + chunk * 1024, bytes), 16 * lane);
  }
  const size_t chunk = (size_t)pm * H + h;
  // channels koff_pair(lane) of k-slot chunk lane/4, held by block lane/16
  const int2 ko = koff_pair(lane);
  const float *krow = a.k_scales + chunk * kRow;
  const float *vrow = a.v_scales + chunk * kRow;
  const float *ksp = krow + 8 * ((lane >> 2) & 3);
  const float2 vs = *reinterpret_cast<const float2 *>(vrow + 2 * (lane & 15));
  t.ks[0] = ksp[ko.x];
  t.ks[1] = ksp[ko.y];
  t.vs[0] = vs.x;
  t.vs[1] = vs.y;
  if constexpr (AFF) {
    const uint8_t *kzp = reinterpret_cast<const uint8_t *>(krow + 32) + 8 * ((lane >> 2) & 3);
    t.kz = (uint32_t)kzp[ko.x] | ((uint32_t)kzp[ko.y] << 8);
    const float *zrow = a.v_scales + ((size_t)pz * H + h) * kRow;
    t.vz = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(zrow + 32) +
                                               8 * (lane >> 4) + 2 * (lane & 3));
  }
}

// The group as the compact path reads it: K scales as above, and the V
// scales of this lane's tokens 4qd..4qd+3 of block (l%16)/4 straight from
// the scale rows (channel groups 0, 1 interleaved: tokens 0, 1 then 2, 3).
struct Group4C {
  u32x4 k[4];
  u32x4 v[4];
  float ks[2];
  f32x4 vsa, vsb;
  // affine: dword l%16 of the 64 zero-point bytes this lane's row of the
  // wave needs: K zero points of channels 32qd..32qd+31 (dwords 0..7), then
  // V zero points of tokens 4qd..4qd+3 of blocks 0..3 (dwords 8..15).  Each
  // lane loads one dword; row broadcasts hand them to the whole row.
  uint32_t zw;
  __device__ explicit Group4C(int = 0) {}
};

// pm as for load_group4; pv: physical block (l%16)/4 of the group.  AFF:
// rows of 40 floats; the zero points this lane's operands need are the
// last 32 bytes of block qd's K and V rows.
template <bool AFF>
__device__ __forceinline__ void load_group4c(Group4C &t, const DecodeArgs &a, const int (&ph)[4],
                                             int pm, int pv, int h, int lane) {
  constexpr int kRow = AFF ? 40 : 32;
  const int H = a.num_kv_heads;
  constexpr uint32_t bytes = 1024;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t chunk = (size_t)ph[u] * H + h;
    t.k[u] = bld16(make_rsrc(a.k_codes + chunk * 1024, bytes), 16 * lane);
    t.v[u] = bld16(make_rsrc(a.v_codes + chunk * 1024, bytes), 16 * lane);
  }
  const int2 ko = koff_pair(lane);
  const float *krow = a.k_scales + ((size_t)pm * H + h) * kRow;
  const float *ksp = krow + 8 * ((lane >> 2) & 3);
  t.ks[0] = ksp[ko.x];
  t.ks[1] = ksp[ko.y];
  const float *vsp = a.v_scales + ((size_t)pv * H + h) * kRow + 8 * (lane >> 4);
  t.vsa = ld16f(vsp);
  t.vsb = ld16f(vsp + 4);
  if constexpr (AFF) {
    const int n = lane & 15;
    const float *zrow = (n < 8 ? a.k_scales : a.v_scales) + ((size_t)pm * H + h) * kRow + 32;
    t.zw = reinterpret_cast<const uint32_t *>(zrow)[n & 7];
  }
}

// Join block b0's and block b1's nibbles of channel tile j (dword j>>1 of
// each, tile A = bytes 0/2, tile B = bytes 1/3) into one dword whose eight
// nibbles convert to tokens 4qd..4qd+3 of b0 then of b1.
__device__ __forceinline__ uint32_t pair_tile(uint32_t w0, uint32_t w1, int odd) {
  return __builtin_amdgcn_perm(w1, w0, odd ? 0x07030501u : 0x06020400u);
}

// 8 nibbles -> 8 exact fp16, k-slot order (0,4,1,5,2,6,3,7) of the nibbles.
__device__ __forceinline__ f16x8 int4x8_to_f16(uint32_t x) {
  uint32_t pr[4];
  int4x8_to_f16_pairs(x, pr);
  return pairs_to_f16x8(pr);
}

// 8 nibbles -> 8 fp16 still carrying the exponent bias of the
// bitwise-select trick: k-slots 0,1,4,5 hold 1032 + code, k-slots 2,3,6,7
// hold 1152 + 16 code (nibbles in the upper half of a byte).  Exact.
[[maybe_unused]] __device__ __forceinline__ f16x8 int4x8_to_f16_biased(uint32_t x) {
  const uint32_t y = x >> 8;
  const uint32_t r[4] = {bsel(x, 0x000F000Fu, 0x64086408u), bsel(x, 0x00F000F0u, 0x64806480u),
                         bsel(y, 0x000F000Fu, 0x64086408u), bsel(y, 0x00F000F0u, 0x64806480u)};
  return pairs_to_f16x8(r);
}

// k-slot order produced by int4x8_to_f16 (nibble index of slot e)
__device__ __forceinline__ int int4_kslot(int e) { return (e >> 1) + 4 * (e & 1); }

// Affine codes: 8 unsigned nibbles minus their zero points, exact, in the
// k-slot order of int4x8_to_f16.  Low nibbles under the fp16 exponent of
// 1024 give 1024 + u, high nibbles 1024 + 16 u (times 1/16: 64 + u); `sub`
// holds -(1024 + z) for slot pairs 0 and 2 and -(64 + z) for 1 and 3.
__device__ __forceinline__ f16x8 uint4x8_minus_zp(uint32_t x, const uint32_t (&sub)[4]) {
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const uint32_t y = x >> 8;
  uint32_t r[4];
  r[0] = as_u32(as_f16x2(and_or(x, 0x000F000Fu, 0x64006400u)) + as_f16x2(sub[0]));
  r[1] = as_u32(as_f16x2(and_or(x, 0x00F000F0u, 0x64006400u)) * sixteenth + as_f16x2(sub[1]));
  r[2] = as_u32(as_f16x2(and_or(y, 0x000F000Fu, 0x64006400u)) + as_f16x2(sub[2]));
  r[3] = as_u32(as_f16x2(and_or(y, 0x00F000F0u, 0x64006400u)) * sixteenth + as_f16x2(sub[3]));
  return pairs_to_f16x8(r);
}

// Affine value codes: 8 unsigned nibbles -> 1024 + u (k-slots 0,1,4,5) and
// 1024 + 16 u (k-slots 2,3,6,7), exact; the bias is removed after the
// product, with the zero points.
__device__ __forceinline__ f16x8 uint4x8_to_f16_biased(uint32_t x) {
  const uint32_t y = x >> 8;
  const uint32_t r[4] = {and_or(x, 0x000F000Fu, 0x64006400u), and_or(x, 0x00F000F0u, 0x64006400u),
                         and_or(y, 0x000F000Fu, 0x64006400u), and_or(y, 0x00F000F0u, 0x64006400u)};
  return pairs_to_f16x8(r);
}

// AFF: affine codes; the zero points are staged beside the scales (float
// 256 on) and enter the key conversion and the value bias operand.
template <bool AFF>
__device__ __forceinline__ void compute_group4(Softmax &st, f32x4 (&vb)[2], const Group4 &t,
                                               const f16 *qs,
                                               float *scl, float qk_scale, int lane, int n,
                                               int qd) {
  // stage the group's scales in this wave's LDS slot (in-order within a wave)
  {
    const int2 ko = koff_pair(lane);
    scl[8 * (lane >> 2) + ko.x] = t.ks[0];
    scl[8 * (lane >> 2) + ko.y] = t.ks[1];
    if constexpr (AFF) {
      scl[256 + 8 * (lane >> 2) + ko.x] = (float)(t.kz & 0xFFu);
      scl[256 + 8 * (lane >> 2) + ko.y] = (float)(t.kz >> 8);
      *reinterpret_cast<float2 *>(scl + 384 + 2 * lane) =
          float2{(float)(t.vz & 0xFFu), (float)(t.vz >> 8)};
    }
  }
  // tokens 2, 3 of every 4 meet the value codes stored as 1152 + 16 code
  // (affine: 1024 + 16 code): their weights carry 1/16 (exact)
  const float vsf = (lane & 2) ? 0.0625f : 1.0f;
  *reinterpret_cast<float2 *>(scl + 128 + 2 * lane) = float2{t.vs[0] * vsf, t.vs[1] * vsf};
  // Scores, channel chunk by chunk: q' = q * s_c for channels 32qd+8j..+7
  // as fp16 hi + lo in the k-slot order of the nibble conversion, applied
  // to the chunk of all four blocks.
  f32x4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x8 qh = *reinterpret_cast<const f16x8 *>(qs + n * kQRow + 32 * qd + 8 * j);
    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(scl + 32 * qd + 8 * j);
    const f32x4 s1 = *reinterpret_cast<const f32x4 *>(scl + 32 * qd + 8 * j + 4);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int c0 = int4_kslot(2 * e2), c1 = int4_kslot(2 * e2 + 1);
      const float x0 = (float)qh[c0] * (c0 < 4 ? s0[c0] : s1[c0 - 4]);
      const float x1 = (float)qh[c1] * (c1 < 4 ? s0[c1] : s1[c1 - 4]);
      split_hi_lo(x0, x1, hi[e2], lo[e2]);
    }
    const f16x8 bhi = pairs_to_f16x8(hi), blo = pairs_to_f16x8(lo);
    // affine: code - zero point of channels 32qd+8j..+7, slot pairs (0,4)
    // (1,5) (2,6) (3,7) of the conversion
    uint32_t sub[4];
    if constexpr (AFF) {
      const f32x4 z0 = *reinterpret_cast<const f32x4 *>(scl + 256 + 32 * qd + 8 * j);
      const f32x4 z1 = *reinterpret_cast<const f32x4 *>(scl + 256 + 32 * qd + 8 * j + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float base = (i & 1) ? 64.0f : 1024.0f;
        sub[i] = pack_rtz(-(base + z0[i]), -(base + z1[i]));
      }
    }
    // all hi products, then all lo products: an accumulator's two updates
    // are four matrix instructions apart
    f16x8 av[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (AFF) {
        av[u] = uint4x8_minus_zp(t.k[u][j], sub);
      } else {
        av[u] = int4x8_to_f16(t.k[u][j]);
      }
      acc[u] = mfma32(av[u], bhi, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = mfma32(av[u], blo, acc[u]);
  }
  f32x4 pg[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] *= qk_scale;
  softmax_update4(st, vb, acc, pg, kSlackInt4);
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const f32x4 &p0 = pg[2 * pr], &p1 = pg[2 * pr + 1];
    // per-token V scales (channel groups 0 and 1) of tokens 4qd..4qd+3
    const float *vsp = scl + 128 + 2 * (32 * pr + 4 * qd);
    const f32x4 va0 = *reinterpret_cast<const f32x4 *>(vsp);        // tokens 0,1 of b0
    const f32x4 va1 = *reinterpret_cast<const f32x4 *>(vsp + 4);    // tokens 2,3 of b0
    const f32x4 vb0 = *reinterpret_cast<const f32x4 *>(vsp + 32);   // tokens 0,1 of b1
    const f32x4 vb1 = *reinterpret_cast<const f32x4 *>(vsp + 36);   // tokens 2,3 of b1
    const f32x4 g0a = {va0[0], va0[2], va1[0], va1[2]}, g1a = {va0[1], va0[3], va1[1], va1[3]};
    const f32x4 g0b = {vb0[0], vb0[2], vb1[0], vb1[2]}, g1b = {vb0[1], vb0[3], vb1[1], vb1[3]};
    const f16x8 pb0 = p_operand(p0 * g0a, p1 * g0b);
    const f16x8 pb1 = p_operand(p0 * g1a, p1 * g1b);
    // every row of the bias operand is the per-k-slot bias of the biased
    // conversion (1032 for slots 0,1,4,5; 1152 for 2,3,6,7), negated.
    // Affine: the bias of slot k is 1024 + z (low nibbles) or 1024 + 16 z
    // (high nibbles) with z the zero point of the slot's token and the
    // tile's channel group, so it differs per lane.
    f16x8 abias0, abias1;
    if constexpr (AFF) {
      const float *zp = scl + 384 + 2 * (32 * pr + 4 * qd);
      const f32x4 za0 = *reinterpret_cast<const f32x4 *>(zp);        // b0 tokens 0,1
      const f32x4 za1 = *reinterpret_cast<const f32x4 *>(zp + 4);    // b0 tokens 2,3
      const f32x4 zb0 = *reinterpret_cast<const f32x4 *>(zp + 32);   // b1 tokens 0,1
      const f32x4 zb1 = *reinterpret_cast<const f32x4 *>(zp + 36);   // b1 tokens 2,3
      auto lo = [](float z) { return (f16)(-(1024.0f + z)); };
      auto hi = [](float z) { return (f16)(-(1024.0f + 16.0f * z)); };
      abias0 = f16x8{lo(za0[0]), lo(za0[2]), hi(za1[0]), hi(za1[2]),
                     lo(zb0[0]), lo(zb0[2]), hi(zb1[0]), hi(zb1[2])};
      abias1 = f16x8{lo(za0[1]), lo(za0[3]), hi(za1[1]), hi(za1[3]),
                     lo(zb0[1]), lo(zb0[3]), hi(zb1[1]), hi(zb1[3])};
    } else {
      const f16 b0 = (f16)-1032.0f, b1 = (f16)-1152.0f;
      abias0 = abias1 = f16x8{b0, b0, b1, b1, b0, b0, b1, b1};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = pair_tile(t.v[2 * pr][j >> 1], t.v[2 * pr + 1][j >> 1], j & 1);
      const f16x8 av = AFF ? uint4x8_to_f16_biased(w) : int4x8_to_f16_biased(w);
      st.o[j] = mfma32(av, j < 4 ? pb0 : pb1, st.o[j]);
    }
    // bias cancellation: the operand's rows are alike, so one product per
    // channel group into its accumulator, added to the tiles at the end
    vb[0] = mfma32(abias0, pb0, vb[0]);
    vb[1] = mfma32(abias1, pb1, vb[1]);
  }
}

// ---------------------------------------------------------------------------
// 2-bit affine KIVI on the generic layout (more than four query heads per KV
// head, or several queries per row): the 16 score columns hold (query,
// head) pairs; q' = q s_c is split into fp16 hi and lo products as for
// INT4.  Codes are converted as FP4 nibbles (see the compact 2-bit path
// below) and the zero points subtracted exactly in fp16 before the key
// products; the value zero points go to a per-channel-group accumulator.
// ---------------------------------------------------------------------------
struct Group2 {
  u32x2 k[4];   // block u: codes of channels 32qd..32qd+31, token l%16
  u32x2 v[4];   // block u: tokens 4qd..4qd+3 of channels 16j + l%16
  float ks[2];  // as Group4: K scales of channels 8(l/4) + koff_pair(l)
  float vs[2];  // V scales (channel groups 0, 1) of token l of the group
  uint32_t kz;  // zero points of those K channels (bytes 0, 1)
  uint32_t vz;  // zero points of those V scales (bytes 0, 1)
  __device__ explicit Group2(int = 0) {}
};

__device__ __forceinline__ u32x2 bld8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2,
                            __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStreamPolicy));
}

// 2-bit codes as FP4: a code u in the low two bits of a nibble (00uu) is
// the OCP FP4 (E2M1) value u / 2 exactly, so a dword masked with kFields02
// (fields 0 and 2 of every byte), or shifted right by 2 and masked (fields
// 1 and 3), converts to exact fp16 codes one byte -- two codes -- per
// hardware FP4 conversion (scale 2).
// Bytes B0 and B0 + 1 of a masked dword (two 2-bit codes in the low bits
// of each nibble) as four exact fp16 codes: byte B0's low then high nibble,
// then byte B0 + 1's.
template <int B0>
__device__ __forceinline__ f16x4 uint2_bytes(uint32_t y) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y, 2.0f, B0);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y, 2.0f, B0 + 1);
  return f16x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ f16x8 uint2_operand(uint32_t y) {
  return cat(uint2_bytes<0>(y), uint2_bytes<2>(y));
}
constexpr uint32_t kFields02 = 0x33333333u;  // fields 0 and 2 of every byte

// pm, pz as for load_group4 (the scale and zero-point rows are those of the
// affine INT4 layout).
__device__ __forceinline__ void load_group2(Group2 &t, const DecodeArgs &a, const int (&ph)[4],
                                            int pm, int pz, int h, int lane) {
  constexpr int kRow = 40;
  const int H = a.num_kv_heads;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t chunk = (size_t)ph[u] * H + h;
    t.k[u] = bld8(make_rsrc(a.k_codes + chunk * 512, 512), 8 * lane);
    t.v[u] = bld8(make_rsrc(a.v_codes + chunk * 512, 512), 8 * lane);
  }
  const size_t chunk = (size_t)pm * H + h;
  const int2 ko = koff_pair(lane);
  const float *krow = a.k_scales + chunk * kRow;
  const float *vrow = a.v_scales + chunk * kRow;
  const float *ksp = krow + 8 * ((lane >> 2) & 3);
  const float2 vs = *reinterpret_cast<const float2 *>(vrow + 2 * (lane & 15));
  t.ks[0] = ksp[ko.x];
  t.ks[1] = ksp[ko.y];
  t.vs[0] = vs.x;
  t.vs[1] = vs.y;
  const uint8_t *kzp = reinterpret_cast<const uint8_t *>(krow + 32) + 8 * ((lane >> 2) & 3);
  t.kz = (uint32_t)kzp[ko.x] | ((uint32_t)kzp[ko.y] << 8);
  const float *zrow = a.v_scales + ((size_t)pz * H + h) * kRow;
  t.vz = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(zrow + 32) +
                                             8 * (lane >> 4) + 2 * (lane & 3));
}

// Element (or float) e of the operand of key chunk J: channel (within the
// 16 of dword J / 2) 4(e/2) + J%2 + 2(e%2).
template <int J>
__device__ __forceinline__ int k2g_idx(int e) {
  return 4 * (e >> 1) + (J & 1) + 2 * (e & 1);
}

__device__ __forceinline__ void compute_group2(Softmax &st, f32x4 (&vb)[2], const Group2 &t,
                                               const f16 *qs, float *scl, float qk_scale,
                                               int lane, int n, int qd) {
  // stage the group's scales and zero points in this wave's LDS slot
  {
    const int2 ko = koff_pair(lane);
    scl[8 * (lane >> 2) + ko.x] = t.ks[0];
    scl[8 * (lane >> 2) + ko.y] = t.ks[1];
    scl[256 + 8 * (lane >> 2) + ko.x] = (float)(t.kz & 0xFFu);
    scl[256 + 8 * (lane >> 2) + ko.y] = (float)(t.kz >> 8);
    *reinterpret_cast<float2 *>(scl + 384 + 2 * lane) =
        float2{(float)(t.vz & 0xFFu), (float)(t.vz >> 8)};
  }
  *reinterpret_cast<float2 *>(scl + 128 + 2 * lane) = float2{t.vs[0], t.vs[1]};
  f32x4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto chunk = [&](auto jc) {
    constexpr int J = decltype(jc)::value;
    const int base = 32 * qd + 16 * (J >> 1);  // the 16 channels of dword J / 2
    const f16x8 q0 = *reinterpret_cast<const f16x8 *>(qs + n * kQRow + base);
    const f16x8 q1 = *reinterpret_cast<const f16x8 *>(qs + n * kQRow + base + 8);
    float sv[16], zv[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(scl + base + 4 * i);
      const f32x4 z = *reinterpret_cast<const f32x4 *>(scl + 256 + base + 4 * i);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sv[4 * i + c] = a[c];
        zv[4 * i + c] = z[c];
      }
    }
    uint32_t hi[4], lo[4], zs[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int c0 = k2g_idx<J>(2 * e2), c1 = k2g_idx<J>(2 * e2 + 1);
      const float x0 = (float)(c0 < 8 ? q0[c0] : q1[c0 - 8]) * sv[c0];
      const float x1 = (float)(c1 < 8 ? q0[c1] : q1[c1 - 8]) * sv[c1];
      split_hi_lo(x0, x1, hi[e2], lo[e2]);
      zs[e2] = pack_rtz(-zv[c0], -zv[c1]);  // small integers: exact
    }
    const f16x8 bhi = pairs_to_f16x8(hi), blo = pairs_to_f16x8(lo);
    const f16x8 zsub = pairs_to_f16x8(zs);
    f16x8 av[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t x = t.k[u][J >> 1];
      av[u] = uint2_operand((J & 1) ? ((x >> 2) & kFields02) : (x & kFields02)) + zsub;
      acc[u] = mfma32(av[u], bhi, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = mfma32(av[u], blo, acc[u]);
  };
  chunk(std::integral_constant<int, 0>{});
  chunk(std::integral_constant<int, 1>{});
  chunk(std::integral_constant<int, 2>{});
  chunk(std::integral_constant<int, 3>{});
  f32x4 pg[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] *= qk_scale;
  softmax_update4(st, vb, acc, pg, kSlackInt2);
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const f32x4 &p0 = pg[2 * pr], &p1 = pg[2 * pr + 1];
    const float *vsp = scl + 128 + 2 * (32 * pr + 4 * qd);
    const f32x4 va0 = *reinterpret_cast<const f32x4 *>(vsp);        // tokens 0,1 of b0
    const f32x4 va1 = *reinterpret_cast<const f32x4 *>(vsp + 4);    // tokens 2,3 of b0
    const f32x4 vb0 = *reinterpret_cast<const f32x4 *>(vsp + 32);   // tokens 0,1 of b1
    const f32x4 vb1 = *reinterpret_cast<const f32x4 *>(vsp + 36);   // tokens 2,3 of b1
    const f32x4 g0a = {va0[0], va0[2], va1[0], va1[2]}, g1a = {va0[1], va0[3], va1[1], va1[3]};
    const f32x4 g0b = {vb0[0], vb0[2], vb1[0], vb1[2]}, g1b = {vb0[1], vb0[3], vb1[1], vb1[3]};
    const f16x8 pb0 = p_operand(p0 * g0a, p1 * g0b);
    const f16x8 pb1 = p_operand(p0 * g1a, p1 * g1b);
    // the value zero points of the slots' tokens, negated, per channel group
    const float *zp = scl + 384 + 2 * (32 * pr + 4 * qd);
    const f32x4 za0 = *reinterpret_cast<const f32x4 *>(zp);
    const f32x4 za1 = *reinterpret_cast<const f32x4 *>(zp + 4);
    const f32x4 zb0 = *reinterpret_cast<const f32x4 *>(zp + 32);
    const f32x4 zb1 = *reinterpret_cast<const f32x4 *>(zp + 36);
    const f16x8 nz0 = {(f16)-za0[0], (f16)-za0[2], (f16)-za1[0], (f16)-za1[2],
                       (f16)-zb0[0], (f16)-zb0[2], (f16)-zb1[0], (f16)-zb1[2]};
    const f16x8 nz1 = {(f16)-za0[1], (f16)-za0[3], (f16)-za1[1], (f16)-za1[3],
                       (f16)-zb0[1], (f16)-zb0[3], (f16)-zb1[1], (f16)-zb1[3]};
    uint32_t y[2][2][2];  // [block of the pair][dword][field parity]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t x = t.v[2 * pr + u][w];
        y[u][w][0] = x & kFields02;
        y[u][w][1] = (x >> 2) & kFields02;
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = j & 3, w = jj >> 1, hf = j >> 2;
      const f16x8 av = (jj & 1) ? cat(uint2_bytes<2>(y[0][w][hf]), uint2_bytes<2>(y[1][w][hf]))
                                : cat(uint2_bytes<0>(y[0][w][hf]), uint2_bytes<0>(y[1][w][hf]));
      st.o[j] = mfma32(av, j < 4 ? pb0 : pb1, st.o[j]);
    }
    vb[0] = mfma32(nz0, pb0, vb[0]);
    vb[1] = mfma32(nz1, pb1, vb[1]);
  }
}

// DT: kInt4, kInt4Affine or kInt2Affine on the generic layout
template <int DT>
__device__ void stream_int4(Softmax &st, const DecodeArgs &a, SharedLds &sh, int b, int h,
                            int p, int seq_len, int wave, int lane, int tid, u32x4 qrow,
                            int pre_id) {
  constexpr bool AFF = DT != kInt4;
  const int n = lane & 15, qd = lane >> 4;
  // the group's queries (fp16, zero rows past the group) stay in LDS and are
  // re-read per channel chunk, which keeps them out of the register budget
  *reinterpret_cast<u32x4 *>(&sh.s.q[tid >> 4][8 * (tid & 15)]) = qrow;
  f32x4 vb[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const int nq = kivi_quantized_len(seq_len, a.residual);
  const int n_blocks = nq / kBlock;
  const int blk0 = p * a.part_blocks;
  const int blk1 = min(n_blocks, blk0 + a.part_blocks);
  const int32_t *bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  float *scl = sh.s.scl[wave];
  for (int c0 = blk0; c0 < blk1; c0 += kIdChunk) {
    const int c1 = min(blk1, c0 + kIdChunk);
    stage_ids(sh, bt, c0, c1, tid, pre_id, c0 == blk0);
    const int ngroups = (c1 - c0) / 4;
    const int cnt = wave < ngroups ? (ngroups - wave + kWaves - 1) / kWaves : 0;
    using Unit = typename std::conditional<DT == kInt2Affine, Group2, Group4>::type;
    auto load = [&](Unit &t, int k) {
      const int j0 = 4 * (wave + kWaves * k);
      const int ph[4] = {uniform(sh.s.ids[j0]), uniform(sh.s.ids[j0 + 1]),
                         uniform(sh.s.ids[j0 + 2]), uniform(sh.s.ids[j0 + 3])};
      // a per-lane LDS read: selecting among ph[] per lane would become a
      // private-array access, whose scratch load joins the in-order vmcnt
      // queue and makes every group wait for all loads in flight
      if constexpr (DT == kInt2Affine) {
        load_group2(t, a, ph, sh.s.ids[j0 + (lane >> 4)], sh.s.ids[j0 + ((lane & 15) >> 2)], h,
                    lane);
      } else {
        load_group4<AFF>(t, a, ph, sh.s.ids[j0 + (lane >> 4)],
                         sh.s.ids[j0 + ((lane & 15) >> 2)], h, lane);
      }
    };
    auto compute = [&](Unit &t, int) {
      if constexpr (DT == kInt2Affine) {
        compute_group2(st, vb, t, &sh.s.q[0][0], scl, a.qk_scale, lane, n, qd);
      } else {
        compute_group4<AFF>(st, vb, t, &sh.s.q[0][0], scl, a.qk_scale, lane, n, qd);
      }
    };
    pipeline<Unit>(cnt, load, compute);
  }
  // the value bias of each channel group, once into its four tiles
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] += vb[j >> 2];
}

// ---------------------------------------------------------------------------
// INT4 with a query group of at most 4: compact score layout.  Four heads
// fill only four of the score product's sixteen columns, so each product
// carries the hi and the lo part of q' in two column banks, and the four
// blocks' scores end in one register set: lane (n, qd) holds tokens
// 4qd..4qd+3 of block n/4 for head n%4, and the softmax runs on four values
// per lane instead of sixteen.  q' = q * s_c is formed once per lane for two
// channels of the four heads and shared through LDS.
// ---------------------------------------------------------------------------

// One score operand serves all four blocks: column 4b + h carries head h's
// hi part of q' in the even banks b and its lo part in the odd banks, so
// block u's product holds hi and lo of head h in banks (0, 1) and again in
// (2, 3).  Adding each even bank's odd neighbour gives the score in banks 0
// and 2; moving block u's score into bank u packs the four blocks into one
// register set (lane (n, qd) = block n/4, head n%4, tokens 4qd..4qd+3).
constexpr int kQuadIdentity = 0xE4;  // DPP quad_perm [0, 1, 2, 3]
__device__ __forceinline__ float hi_plus_lo(float x) {
  return x + dpp_f32<kRowShl + 4>(0.0f, x);  // even banks: bank + next bank
}
__device__ __forceinline__ f32x4 pack_scores(const f32x4 (&acc)[4]) {
  f32x4 s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float c = hi_plus_lo(acc[0][i]);                                    // bank 0
    c = dpp_f32<kQuadIdentity, 0x4>(c, hi_plus_lo(acc[2][i]));          // bank 2
    c = dpp_f32<kRowShr + 4, 0x2>(c, hi_plus_lo(acc[1][i]));            // bank 1 <- 0
    s[i] = dpp_f32<kRowShr + 4, 0x8>(c, hi_plus_lo(acc[3][i]));         // bank 3 <- 2
  }
  return s;
}
// A value valid in banks 0 and 2 (hi + lo of a column product) in every bank.
__device__ __forceinline__ float all_banks(float x) {
  const float c = hi_plus_lo(x);
  return dpp_f32<kRowShr + 4, 0xA>(c, c);
}

// Online softmax on compact scores.  The running max moves only when some
// score exceeds it by more than the slack; only then is the head-wide max
// taken (over the four banks and the four row groups).
__device__ __forceinline__ void softmax_update_c(Softmax &st, f32x4 (&vb)[4], const f32x4 &s,
                                                 f32x4 &p, float slack) {
  const float lm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  if (__any(lm > st.m + slack)) {
    const float bm = max_over_quads(bank_max(lm));
    const bool need = bm > st.m + slack;
    const float mn = need ? bm : st.m;
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - mn) : 1.0f;
    st.l *= alpha;
    // o column n belongs to head n; for n < 4 that is this lane's head
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= alpha;
#pragma unroll
    for (int g = 0; g < 4; ++g) vb[g] *= alpha;
    st.m = mn;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - st.m);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
}

__device__ __forceinline__ uint32_t pack_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(f16)a, (f16)b});
}

// P^T operand of block pair pr (blocks 2pr, 2pr+1) for lanes n < 4 from
// the compact p dwords d[0] (tokens 0,1) and d[1] (tokens 2,3).
template <int PR>
__device__ __forceinline__ f16x8 p_operand_c(const uint32_t (&d)[2]) {
  const u32x4 w = {dpp_u32<kRowShl + 8 * PR>(0u, d[0]), dpp_u32<kRowShl + 8 * PR>(0u, d[1]),
                   dpp_u32<kRowShl + 8 * PR + 4>(0u, d[0]),
                   dpp_u32<kRowShl + 8 * PR + 4>(0u, d[1])};
  return u4_to_f16x8(w);
}

// The bias operand's rows are all alike, so its product adds the same
// value to every channel row of a channel group's four tiles: it goes to
// one accumulator per group (vb), added to o once at the end, instead of
// one product per tile.
template <int PR, bool AFF>
__device__ __forceinline__ void value_pair_c(Softmax &st, f32x4 (&vb)[4], const Group4C &t,
                                             const f16x8 &pb0, const f16x8 &pb1) {
  f16x8 abias0, abias1;
  if constexpr (AFF) {
    const u32x4 w = {row_bcast<8 + 4 * PR>(t.zw), row_bcast<9 + 4 * PR>(t.zw),
                     row_bcast<10 + 4 * PR>(t.zw), row_bcast<11 + 4 * PR>(t.zw)};
    abias0 = zp_value_bias<0>(w);
    abias1 = zp_value_bias<1>(w);
  } else {
    const f16 b0 = (f16)-1032.0f, b1 = (f16)-1152.0f;
    abias0 = abias1 = f16x8{b0, b0, b1, b1, b0, b0, b1, b1};
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = pair_tile(t.v[2 * PR][j >> 1], t.v[2 * PR + 1][j >> 1], j & 1);
    const f16x8 av = AFF ? uint4x8_to_f16_biased(w) : int4x8_to_f16_biased(w);
    st.o[j] = mfma32(av, j < 4 ? pb0 : pb1, st.o[j]);
  }
  vb[0] = mfma32(abias0, pb0, vb[0]);
  vb[1] = mfma32(abias1, pb1, vb[1]);
}

// qv[hh]: this lane's query values of head hh at channels 8(lane/4) +
// koff_pair(lane), times 1/16 for the high-nibble slots; qb: this wave's q'
// rows; qrd: dword offset of this lane's score-operand row (hi row of head
// n%4 in even banks, lo row in odd banks) and row group.
template <bool AFF>
__device__ __forceinline__ void compute_group4c(Softmax &st, f32x4 (&vb)[4], const Group4C &t,
                                                const float (&qv)[4][2], uint32_t *qb, int qrd,
                                                float qk_scale, int lane, int n) {
  // q' of this lane's two channels for the four heads (dword `lane` of each row)
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    uint32_t hi, lo;
    split_hi_lo(qv[hh][0] * t.ks[0], qv[hh][1] * t.ks[1], hi, lo);
    qb[hh * kQbRow + lane] = hi;
    qb[(4 + hh) * kQbRow + lane] = lo;
  }
  // every row of the offset operand is the conversion's per-slot offset
  // (affine: the zero points of this lane's channels, per chunk j)
  const f16 o_lo = (f16)8.0f, o_hi = (f16)1152.0f;
  const f16x8 aoff_sym = {o_lo, o_lo, o_hi, o_hi, o_lo, o_lo, o_hi, o_hi};
  f16x8 bq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bq[j] = u4_to_f16x8(*reinterpret_cast<const u32x4 *>(qb + qrd + 4 * j));
  f32x4 acc[4], ac = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f16x8 av = AFF ? uint4x8_to_f16_koff(t.k[u][j]) : int4x8_to_f16_koff(t.k[u][j]);
      acc[u] = mfma32(av, bq[j], acc[u]);
    }
    f16x8 aoff = aoff_sym;
    if constexpr (AFF) {
      // zero-point dwords 2j, 2j+1 of the row (channels 8j..8j+7)
      uint32_t d0, d1;
      if (j == 0) { d0 = row_bcast<0>(t.zw); d1 = row_bcast<1>(t.zw); }
      else if (j == 1) { d0 = row_bcast<2>(t.zw); d1 = row_bcast<3>(t.zw); }
      else if (j == 2) { d0 = row_bcast<4>(t.zw); d1 = row_bcast<5>(t.zw); }
      else { d0 = row_bcast<6>(t.zw); d1 = row_bcast<7>(t.zw); }
      aoff = zp_key_offsets(d0, d1);
    }
    ac = mfma32(aoff, bq[j], ac);
  }
  // every row of ac holds the offsets' products with head n%4's hi / lo
  const float off = all_banks(ac[0]);
  f32x4 s = pack_scores(acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = (s[i] - off) * qk_scale;
  f32x4 p;
  softmax_update_c(st, vb, s, p, kSlackInt4);
  // weights times the V scales of this lane's tokens (channel groups 0, 1)
  // tokens 2, 3 of every 4 meet value codes stored as 1152 + 16 code
  const float p2 = p[2] * 0.0625f, p3 = p[3] * 0.0625f;
  const uint32_t d0[2] = {pack_rne(p[0] * t.vsa[0], p[1] * t.vsa[2]),
                          pack_rne(p2 * t.vsb[0], p3 * t.vsb[2])};
  const uint32_t d1[2] = {pack_rne(p[0] * t.vsa[1], p[1] * t.vsa[3]),
                          pack_rne(p2 * t.vsb[1], p3 * t.vsb[3])};
  value_pair_c<0, AFF>(st, vb, t, p_operand_c<0>(d0), p_operand_c<0>(d1));
  value_pair_c<1, AFF>(st, vb, t, p_operand_c<1>(d0), p_operand_c<1>(d1));
}

// ---------------------------------------------------------------------------
// 2-bit affine KIVI on the compact layout, codes converted as FP4 nibbles
// (uint2_bytes above).  Key codes: byte b of a lane's dword w holds
// channels 16w + 4b + f at bits 2f, so the operand of (w, field parity h)
// holds channels 16w + 4b + h and 16w + 4b + h + 2 in slots 2b, 2b + 1.
// Value codes are stored so that each byte holds two
// consecutive tokens of two tiles (the layout in kvq.h): one conversion
// gives a tile's two tokens, four give its operand of a block pair.
// ---------------------------------------------------------------------------
struct Group2C {
  u32x2 k[4];   // block u: codes of channels 32qd..32qd+31, token l%16
  u32x2 v[4];   // block u: tokens 4qd..4qd+3 of channels 16j + l%16, j = 0..7
  float ks[2];
  f32x4 vsa, vsb;
  uint32_t zw;  // as Group4C
  __device__ explicit Group2C(int = 0) {}
};

// Channel (within its 32) of the first of lane l's two q' channels: operand
// J = (l/4)%4, slot pair i = l%4 -> 16(J/2) + 4i + J%2; the second is + 2.
__device__ __forceinline__ int k2_chan(int lane) {
  const int J = (lane >> 2) & 3, i = lane & 3;
  return 16 * (J >> 1) + 4 * i + (J & 1);
}

__device__ __forceinline__ void load_group2c(Group2C &t, const DecodeArgs &a, const int (&ph)[4],
                                             int pm, int pv, int h, int lane) {
  constexpr int kRow = 40;
  const int H = a.num_kv_heads;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t chunk = (size_t)ph[u] * H + h;
    t.k[u] = bld8(make_rsrc(a.k_codes + chunk * 512, 512), 8 * lane);
    t.v[u] = bld8(make_rsrc(a.v_codes + chunk * 512, 512), 8 * lane);
  }
  const float *krow = a.k_scales + ((size_t)pm * H + h) * kRow;
  const int c = k2_chan(lane);
  t.ks[0] = krow[c];
  t.ks[1] = krow[c + 2];
  const float *vsp = a.v_scales + ((size_t)pv * H + h) * kRow + 8 * (lane >> 4);
  t.vsa = ld16f(vsp);
  t.vsb = ld16f(vsp + 4);
  const int n = lane & 15;
  const float *zrow = (n < 8 ? a.k_scales : a.v_scales) + ((size_t)pm * H + h) * kRow + 32;
  t.zw = reinterpret_cast<const uint32_t *>(zrow)[n & 7];
}

// The zero-point bytes of this lane's dword zw (see Group4C) as fp16 pairs,
// exact (a byte z < 16 read as an E4M3 byte is z / 512): z[0] = bytes 0
// and 2, z[1] = bytes 1 and 3.  K dwords (lanes n < 8) hold channels
// 4n .. 4n+3; V dwords (lanes 8 + w) hold tokens 2(w%2), 2(w%2)+1 of block
// w/2 for channel groups 0, 1 (the group-transposed rows).  Converted once
// per group; the operands below are row broadcasts of them.
__device__ __forceinline__ void zp2_pairs(uint32_t zw, uint32_t (&z)[2]) {
  z[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
      __builtin_amdgcn_perm(zw, zw, 0x0C0C0200u), 512.0f, false));
  z[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
      __builtin_amdgcn_perm(zw, zw, 0x0C0C0301u), 512.0f, false));
}

// Key offset operand J: the zero points z of slots (2i, 2i+1) = channels
// 16(J/2) + 4i + J%2 and + 2, i.e. pair J%2 of K dword 4(J/2) + i.
template <int J>
__device__ __forceinline__ f16x8 zp2_key_offsets(const uint32_t (&z)[2]) {
  const u32x4 r = {row_bcast<4 * (J >> 1) + 0>(z[J & 1]), row_bcast<4 * (J >> 1) + 1>(z[J & 1]),
                   row_bcast<4 * (J >> 1) + 2>(z[J & 1]), row_bcast<4 * (J >> 1) + 3>(z[J & 1])};
  return u4_to_f16x8(r);
}

// Zero points (as fp16, exact) of the slots of block pair PR for channel
// group G: tokens 0..3 of block 2PR, then of block 2PR+1 (pair G of V
// dwords 4PR .. 4PR+3).
template <int PR, int G>
__device__ __forceinline__ f16x8 zp2_value_points(const uint32_t (&z)[2]) {
  const u32x4 r = {row_bcast<8 + 4 * PR>(z[G]), row_bcast<9 + 4 * PR>(z[G]),
                   row_bcast<10 + 4 * PR>(z[G]), row_bcast<11 + 4 * PR>(z[G])};
  return u4_to_f16x8(r);
}

// Value product of block pair PR.  Tile j (jj = j % 4) is in dword jj / 2
// of each block, bytes 2(jj % 2) and 2(jj % 2) + 1 (tokens 0, 1 and 2, 3),
// among fields 0 and 2 for tiles 0..3 and fields 1 and 3 for tiles 4..7.
// vb[2 + g] takes the weights times the zero points.
template <int PR>
__device__ __forceinline__ void value_pair2c(Softmax &st, f32x4 (&vb)[4], const Group2C &t,
                                             const uint32_t (&z)[2], const f16x8 &pb0,
                                             const f16x8 &pb1) {
  uint32_t y[2][2][2];  // [block of the pair][dword][field parity]
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t x = t.v[2 * PR + u][w];
      y[u][w][0] = x & kFields02;
      y[u][w][1] = (x >> 2) & kFields02;
    }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int jj = j & 3, w = jj >> 1, hf = j >> 2;
    const f16x8 av = (jj & 1) ? cat(uint2_bytes<2>(y[0][w][hf]), uint2_bytes<2>(y[1][w][hf]))
                              : cat(uint2_bytes<0>(y[0][w][hf]), uint2_bytes<0>(y[1][w][hf]));
    st.o[j] = mfma32(av, j < 4 ? pb0 : pb1, st.o[j]);
  }
  vb[2] = mfma32(zp2_value_points<PR, 0>(z), pb0, vb[2]);
  vb[3] = mfma32(zp2_value_points<PR, 1>(z), pb1, vb[3]);
}

__device__ __forceinline__ void compute_group2c(Softmax &st, f32x4 (&vb)[4], const Group2C &t,
                                                const float (&qv)[4][2], uint32_t *qb, int qrd,
                                                float qk_scale, int lane, int n) {
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    uint32_t hi, lo;
    split_hi_lo(qv[hh][0] * t.ks[0], qv[hh][1] * t.ks[1], hi, lo);
    qb[hh * kQbRow + lane] = hi;
    qb[(4 + hh) * kQbRow + lane] = lo;
  }
  f16x8 bq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bq[j] = u4_to_f16x8(*reinterpret_cast<const u32x4 *>(qb + qrd + 4 * j));
  f32x4 acc[4], ac = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t x = t.k[u][w];
      acc[u] = mfma32(uint2_operand(x & kFields02), bq[2 * w], acc[u]);
      acc[u] = mfma32(uint2_operand((x >> 2) & kFields02), bq[2 * w + 1], acc[u]);
    }
  }
  uint32_t z[2];
  zp2_pairs(t.zw, z);
  ac = mfma32(zp2_key_offsets<0>(z), bq[0], ac);
  ac = mfma32(zp2_key_offsets<1>(z), bq[1], ac);
  ac = mfma32(zp2_key_offsets<2>(z), bq[2], ac);
  ac = mfma32(zp2_key_offsets<3>(z), bq[3], ac);
  const float off = all_banks(ac[0]);
  f32x4 s = pack_scores(acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = (s[i] - off) * qk_scale;
  f32x4 p;
  softmax_update_c(st, vb, s, p, kSlackInt2);
  // weights times the V scales of this lane's tokens (channel groups 0, 1)
  const uint32_t d0[2] = {pack_rne(p[0] * t.vsa[0], p[1] * t.vsa[2]),
                          pack_rne(p[2] * t.vsb[0], p[3] * t.vsb[2])};
  const uint32_t d1[2] = {pack_rne(p[0] * t.vsa[1], p[1] * t.vsa[3]),
                          pack_rne(p[2] * t.vsb[1], p[3] * t.vsb[3])};
  value_pair2c<0>(st, vb, t, z, p_operand_c<0>(d0), p_operand_c<0>(d1));
  value_pair2c<1>(st, vb, t, z, p_operand_c<1>(d0), p_operand_c<1>(d1));
}

template <int DT> struct CompactUnit { using T = Group4C; };
template <> struct CompactUnit<kInt2Affine> { using T = Group2C; };

// DT: kInt4, kInt4Affine or kInt2Affine
template <int DT>
__device__ void stream_int4c(Softmax &st, const DecodeArgs &a, SharedLds &sh, int b, int h,
                             int p, int seq_len, int wave, int lane, int tid, u32x4 qrow,
                             int pre_id) {
  const int n = lane & 15, qd = lane >> 4;
  *reinterpret_cast<u32x4 *>(&sh.s.q[tid >> 4][8 * (tid & 15)]) = qrow;
  uint32_t *qb = &sh.s.qb[wave][0][0][0];
  __syncthreads();
  constexpr bool AFF = DT != kInt4;
  float qv[4][2];
  if constexpr (DT == kInt2Affine) {
    const int c = 32 * qd + k2_chan(lane);
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      qv[hh][0] = (float)sh.s.q[hh][c];
      qv[hh][1] = (float)sh.s.q[hh][c + 2];
    }
  } else {
    const int2 ko = koff_pair(lane);
    const int c = 8 * (lane >> 2);
    // high-nibble slots (odd lanes) carry 16 x code: their q' is taken / 16
    const float f = (lane & 1) ? 0.0625f : 1.0f;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      qv[hh][0] = (float)sh.s.q[hh][c + ko.x] * f;
      qv[hh][1] = (float)sh.s.q[hh][c + ko.y] * f;
    }
  }
  const int qrd = ((n & 4) ? 4 + (n & 3) : (n & 3)) * kQbRow + 16 * qd;
  // from one head per lane (lanes n < 4, as the window left it) to the
  // compact layout: every bank takes head n%4's running max, the sum stays
  // in bank 0 (the banks' shares are added back at the end)
  st.m = dpp_f32<kRowShr + 4, 0x2>(st.m, st.m);
  st.m = dpp_f32<kRowShr + 8, 0x4>(st.m, st.m);
  st.m = dpp_f32<kRowShr + 12, 0x8>(st.m, st.m);
  st.l = n < 4 ? st.l : 0.0f;
  f32x4 vb[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) vb[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nq = kivi_quantized_len(seq_len, a.residual);
  const int n_blocks = nq / kBlock;
  const int blk0 = p * a.part_blocks;
  const int blk1 = min(n_blocks, blk0 + a.part_blocks);
  const int32_t *bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  for (int c0 = blk0; c0 < blk1; c0 += kIdChunk) {
    const int c1 = min(blk1, c0 + kIdChunk);
    stage_ids(sh, bt, c0, c1, tid, pre_id, c0 == blk0);
    const int ngroups = (c1 - c0) / 4;
    const int cnt = wave < ngroups ? (ngroups - wave + kWaves - 1) / kWaves : 0;
    using Unit = typename CompactUnit<DT>::T;
    auto load = [&](Unit &t, int k) {
      const int j0 = 4 * (wave + kWaves * k);
      const int ph[4] = {uniform(sh.s.ids[j0]), uniform(sh.s.ids[j0 + 1]),
                         uniform(sh.s.ids[j0 + 2]), uniform(sh.s.ids[j0 + 3])};
      if constexpr (DT == kInt2Affine) {
        load_group2c(t, a, ph, sh.s.ids[j0 + (lane >> 4)], sh.s.ids[j0 + (n >> 2)], h, lane);
      } else {
        load_group4c<AFF>(t, a, ph, sh.s.ids[j0 + (lane >> 4)], sh.s.ids[j0 + (n >> 2)], h,
                          lane);
      }
    };
    auto compute = [&](Unit &t, int) {
      if constexpr (DT == kInt2Affine) {
        compute_group2c(st, vb, t, qv, qb, qrd, a.qk_scale, lane, n);
      } else {
        compute_group4c<AFF>(st, vb, t, qv, qb, qrd, a.qk_scale, lane, n);
      }
    };
    pipeline<Unit>(cnt, load, compute);
  }
  if constexpr (DT == kInt2Affine) {
    // tile j: remove the zero points of its channel group j / 4
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] -= vb[2 + (j >> 2)];
  } else {
    // the value bias of each channel group, once into its four tiles
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] += vb[j >> 2];
  }
  // back to one head per lane (n < 4): this lane's share of head n's sum
  st.l = bank_sum(st.l);
}

// fp16 residual ring of an INT4 cache: tokens nq .. seq_len-1, two 16-token
// tiles per step (wave w takes tile pairs w, w+4, ...).
__device__ void stream_ring(Softmax &st, const DecodeArgs &a, int b, int h, int seq_len,
                            int wave, int lane) {
  const int n = lane & 15, qd = lane >> 4;
  u32x4 qr[4];
  load_q(qr, a, b, h, n, qd);
  f16x8 bq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bq[j] = u4_to_f16x8(qr[j]);
  const int nq = kivi_quantized_len(seq_len, a.residual);
  // last position this lane's column sees (several queries per row: the
  // INT4 groups end at least a residual window before the newest token, so
  // only the fp16 window needs per-column masks)
  const int last_pos = seq_len - a.n_query + (n < a.cols ? n / a.group : a.n_query - 1);
  const size_t row = (size_t)b * a.num_kv_heads + h;
  const uint16_t *kr = a.k_resid + row * a.ring * kHeadDim;
  const uint16_t *vr = a.v_resid + row * (a.ring / 4) * kHeadDim * 4;
  for (int t0 = nq + 32 * wave; t0 < seq_len; t0 += 32 * kWaves) {
    f32x4 s[2];
    u32x2 vw[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // ring slots of one 16-token tile are contiguous: nq and the ring
      // length are multiples of 16
      const int tok = t0 + 16 * u;
      const int slot0 = tok % a.ring;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 kv = ld16(kr + (size_t)(slot0 + n) * kHeadDim + 32 * qd + 8 * j);
        acc = mfma32(u4_to_f16x8(kv), bq[j], acc);
      }
      const int valid = seq_len - (tok + 4 * qd);               // tokens that exist
      const int valid_s = min(valid, last_pos + 1 - (tok + 4 * qd));  // and are seen
#pragma unroll
      for (int r = 0; r < 4; ++r) s[u][r] = r < valid_s ? acc[r] * a.qk_scale : kNegInf;
      const uint16_t *vq = vr + ((size_t)(slot0 / 4 + qd) * kHeadDim + n) * 4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x2 w = *reinterpret_cast<const u32x2 *>(vq + 16 * j * 4);
        // zero the halves of tokens past the end (the ring may hold stale data)
        if (valid <= 0) w = u32x2{0u, 0u};
        else if (valid == 1) w = u32x2{w[0] & 0xFFFFu, 0u};
        else if (valid == 2) w = u32x2{w[0], 0u};
        else if (valid == 3) w = u32x2{w[0], w[1] & 0xFFFFu};
        vw[u][j] = w;
      }
    }
    f32x4 p0, p1;
    softmax_update(st, s[0], s[1], p0, p1);
    const f16x8 pb = p_operand(p0, p1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      st.o[j] = mfma32(cat(u2_to_f16x4(vw[0][j]), u2_to_f16x4(vw[1][j])), pb, st.o[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// workgroup merge and partial / output store
// ---------------------------------------------------------------------------
__device__ void merge_and_store(const DecodeArgs &a, SharedLds &sh, Softmax &st, int b, int h,
                                int slot, bool direct, int wave, int lane, int tid) {
  const int n = lane & 15, qd = lane >> 4;
  const float lsum = sum_over_quads(st.l);
  __syncthreads();  // streaming LDS is dead from here on
  if (qd == 0) {
    sh.g.m[wave][n] = st.m;
    sh.g.l[wave][n] = lsum;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<f32x4 *>(&sh.g.o[wave][n][16 * j + 4 * qd]) = st.o[j];
  __syncthreads();
  // thread -> (column hn, channels 8*c8 .. 8*c8+7)
  const int hn = tid >> 4, c8 = tid & 15;
  if (hn >= a.cols) return;
  float big = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) big = fmaxf(big, sh.g.m[w][hn]);
  float lt = 0.0f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sh.g.m[w][hn];
    // a wave that saw no token has m = -inf and contributes nothing
    const float f = mw == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mw - big);
    lt += f * sh.g.l[w][hn];
    acc0 += f * *reinterpret_cast<const f32x4 *>(&sh.g.o[w][hn][8 * c8]);
    acc1 += f * *reinterpret_cast<const f32x4 *>(&sh.g.o[w][hn][8 * c8 + 4]);
  }
  const int qt = hn / a.group;
  const size_t row =
      ((size_t)b * a.n_query + qt) * a.num_q_heads + h * a.group + (hn - qt * a.group);
  if (direct) {
    // a query that saw no token (several queries, short row) gets zeros; a
    // non-finite sum (NaN or infinite values in the cache) stays visible
    const float inv = lt != 0.0f ? 1.0f / lt : 0.0f;
    float *out = a.out + row * kHeadDim + 8 * c8;
    *reinterpret_cast<f32x4 *>(out) = acc0 * inv;
    *reinterpret_cast<f32x4 *>(out + 4) = acc1 * inv;
  } else {
    const size_t idx = row * a.slots + slot;
    float *o = a.ws_o + idx * kHeadDim + 8 * c8;
    *reinterpret_cast<f32x4 *>(o) = acc0;
    *reinterpret_cast<f32x4 *>(o + 4) = acc1;
    if (c8 == 0) {
      a.ws_m[idx] = big;
      a.ws_l[idx] = lt;
    }
  }
}

// Fused append of row b's new token for KV head h (INT8/FP8): wave 0
// quantizes and stores K, wave 1 V, exactly as the write kernel does.
template <int DT, int KS, int VS>
__device__ __forceinline__ void append_token_q8(const DecodeArgs &a, int b, int h, int seq_len,
                                                int wave, int lane) {
  if (wave >= 2) return;
  const bool is_v = wave == 1;
  const int kind = is_v ? VS : KS;
  const int H = a.num_kv_heads;
  const int pos = seq_len - 1;
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + pos / kBlock];
  const int slot = pos % kBlock;
  const size_t chunk = (size_t)phys * H + h;
  const uint16_t *src = (is_v ? a.v_new : a.k_new) + ((size_t)b * H + h) * kHeadDim;
  const uint32_t raw = reinterpret_cast<const uint32_t *>(src)[lane];
  // the cache arrays are the caller's writable buffers (const in DecodeArgs
  // because streaming only reads them)
  float *scales = const_cast<float *>(is_v ? a.v_scales : a.k_scales);
  float2 st = {0.f, 0.f};
  if (kind == kUniform) {
    const float s = scales[h * (is_v ? a.v_head_stride : a.k_head_stride)];
    st = float2{s, s};
  } else if (kind == kChannel) {
    st = float2{scales[h * kHeadDim + 2 * lane], scales[h * kHeadDim + 2 * lane + 1]};
  }
  const CodePair q = quantize_pair<DT>(raw, kind == kToken ? kPerToken : kPerTensor, st);
  uint8_t *codes = const_cast<uint8_t *>(is_v ? a.v_codes : a.k_codes) + chunk * 2048;
  if (is_v) {
    store_v_codes(codes, slot, lane, q);
  } else {
    store_k_codes(codes, slot, lane, q);
  }
  if (kind == kToken && lane == 0) scales[chunk * kBlock + slot] = q.scale;
}

// Fused append of row b's new token for KV head h (FP16): wave 0 stores K,
// wave 1 V, as the write kernel does.
__device__ __forceinline__ void append_token_f16(const DecodeArgs &a, int b, int h, int seq_len,
                                                 int wave, int lane) {
  if (wave >= 2) return;
  const bool is_v = wave == 1;
  const int H = a.num_kv_heads;
  const int pos = seq_len - 1;
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + pos / kBlock];
  const uint16_t *src = (is_v ? a.v_new : a.k_new) + ((size_t)b * H + h) * kHeadDim;
  const uint32_t raw = reinterpret_cast<const uint32_t *>(src)[lane];
  uint8_t *chunk = const_cast<uint8_t *>(is_v ? a.v_codes : a.k_codes) +
                   ((size_t)phys * H + h) * 4096;
  if (is_v) {
    store_v_f16(chunk, pos % kBlock, lane, raw);
  } else {
    store_k_f16(chunk, pos % kBlock, lane, raw);
  }
}

// G4: INT4 cache with a query group of at most 4 (compact score layout).
// Workgroup -> (partition p, KV head h, row b).  The dispatcher deals a
// launch's workgroups to the eight XCDs in turn (workgroup i to XCD i % 8),
// and each XCD has its own L2.  Where neighbouring heads of one block share
// 128-byte lines of the scale rows (per-token rows of 64 bytes, affine KIVI
// rows of 160: a.xcd_heads), all heads of one (row, partition) go to one
// XCD: workgroup i takes head (i / 8) % H of pair bp = ((i / 8) / H) * 8 +
// i % 8, bp = b * num_parts + p.  Otherwise the plain order: partition
// fastest, then head, then row.  The grid holds the (row, partition) pairs
// padded to a multiple of 8, times H; padding workgroups exit at once.
struct WgCoord {
  int p, h, b;
  bool live;
};
__device__ __forceinline__ WgCoord wg_coord(const DecodeArgs &a) {
  const int i = blockIdx.x;
  if (a.xcd_heads) {
    const int j = i >> 3;
    const int bp = (j / a.num_kv_heads) * 8 + (i & 7);
    return {bp % a.num_parts, j % a.num_kv_heads, bp / a.num_parts,
            bp < a.num_parts * a.batch};
  }
  const int r = i / a.num_parts;
  const int b = r / a.num_kv_heads;
  return {i - r * a.num_parts, r - b * a.num_kv_heads, b, b < a.batch};
}

// Workgroups of the decode grid: (row, partition) pairs padded to a
// multiple of 8, times the KV heads (wg_coord).  A KIVI decode step
// (kvq_write_decode) adds 2 x batch x H flush workgroups after them.
__device__ __forceinline__ int decode_grid_main(const DecodeArgs &a) {
  return (a.num_parts * a.batch + 7) / 8 * 8 * a.num_kv_heads;
}

// The write arguments of one decode step's new tokens (one per row, entry b
// of k_new / v_new).  The cache arrays are the caller's writable buffers
// (const in DecodeArgs because streaming only reads them).
__device__ __forceinline__ WriteArgs step_write_args(const DecodeArgs &a) {
  WriteArgs w;
  w.k_codes = const_cast<uint8_t *>(a.k_codes);
  w.v_codes = const_cast<uint8_t *>(a.v_codes);
  w.k_scales = const_cast<float *>(a.k_scales);
  w.v_scales = const_cast<float *>(a.v_scales);
  w.k_resid = const_cast<uint16_t *>(a.k_resid);
  w.v_resid = const_cast<uint16_t *>(a.v_resid);
  w.k_new = a.k_new;
  w.v_new = a.v_new;
  w.cu_new = nullptr;
  w.block_tables = a.block_tables;
  w.seq_lens = a.seq_lens;
  w.num_kv_heads = a.num_kv_heads;
  w.max_blocks_per_seq = a.max_blocks_per_seq;
  w.k_gran = 0;  // KIVI groups fix their own granularities
  w.v_gran = 0;
  w.ring = a.ring;
  w.residual = a.residual;
  return w;
}

// Prefix sums of the rows' block counts, for the balanced partitions:
// pre[0] = 0, pre[b + 1] = blocks of rows 0 .. b.  A row of length <= 0 or
// above the host's max_seq_len counts no blocks (no workgroup streams it;
// the merge gives it zeros or NaN).  All 256 threads of the workgroup call
// it (batch <= 256); it ends with a barrier.
__device__ void row_block_prefix(const DecodeArgs &a, int *pre, int tid) {
  int x = 0;
  if (tid < a.batch) {
    const int s = a.seq_lens[tid];
    x = (s > 0 && s <= a.max_seq_len) ? (s + kBlock - 1) / kBlock : 0;
  }
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) pre[kMaxBalancedRows + 1 + wave] = x;  // wave totals
  __syncthreads();
  for (int w = 0; w < wave; ++w) x += pre[kMaxBalancedRows + 1 + w];
  pre[tid + 1] = x;
  if (tid == 0) pre[0] = 0;
  __syncthreads();
}

// The balanced range of workgroup w: blocks [start, end) of the
// concatenation, range = ceil(total / wg_per_head) blocks per workgroup.
struct BalancedRange {
  int range, start, end;
};
__device__ __forceinline__ BalancedRange balanced_range(const DecodeArgs &a, const int *pre,
                                                        int w) {
  const int total = pre[a.batch];
  const int range = max(1, (total + a.wg_per_head - 1) / a.wg_per_head);
  const int start = min(total, w * range);
  return {range, start, min(total, start + range)};
}

// out rows of (row b, KV head h): column hn of this thread (tid / 16), its
// eight channels 8 (tid % 16) ..
__device__ __forceinline__ float *out_cols(const DecodeArgs &a, int b, int h, int tid) {
  const int hn = tid >> 4, c8 = tid & 15;
  const int qt = hn / a.group;
  return a.out + (((size_t)b * a.n_query + qt) * a.num_q_heads + h * a.group +
                  (hn - qt * a.group)) * kHeadDim + 8 * c8;
}

template <int DT, int KS, int VS, bool G4>
__device__ __forceinline__ void decode_workgroup(const DecodeArgs &a, SharedLds &sh) {
  if constexpr (is_kivi(DT)) {
    const int main_wgs = decode_grid_main(a);
    if ((int)blockIdx.x >= main_wgs) {
      // A decode step's flush of the group that leaves the fp16 window at
      // the next length (K or V of one (row, KV head)).  No workgroup of
      // this launch reads what it writes or writes what it reads: the
      // decode reads groups below nq(S), and the appended token's ring slot
      // is none of the group's.
      const int f = blockIdx.x - main_wgs;
      const int r = f >> 1;
      const int fb = r / a.num_kv_heads;
      // a row longer than the launch covers (above the host's max_seq_len)
      // is left as it is, as its decode workgroups leave it
      if (fb < a.batch && a.seq_lens[fb] <= a.max_seq_len)
        int4_flush<DT>(step_write_args(a), f & 1, r - fb * a.num_kv_heads, fb,
                       *reinterpret_cast<FlushLds<DT != kInt4> *>(&sh.f));
      return;
    }
  }
  const WgCoord wc = wg_coord(a);
  if (!wc.live) return;
  const int p = wc.p;
  const int h = wc.h;
  const int b = wc.b;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // Loads that do not need the row length are issued before it arrives: the
  // partition's first block ids (within the table row; ids past the row's
  // blocks are never used) and, for INT4, the query group (one 16-byte unit
  // per thread, zero past the group).
  const int blk0 = p * a.part_blocks;
  const int pre_id = blk0 + tid < a.max_blocks_per_seq
                         ? a.block_tables[(size_t)b * a.max_blocks_per_seq + blk0 + tid]
                         : 0;
  u32x4 qrow = {0u, 0u, 0u, 0u};
  if constexpr (is_kivi(DT)) {
    const int hn = tid >> 4, c8 = tid & 15;
    if (hn < a.cols) {  // column hn: query token hn / g, head hn % g
      const int qt = hn / a.group;
      qrow = ld16(a.q + (((size_t)b * a.n_query + qt) * a.num_q_heads + h * a.group +
                         (hn - qt * a.group)) * kHeadDim + 8 * c8);
    }
  }
  const int seq_len = a.seq_lens[b];
  const bool direct = a.slots == 1;

  if (seq_len <= 0) {
    // rows of length 0: zeros (written here only when no reduce follows)
    if (direct && p == 0 && (tid >> 4) < a.cols) {
      float *out = out_cols(a, b, h, tid);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4 *>(out) = z;
      *reinterpret_cast<f32x4 *>(out + 4) = z;
    }
    return;
  }
  if (seq_len > a.max_seq_len) {
    // A row longer than the host's max_seq_len may have partitions this
    // launch does not hold (and, in a decode step, its token is not
    // appended): its outputs become NaN instead of attention over part of
    // the row (the partition merge writes them when it runs).
    if (direct && p == 0 && (tid >> 4) < a.cols) {
      float *out = out_cols(a, b, h, tid);
      const float nan = __builtin_nanf("");
      *reinterpret_cast<f32x4 *>(out) = f32x4{nan, nan, nan, nan};
      *reinterpret_cast<f32x4 *>(out + 4) = f32x4{nan, nan, nan, nan};
    }
    return;
  }

  Softmax st;
  softmax_init(st);
  if constexpr (is_kivi(DT)) {
    // the fp16 residual tokens ride with the row's last partition, so a
    // launch has no short extra workgroups to leave a ragged last round
    const int nq = kivi_quantized_len(seq_len, a.residual);
    const int n_main = max(1, (nq / kBlock + a.part_blocks - 1) / a.part_blocks);
    if (p >= n_main) return;
    if (a.k_new != nullptr && p == n_main - 1) {
      // one decode step: this workgroup streams the row's fp16 window, so it
      // stores the new token in the ring first and completes the store
      // (every counter drained, workgroup barrier) before any wave loads it
      if (wave == 0) append_token(step_write_args(a), 0, h, b, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if constexpr (G4 && DT == kInt2Affine) {
      // the 2-bit stream rescales its whole output at the end, so the
      // window follows it
      stream_int4c<DT>(st, a, sh, b, h, p, seq_len, wave, lane, tid, qrow, pre_id);
      if (p == n_main - 1 && seq_len > nq) stream_ring(st, a, b, h, seq_len, wave, lane);
    } else if constexpr (G4) {
      // the window first: its loads and arithmetic overlap the start of the
      // INT4 stream instead of trailing it with nothing else in flight
      if (p == n_main - 1 && seq_len > nq) stream_ring(st, a, b, h, seq_len, wave, lane);
      stream_int4c<DT>(st, a, sh, b, h, p, seq_len, wave, lane, tid, qrow, pre_id);
    } else {
      stream_int4<DT>(st, a, sh, b, h, p, seq_len, wave, lane, tid, qrow, pre_id);
      if (p == n_main - 1 && seq_len > nq) stream_ring(st, a, b, h, seq_len, wave, lane);
    }
  } else {
    const int n_main = ((seq_len + kBlock - 1) / kBlock + a.part_blocks - 1) / a.part_blocks;
    if (p >= n_main) return;
    if (a.k_new != nullptr && p == n_main - 1) {
      // this workgroup streams the row's last block: store the new token
      // first, complete (every counter drained) before any wave reads it
      if constexpr (is_f16_cache(DT)) {
        append_token_f16(a, b, h, seq_len, wave, lane);
      } else {
        append_token_q8<DT, KS, VS>(a, b, h, seq_len, wave, lane);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    const int blk0 = p * a.part_blocks;
    const int blk1 = min((seq_len + kBlock - 1) / kBlock, blk0 + a.part_blocks);
    stream_q8<DT, KS, VS>(st, a, sh, b, h, blk0, blk1, seq_len, wave, lane, tid, pre_id, true);
  }
  merge_and_store(a, sh, st, b, h, p, direct, wave, lane, tid);
}

// Balanced partitions (INT8 / FP8 / FP16): workgroup i takes KV head
// i % H and the range w = i / H of that head's blocks, the rows'
// blocks laid end to end in row order ([oh-bug] "KV Cache Quantization 生产实战",
// section "为什么长上下文更需要 KV Cache Quantization": every step streams
// each row's whole history, so ragged rows leave short workgroups idle when
// each row is split on its own).  The range crosses row boundaries; each
// row segment is streamed as a partition is (the row's own query group,
// online softmax, LDS merge of the four waves) and leaves one partial in
// slot w - floor(first block of the row / range) of the row, which the
// merge finds from the same prefix sums.  A decode step's new token is
// appended by the workgroup whose segment holds the row's last block.
template <int DT, int KS, int VS>
__device__ void decode_balanced(const DecodeArgs &a, SharedLds &sh, int *pre) {
  const int i = blockIdx.x;
  int h, w;
  if (a.xcd_heads) {
    // all heads of range w on one XCD (workgroup i runs on XCD i % 8), as
    // wg_coord deals them: neighbouring heads share lines of the scale rows
    const int j = i >> 3;
    h = j % a.num_kv_heads;
    w = (j / a.num_kv_heads) * 8 + (i & 7);
  } else {
    h = i % a.num_kv_heads;
    w = i / a.num_kv_heads;
  }
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  row_block_prefix(a, pre, tid);
  if (w >= a.wg_per_head) return;  // padding of the XCD-dealt grid
  const BalancedRange r = balanced_range(a, pre, w);
  if (r.start >= r.end) return;
  // first row whose blocks reach past start (binary search over pre)
  int lo = 0, hi = a.batch;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid + 1] <= r.start) lo = mid + 1;
    else hi = mid;
  }
  for (int b = lo; b < a.batch && pre[b] < r.end; ++b) {
    const int nb = pre[b + 1] - pre[b];
    if (nb == 0) continue;
    const int blk0 = max(r.start, pre[b]) - pre[b];
    const int blk1 = min(r.end, pre[b + 1]) - pre[b];
    const int seq_len = a.seq_lens[b];
    Softmax st;
    softmax_init(st);
    if (a.k_new != nullptr && blk1 == nb) {
      // this segment holds the row's last block: store the new token first
      if constexpr (is_f16_cache(DT)) {
        append_token_f16(a, b, h, seq_len, wave, lane);
      } else {
        append_token_q8<DT, KS, VS>(a, b, h, seq_len, wave, lane);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    stream_q8<DT, KS, VS>(st, a, sh, b, h, blk0, blk1, seq_len, wave, lane, tid, 0, false);
    merge_and_store(a, sh, st, b, h, w - pre[b] / r.range, false, wave, lane, tid);
  }
}

// INT8 / FP8 / FP16 and INT4 caches get separate kernels so that each is
// held to the register budget of its own occupancy.
template <int DT, int KS, int VS>
__global__ __launch_bounds__(kThreads, decode_wg_per_cu(DT, KS, VS)) void kvq_paged_decode_kernel(
    DecodeArgs a) {
  __shared__ SharedLds sh;
  if (a.balanced) {
    __shared__ int pre[kMaxBalancedRows + 1 + kWaves];
    decode_balanced<DT, KS, VS>(a, sh, pre);
    return;
  }
  decode_workgroup<DT, KS, VS, false>(a, sh);
}

// DT: kInt4 or kInt4Affine
template <int DT, bool G4>
__global__ __launch_bounds__(kThreads, decode_wg_per_cu(DT, kChannel, kToken)) void kvq_paged_decode_int4_kernel(
    DecodeArgs a) {
  static_assert(is_kivi(DT), "KIVI-grouped INT4 caches only");
  __shared__ SharedLds sh;
  decode_workgroup<DT, kChannel, kToken, G4>(a, sh);
}

// Log-sum-exp merge of the partition partials of each (row, query head):
// M = max_p m_p, w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p, in
// partition order.  One thread per 4 channels, 32 threads per (row, query
// head).  Partials are read eight at a time with indices clamped to the
// workspace's slots, so the first eight are in flight together with the
// row length; slots at or past the row's partition count (never written by
// this launch, possibly stale or uninitialised) are excluded by selects.
// More than eight partitions merge chunk by chunk with a running max.
__global__ __launch_bounds__(256) void kvq_partition_reduce_kernel(DecodeArgs a, int is_int4) {
  constexpr int kUnroll = 8;
  const int gid = blockIdx.x * 8 + (threadIdx.x >> 5);   // (b, query, hq) row
  const int c4 = threadIdx.x & 31;
  const int rows = a.batch * a.n_query * a.num_q_heads;
  const bool live = gid < rows;
  const int b = gid / (a.num_q_heads * a.n_query);
  const size_t base = (size_t)(live ? gid : rows - 1) * a.slots;
  float mv[kUnroll], lv[kUnroll];
  f32x4 ov[kUnroll];
  auto load_chunk = [&](int p0) {
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const size_t slot = base + min(p0 + i, a.slots - 1);
      mv[i] = a.ws_m[slot];
      lv[i] = a.ws_l[slot];
      ov[i] = *reinterpret_cast<const f32x4 *>(a.ws_o + slot * kHeadDim + 4 * c4);
    }
  };
  // the first chunk is in flight while the row length (and, for balanced
  // partitions, the rows' block prefix sums) arrive
  load_chunk(0);
  // balanced partitions: the row's partials are those of the ranges its
  // blocks meet (the decode kernel's prefix sums, recomputed here)
  __shared__ int pre[kMaxBalancedRows + 1 + kWaves];
  int bal_total = 0;
  if (a.balanced) {
    row_block_prefix(a, pre, threadIdx.x);
    if (live && pre[b + 1] > pre[b]) {
      const int range = balanced_range(a, pre, 0).range;
      bal_total = (pre[b + 1] - 1) / range - pre[b] / range + 1;
    }
  }
  if (!live) return;
  float *out = a.out + (size_t)gid * kHeadDim + 4 * c4;
  const int seq_len = a.seq_lens[b];
  if (seq_len <= 0) {
    *reinterpret_cast<f32x4 *>(out) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  if (seq_len > a.max_seq_len) {
    // the row is longer than the host's max_seq_len: NaN, not a partial
    // answer
    const float nan = __builtin_nanf("");
    *reinterpret_cast<f32x4 *>(out) = f32x4{nan, nan, nan, nan};
    return;
  }
  int total;
  if (a.balanced) {
    total = bal_total;
  } else if (is_int4) {
    const int nq = kivi_quantized_len(seq_len, a.residual);
    total = max(1, (nq / kBlock + a.part_blocks - 1) / a.part_blocks);
  } else {
    total = ((seq_len + kBlock - 1) / kBlock + a.part_blocks - 1) / a.part_blocks;
  }
  float big = kNegInf, lt = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < total; p0 += kUnroll) {
    if (p0 > 0) load_chunk(p0);
    float cm = big;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) cm = p0 + i < total ? fmaxf(cm, mv[i]) : cm;
    // rescale what earlier chunks summed (factor 1 for the first chunk)
    const float r = big == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(big - cm);
    lt *= r;
    acc *= r;
    big = cm;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (p0 + i < total) {
        // a partition a query saw nothing of (m = -inf) weighs 0
        const float w = mv[i] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mv[i] - big);
        lt += w * lv[i];
        acc += w * ov[i];
      }
    }
  }
  // a query that saw no token (several queries, short row) gets zeros; a
  // non-finite sum (NaN or infinite values in the cache) stays visible
  *reinterpret_cast<f32x4 *>(out) = lt != 0.0f ? acc * (1.0f / lt) : f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int DT, int KS>
void launch_v(const DecodeArgs &a, int v_kind, dim3 grid, hipStream_t s) {
  switch (v_kind) {
    case kUniform:
      hipLaunchKernelGGL((kvq_paged_decode_kernel<DT, KS, kUniform>), grid, dim3(kThreads), 0, s,
                         a);
      break;
    case kChannel:
      hipLaunchKernelGGL((kvq_paged_decode_kernel<DT, KS, kChannel>), grid, dim3(kThreads), 0, s,
                         a);
      break;
    default:
      hipLaunchKernelGGL((kvq_paged_decode_kernel<DT, KS, kToken>), grid, dim3(kThreads), 0, s,
                         a);
      break;
  }
}

template <int DT>
void launch_k(const DecodeArgs &a, int k_kind, int v_kind, dim3 grid, hipStream_t s) {
  switch (k_kind) {
    case kUniform: launch_v<DT, kUniform>(a, v_kind, grid, s); break;
    case kChannel: launch_v<DT, kChannel>(a, v_kind, grid, s); break;
    default: launch_v<DT, kToken>(a, v_kind, grid, s); break;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int dtype, int k_kind, int v_kind, int batch,
                         hipStream_t stream) {
  // one workgroup per (partition, KV head, row), ordered for the XCDs by
  // wg_coord: the (row, partition) pairs padded to a multiple of eight
  const long pairs8 = ((long)a.num_parts * batch + 7) / 8 * 8;
  // a KIVI decode step: its flush workgroups (K and V of every (row, head))
  const long flush = is_kivi(dtype) && a.k_new != nullptr ? 2L * batch * a.num_kv_heads : 0;
  // balanced: the ranges of every head, padded to a multiple of 8 ranges
  // when the heads of a range are dealt to one XCD
  const long bal = a.xcd_heads ? ((long)a.wg_per_head + 7) / 8 * 8 * a.num_kv_heads
                               : (long)a.wg_per_head * a.num_kv_heads;
  const dim3 grid(a.balanced ? (unsigned)bal : (unsigned)(pairs8 * a.num_kv_heads + flush));
  // the compact INT4 layout holds one query token's four heads per block
  if (dtype == kInt4 && a.group <= 4 && a.n_query == 1) {
    hipLaunchKernelGGL((kvq_paged_decode_int4_kernel<kInt4, true>), grid, dim3(kThreads), 0,
                       stream, a);
  } else if (dtype == kInt4) {
    hipLaunchKernelGGL((kvq_paged_decode_int4_kernel<kInt4, false>), grid, dim3(kThreads), 0,
                       stream, a);
  } else if (dtype == kInt2Affine && a.group <= 4 && a.n_query == 1) {
    hipLaunchKernelGGL((kvq_paged_decode_int4_kernel<kInt2Affine, true>), grid, dim3(kThreads),
                       0, stream, a);
  } else if (dtype == kInt2Affine) {
    hipLaunchKernelGGL((kvq_paged_decode_int4_kernel<kInt2Affine, false>), grid, dim3(kThreads),
                       0, stream, a);
  } else if (dtype == kInt4Affine && a.group <= 4 && a.n_query == 1) {
    hipLaunchKernelGGL((kvq_paged_decode_int4_kernel<kInt4Affine, true>), grid, dim3(kThreads),
                       0, stream, a);
  } else if (dtype == kInt4Affine) {
    hipLaunchKernelGGL((kvq_paged_decode_int4_kernel<kInt4Affine, false>), grid, dim3(kThreads),
                       0, stream, a);
  } else if (dtype == kBf16) {
    hipLaunchKernelGGL((kvq_paged_decode_kernel<kBf16, kUniform, kUniform>), grid, dim3(kThreads),
                       0, stream, a);
  } else if (dtype == kFp16) {
    hipLaunchKernelGGL((kvq_paged_decode_kernel<kFp16, kUniform, kUniform>), grid, dim3(kThreads),
                       0, stream, a);
  } else if (dtype == kFp8) {
    launch_k<kFp8>(a, k_kind, v_kind, grid, stream);
  } else if (dtype == kFp8E5M2) {
    launch_k<kFp8E5M2>(a, k_kind, v_kind, grid, stream);
  } else {
    launch_k<kInt8>(a, k_kind, v_kind, grid, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (a.slots == 1 && !a.balanced)) return e;
  const int rows = batch * a.n_query * a.num_q_heads;
  hipLaunchKernelGGL(kvq_partition_reduce_kernel, dim3((rows + 7) / 8), dim3(256), 0, stream, a,
                     is_kivi(dtype) ? 1 : 0);
  return hipGetLastError();
}

}  // namespace kvq
