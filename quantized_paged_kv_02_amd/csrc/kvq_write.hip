// Quantize-on-write kernels.
//
// INT8 / FP8: one wavefront per (new token, KV head) quantizes the token's K
// and V vectors (128 values each, two per lane) and scatters the codes into
// the block slot given by the block table.  Symmetric rule from
// [intelli] "大模型KV Cache显存优化与量化技术实践" §3.1 对称量化算法 and
// [yunthe] "KV Cache量化压缩技术与vLLM推理引擎显存优化实战", section
// "KV Cache量化策略：INT8与FP8精度对比与选择": scale = max|x| / 127 (448 for
// E4M3), code = clamp(round(x / scale)).  Dynamic per-token scales follow
// [intelli] §3.2 动态量化策略.  fp32 division is the correctly rounded IEEE
// one (the library is built without fast-math); rounding is rintf
// (half-to-even).
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

namespace kvq {
namespace {

constexpr int kPerTensor = 0, kPerHead = 1, kPerToken = 3;

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

__device__ __forceinline__ float fp8_prescale(float x, float s) {
  if (s == 0.0f) return 0.0f;
  const float y = x / s;
  return fminf(fmaxf(y, -448.0f), 448.0f);
}

// Quantize one tensor (K or V) of one (token, KV head) and store its codes
// (and its scale for per-token granularity).
template <int DT, bool IS_V>
__device__ __forceinline__ void write_vector(const uint16_t *src, uint8_t *chunk,
                                             float *scales, int gran, int h,
                                             int slot, size_t token_scale_index) {
  const int lane = threadIdx.x;
  const uint32_t raw = reinterpret_cast<const uint32_t *>(src)[lane];
  const float x0 = half_bits_to_float(raw & 0xFFFFu);
  const float x1 = half_bits_to_float(raw >> 16);
  const int c0 = 2 * lane;
  float s0, s1;
  if (gran == kPerToken) {
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    s0 = s1 = amax / (DT == kFp8 ? 448.0f : 127.0f);
    if (lane == 0) scales[token_scale_index] = s0;
  } else if (gran == kPerTensor) {
    s0 = s1 = scales[0];
  } else if (gran == kPerHead) {
    s0 = s1 = scales[h];
  } else {
    s0 = scales[h * kHeadDim + c0];
    s1 = scales[h * kHeadDim + c0 + 1];
  }
  uint32_t q0, q1;
  if (DT == kFp8) {
    const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        fp8_prescale(x0, s0), fp8_prescale(x1, s1), 0, false);
    q0 = pk & 0xFFu;
    q1 = (pk >> 8) & 0xFFu;
  } else {
    q0 = quant_int(x0, s0, -128.0f, 127.0f) & 0xFFu;
    q1 = quant_int(x1, s1, -128.0f, 127.0f) & 0xFFu;
  }
  if (!IS_V) {
    // channels c0 and c0+1 are adjacent bytes of one 16-byte run
    *reinterpret_cast<uint16_t *>(chunk + k8_offset(slot, c0)) =
        (uint16_t)(q0 | (q1 << 8));
  } else {
    chunk[v8_offset(slot, c0)] = (uint8_t)q0;
    chunk[v8_offset(slot, c0 + 1)] = (uint8_t)q1;
  }
}

template <int DT>
__global__ __launch_bounds__(64) void kvq_write_q8_kernel(WriteArgs a) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int c_begin = a.cu_new[b];
  const int n_new = a.cu_new[b + 1] - c_begin;
  if (i >= n_new) return;
  const int pos = a.seq_lens[b] - n_new + i;
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + pos / kBlock];
  const int slot = pos % kBlock;
  const size_t chunk = (size_t)phys * a.num_kv_heads + h;
  const size_t src = ((size_t)(c_begin + i) * a.num_kv_heads + h) * kHeadDim;
  const size_t tsi = chunk * kBlock + slot;
  write_vector<DT, false>(a.k_new + src, a.k_codes + chunk * 2048, a.k_scales,
                          a.k_gran, h, slot, tsi);
  write_vector<DT, true>(a.v_new + src, a.v_codes + chunk * 2048, a.v_scales,
                         a.v_gran, h, slot, tsi);
}

// ---------------------------------------------------------------------------
// INT4 KIVI
// ---------------------------------------------------------------------------

__device__ __forceinline__ int kivi_len(int s, int residual) {
  return kivi_quantized_len(s, residual);
}

// Gather one token's 128 fp16 values of K and V for the flush: from the ring
// when the token was already cached, else from the call's new tokens.
__global__ __launch_bounds__(256) void kvq_int4_flush_kernel(WriteArgs a) {
  __shared__ f16 kx[kGroup][kHeadDim];
  __shared__ f16 vx[kGroup][kHeadDim];
  __shared__ float ksc[kHeadDim];
  __shared__ float vsc[kGroup][2];
  __shared__ int phys_s[4];

  const int gs = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int H = a.num_kv_heads;
  const int c_begin = a.cu_new[b];
  const int n_new = a.cu_new[b + 1] - c_begin;
  const int s_new = a.seq_lens[b];
  const int s_old = s_new - n_new;
  const int nq_old = kivi_len(s_old, a.residual);
  const int nq_new = kivi_len(s_new, a.residual);
  const int t0 = nq_old + kGroup * gs;
  if (t0 >= nq_new) return;

  const size_t ring_row = (size_t)b * H + h;
  // gather: 64 tokens x 64 channel pairs = 4096 pairs, 16 per thread
  for (int e = tid; e < kGroup * (kHeadDim / 2); e += 256) {
    const int tt = e >> 6;
    const int c = (e & 63) * 2;
    const int t = t0 + tt;
    uint32_t kp, vp;
    if (t < s_old) {
      const int slot = t % a.ring;
      kp = *reinterpret_cast<const uint32_t *>(
          a.k_resid + (ring_row * a.ring + slot) * kHeadDim + c);
      const uint16_t *vb = a.v_resid +
                           ((ring_row * (a.ring / 4) + slot / 4) * kHeadDim + c) * 4 +
                           (slot & 3);
      vp = (uint32_t)vb[0] | ((uint32_t)vb[4] << 16);
    } else {
      const size_t src = ((size_t)(c_begin + t - s_old) * H + h) * kHeadDim + c;
      kp = *reinterpret_cast<const uint32_t *>(a.k_new + src);
      vp = *reinterpret_cast<const uint32_t *>(a.v_new + src);
    }
    *reinterpret_cast<uint32_t *>(&kx[tt][c]) = kp;
    *reinterpret_cast<uint32_t *>(&vx[tt][c]) = vp;
  }
  if (tid < 4) {
    phys_s[tid] = a.block_tables[(size_t)b * a.max_blocks_per_seq + t0 / kBlock + tid];
  }
  __syncthreads();

  if (tid < kHeadDim) {
    // K: per-channel scale over the group's 64 tokens
    float amax = 0.0f;
    for (int tt = 0; tt < kGroup; ++tt) amax = fmaxf(amax, fabsf((float)kx[tt][tid]));
    ksc[tid] = amax / 7.0f;
  } else {
    // V: per-token scale over each 64-channel group
    const int tt = (tid - kHeadDim) >> 1;
    const int grp = tid & 1;
    float amax = 0.0f;
    for (int c = 0; c < kGroup; ++c) amax = fmaxf(amax, fabsf((float)vx[tt][grp * kGroup + c]));
    vsc[tt][grp] = amax / 7.0f;
  }
  __syncthreads();

  // scales to the pool
  if (tid < kHeadDim) {
    const int ub = tid >> 5;  // block of the group that holds this channel's scale
    a.k_scales[((size_t)phys_s[ub] * H + h) * 32 + (tid & 31)] = ksc[tid];
  } else {
    const int tt = (tid - kHeadDim) >> 1;
    const int grp = tid & 1;
    a.v_scales[(((size_t)phys_s[tt >> 4] * H + h) * kBlock + (tt & 15)) * 2 + grp] =
        vsc[tt][grp];
  }

  // K codes: 1024 dwords, 8 channels of one token each
  for (int di = tid; di < 1024; di += 256) {
    const int tt = di >> 4;
    const int d0 = (di & 15) * 8;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t q = quant_int((float)kx[tt][d0 + e], ksc[d0 + e], -8.0f, 7.0f) & 0xFu;
      word |= q << (4 * e);
    }
    uint8_t *chunk = a.k_codes + ((size_t)phys_s[tt >> 4] * H + h) * 1024;
    *reinterpret_cast<uint32_t *>(chunk + 256 * (d0 >> 5) + 16 * (tt & 15) +
                                  ((d0 & 31) >> 1)) = word;
  }
  // V codes: per block 64 units x 4 dwords; a dword holds channels
  // A = 32w + m and B = 32w + 16 + m for the unit's four tokens.
  for (int di = tid; di < 1024; di += 256) {
    const int ub = di >> 8;          // block within the group
    const int u = (di >> 2) & 63;    // 16-byte unit
    const int w = di & 3;            // dword within the unit
    const int m = u & 15;
    const int qd = u >> 4;
    const int ca = 32 * w + m;
    const int cb = ca + 16;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tt = ub * kBlock + 4 * qd + e;
      const uint32_t qa = quant_int((float)vx[tt][ca], vsc[tt][ca >> 6], -8.0f, 7.0f) & 0xFu;
      const uint32_t qb = quant_int((float)vx[tt][cb], vsc[tt][cb >> 6], -8.0f, 7.0f) & 0xFu;
      const int pa = (e >> 1) + 4 * (e & 1);
      word |= qa << (4 * pa);
      word |= qb << (4 * (pa + 2));
    }
    uint8_t *chunk = a.v_codes + ((size_t)phys_s[ub] * H + h) * 1024;
    *reinterpret_cast<uint32_t *>(chunk + 16 * u + 4 * w) = word;
  }
}

// Append the new tokens that stay fp16 to the ring.
__global__ __launch_bounds__(64) void kvq_int4_append_kernel(WriteArgs a) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int H = a.num_kv_heads;
  const int c_begin = a.cu_new[b];
  const int n_new = a.cu_new[b + 1] - c_begin;
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

}  // namespace

hipError_t launch_write_q8(const WriteArgs &a, int dtype, int batch, int max_new,
                           hipStream_t stream) {
  const dim3 grid(max_new, a.num_kv_heads, batch);
  if (dtype == kFp8) {
    hipLaunchKernelGGL(kvq_write_q8_kernel<kFp8>, grid, dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(kvq_write_q8_kernel<kInt8>, grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_write_int4(const WriteArgs &a, int batch, int max_new,
                             int max_flush_groups, hipStream_t stream) {
  if (max_flush_groups > 0) {
    hipLaunchKernelGGL(kvq_int4_flush_kernel, dim3(max_flush_groups, a.num_kv_heads, batch),
                       dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kvq_int4_append_kernel, dim3(max_new, a.num_kv_heads, batch), dim3(64),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
