// Static-scale calibration: scale = max|x| / divisor over calibration
// tokens, per tensor, head or channel ([yunthe] "KV Cache量化压缩技术与vLLM
// 推理引擎显存优化实战", sections "KV Cache量化策略" (scale = max(abs(x)) /
// 127) and "配置与启动参数" (per-layer K and V scales computed from
// calibration data); [oh-bug] "KV Cache Quantization 生产实战", vLLM section
// (per-tensor and per-head FP8 scales from a random-token warmup)).
//
// Two launches.  Pass 1: workgroup (chunk, octet block, K|V) reduces its
// chunk of tokens for 64 channel octets (16-byte loads, four token lanes per
// octet, coalesced 1 KiB rows) to per-channel maxima, stored as the chunk's
// partial.  Pass 2: one workgroup per K|V folds the chunks' partials per
// channel and reduces channels to heads or to the tensor as the
// granularity asks, divides by the format's largest code and stores (or,
// accumulating, raises) the scales (per head through an LDS max; no
// global atomics).  The result does not depend on the launch shape: max
// is exact and order-free.
#include "kvq_args.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kOctBlock = 64;     // channel octets per pass-1 workgroup
constexpr int kTokLanes = 4;      // token lanes per octet

__global__ __launch_bounds__(256) void kvq_calibrate_partial_kernel(CalibArgs a) {
  __shared__ float red[kTokLanes][kOctBlock][9];  // padded
  const int chunk = blockIdx.x;
  const int ob = blockIdx.y;
  const int kv = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane_oct = tid % kOctBlock, tl = tid / kOctBlock;
  const int n_oct = a.num_kv_heads * (kHeadDim / 8);
  const int oct = ob * kOctBlock + lane_oct;
  const uint16_t *x = kv ? a.v : a.k;
  if ((kv ? a.v_scales : a.k_scales) == nullptr) return;  // not calibrated
  const int t0 = chunk * a.chunk_tokens;
  const int t1 = min(a.n_tokens, t0 + a.chunk_tokens);
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.0f;
  if (oct < n_oct) {
    // kUnroll tokens per step, all loads issued before any use; tokens past
    // the chunk are skipped by predication
    constexpr int kUnroll = 8;
    for (int t = t0 + tl; t < t1; t += kTokLanes * kUnroll) {
      u32x4 w[kUnroll];
#pragma unroll
      for (int i = 0; i < kUnroll; ++i) {
        const int ti = t + kTokLanes * i;
        w[i] = ti < t1 ? ld16_stream(x + ((size_t)ti * n_oct + oct) * 8) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kUnroll; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 p = as_f16x2(w[i][e]);
          m[2 * e] = fmaxf(m[2 * e], fabsf((float)p.x));
          m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf((float)p.y));
        }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tl][lane_oct][e] = m[e];
  __syncthreads();
  if (tl == 0 && oct < n_oct) {
    float *dst = a.partial + ((size_t)chunk * 2 + kv) * a.num_kv_heads * kHeadDim + oct * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = red[0][lane_oct][e];
#pragma unroll
      for (int l = 1; l < kTokLanes; ++l) v = fmaxf(v, red[l][lane_oct][e]);
      dst[e] = v;
    }
  }
}

// Block-wide max over 1024 threads (every thread gets the result).
__device__ __forceinline__ float block_max(float v, float *scratch) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, scratch[w]);
  return r;
}

__global__ __launch_bounds__(1024) void kvq_calibrate_finalize_kernel(CalibArgs a) {
  __shared__ float scratch[16];
  __shared__ float head_max[kMaxCalibHeads];
  const int kv = blockIdx.x;
  const int gran = kv ? a.v_gran : a.k_gran;
  float *out = kv ? a.v_scales : a.k_scales;
  if (out == nullptr) return;  // per-token granularity: nothing to calibrate
  const int tid = threadIdx.x;
  const int nch = a.num_kv_heads * kHeadDim;
  const size_t stride = (size_t)2 * nch;
  const float *part = a.partial + (size_t)kv * nch;
  for (int h = tid; h < a.num_kv_heads; h += blockDim.x) head_max[h] = 0.0f;
  __syncthreads();
  float tmax = 0.0f;
  // channel c of the 1024-thread sweep: thread tid takes c = tid, tid+1024, ...
  for (int c = tid; c < nch; c += blockDim.x) {
    float v = 0.0f;
#pragma unroll 8
    for (int q = 0; q < a.n_chunks; ++q) v = fmaxf(v, part[q * stride + c]);
    if (gran == kCalibChannel) {
      const float s = v / a.divisor;
      out[c] = a.accumulate ? fmaxf(out[c], s) : s;
    }
    tmax = fmaxf(tmax, v);
    if (gran == kCalibHead) {
      // maxima of non-negative floats order like their bit patterns
      atomicMax(reinterpret_cast<unsigned int *>(&head_max[c / kHeadDim]),
                __builtin_bit_cast(unsigned int, v));
    }
  }
  if (gran == kCalibTensor) {
    const float v = block_max(tmax, scratch);
    if (tid == 0) {
      const float s = v / a.divisor;
      out[0] = a.accumulate ? fmaxf(out[0], s) : s;
    }
  } else if (gran == kCalibHead) {
    __syncthreads();
    for (int h = tid; h < a.num_kv_heads; h += blockDim.x) {
      const float s = head_max[h] / a.divisor;
      out[h] = a.accumulate ? fmaxf(out[h], s) : s;
    }
  }
}

}  // namespace

hipError_t launch_calibrate(const CalibArgs &a, hipStream_t stream) {
  const int n_oct = a.num_kv_heads * (kHeadDim / 8);
  const dim3 grid(a.n_chunks, (n_oct + kOctBlock - 1) / kOctBlock, 2);
  hipLaunchKernelGGL(kvq_calibrate_partial_kernel, grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kvq_calibrate_finalize_kernel, dim3(2), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
