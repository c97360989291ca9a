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

// ---------------------------------------------------------------------------
// INT4 KIVI
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(256) void kvq_int4_flush_kernel(WriteArgs a) {
  int4_flush<DT>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

__global__ __launch_bounds__(64) void kvq_int4_append_kernel(WriteArgs a) {
  append_token(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

// Flush and append in one launch: workgroups x < 2*groups flush, the rest
// append.  Only for calls that add at most one token per row: the appended
// token is then fewer than R + G positions after any token the flush reads
// from the ring, so its ring slot is never one of them.
template <int DT>
__global__ __launch_bounds__(256) void kvq_int4_flush_append_kernel(WriteArgs a, int groups) {
  if ((int)blockIdx.x < 2 * groups) {
    int4_flush<DT>(a, blockIdx.x, blockIdx.y, blockIdx.z);
  } else if (threadIdx.x < 64) {
    append_token(a, blockIdx.x - 2 * groups, blockIdx.y, blockIdx.z, threadIdx.x);
  }
}

}  // namespace

hipError_t launch_write_q8(const WriteArgs &a, int dtype, int batch, int max_new,
                           hipStream_t stream) {
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
  hipLaunchKernelGGL(kvq_int4_append_kernel, dim3(max_new, a.num_kv_heads, batch), dim3(64),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
