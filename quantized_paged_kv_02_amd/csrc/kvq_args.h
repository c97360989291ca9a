// Kernel argument blocks and launch entry points shared by the host API
// (kvq_api.cpp) and the kernel files.  Internal to libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

enum Dtype : int {  // kvq_dtype
  kInt8 = 1, kFp8 = 2, kInt4 = 3, kFp16 = 4, kInt4Affine = 5, kFp8E5M2 = 6, kInt2Affine = 7,
  kBf16 = 8
};
// Unquantized caches (fp16 or bf16 values, no scales)
constexpr bool is_f16_cache(int dtype) { return dtype == kFp16 || dtype == kBf16; }
// KIVI-grouped caches: INT4 symmetric or affine, 2-bit affine
constexpr bool is_kivi(int dtype) {
  return dtype == kInt4 || dtype == kInt4Affine || dtype == kInt2Affine;
}
// bytes of one (block, head) code chunk of a KIVI-grouped cache
constexpr int kivi_chunk_bytes(int dtype) { return dtype == kInt2Affine ? 512 : 1024; }
// Granularity as the decode kernel sees it: a scale that is uniform over a
// (row, KV head) (per-tensor or per-head), per channel, or per token.
enum ScaleKind : int { kUniform = 0, kChannel = 1, kToken = 2 };

// Decode workgroups (four wavefronts) guaranteed resident per CU for a cache
// dtype and K / V scale kinds: the kernel's register bound and the partition
// plan's round size.  INT4, FP16 (twice the bytes in flight per unit) and
// FP8 (E4M3 or E5M2) with per-token V and non-uniform K scales need the
// larger per-wave register budget of two per CU.  (The compact 2-bit kernel
// fits three per CU in registers and LDS, but on the KIVI shape six
// partitions per row at three per CU ran 3 % slower than four at two.)
constexpr int decode_wg_per_cu(int dtype, int k_kind, int v_kind) {
  return (is_kivi(dtype) || is_f16_cache(dtype)) ? 2
         : ((dtype == kFp8 || dtype == kFp8E5M2) && v_kind == kToken && k_kind != kUniform) ? 2
                                                                      : 3;
}

struct WriteArgs {
  uint8_t *k_codes;
  uint8_t *v_codes;
  float *k_scales;
  float *v_scales;
  uint16_t *k_resid;
  uint16_t *v_resid;
  const uint16_t *k_new;
  const uint16_t *v_new;
  const int32_t *cu_new;
  const int32_t *block_tables;
  const int32_t *seq_lens;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t k_gran;        // kvq_granularity
  int32_t v_gran;
  int32_t ring;          // INT4: residual_len + group
  int32_t residual;      // INT4: residual_len
};

struct DecodeArgs {
  const uint8_t *k_codes;
  const uint8_t *v_codes;
  const float *k_scales;
  const float *v_scales;
  const uint16_t *k_resid;
  const uint16_t *v_resid;
  const uint16_t *q;
  const int32_t *block_tables;
  const int32_t *seq_lens;
  // Fused append (INT8/FP8/FP16): row b's new token, fp16 [B][H][128] at position
  // seq_lens[b] - 1, quantized and stored (codes, per-token scales) by the
  // workgroup that streams the row's last partition.  Null: no append.
  const uint16_t *k_new;
  const uint16_t *v_new;
  float *out;       // [B][Nq][Hq][128]
  float *ws_o;      // [B][Nq][Hq][slots][128] unnormalised partial outputs
  float *ws_m;      // [B][Nq][Hq][slots] partial running max (log2 domain)
  float *ws_l;      // [B][Nq][Hq][slots] partial softmax sums
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;            // Hq / H
  // Query tokens per row (1 for decode): query j of row b sits at position
  // seq_lens[b] - n_query + j and sees tokens up to it.  The score product's
  // columns are (query j, head) pairs, column n = j * group + head.
  int32_t n_query;
  int32_t cols;             // n_query * group <= 16
  int32_t max_blocks_per_seq;
  int32_t max_seq_len;      // the host's bound; longer rows get NaN outputs
  int32_t part_blocks;      // blocks per main partition
  int32_t num_parts;        // main partitions in the grid
  int32_t slots;            // partial slots per (b, hq) = num_parts (balanced:
                            // wg_per_head); 1 = the decode kernel writes out
                            // directly
  // Balanced partitions (INT8 / FP8 / FP16, batch <= kMaxBalancedRows): the
  // rows' blocks of each KV head, concatenated, are cut into wg_per_head
  // equal ranges, one per workgroup; a workgroup writes one partial per row
  // segment of its range (see decode_balanced in kvq_decode.hip).
  int32_t balanced;
  int32_t wg_per_head;
  int32_t ring;             // INT4 ring slots
  int32_t residual;         // INT4 residual length
  int32_t k_head_stride;    // 0 for a per-tensor K scale, 1 per head
  int32_t v_head_stride;
  // Neighbouring KV heads share 128-byte lines of the scale rows (per-token
  // INT8/FP8 rows, affine KIVI rows): the heads of one (row, partition) are
  // then dispatched to one XCD (see wg_coord in kvq_decode.hip).
  int32_t xcd_heads;
  float qk_scale;           // softmax_scale * log2(e)
};

constexpr int kMaxBalancedRows = 256;

// Kernel-side scale kind of a kvq_granularity (0 tensor, 1 head, 2
// channel, 3 token).
constexpr int decode_scale_kind(int granularity) {
  return granularity == 2 ? kChannel : (granularity == 3 ? kToken : kUniform);
}

// Static-scale calibration (kvq_calibrate).  Granularities are kvq_granularity
// values; a null scale array is not calibrated (per-token granularity).
constexpr int kCalibTensor = 0, kCalibHead = 1, kCalibChannel = 2;
constexpr int kMaxCalibHeads = 256;  // KV heads of the per-head reduction in LDS
struct CalibArgs {
  const uint16_t *k;     // fp16 [n_tokens][H][128]
  const uint16_t *v;
  float *k_scales;
  float *v_scales;
  float *partial;        // workspace: [n_chunks][2][H * 128] channel maxima
  int32_t n_tokens;
  int32_t num_kv_heads;
  int32_t chunk_tokens;
  int32_t n_chunks;
  int32_t k_gran;
  int32_t v_gran;
  int32_t accumulate;    // raise existing scales instead of replacing them
  float divisor;         // 127, 448 or 57344
};
hipError_t launch_calibrate(const CalibArgs &a, hipStream_t stream);

hipError_t launch_write_q8(const WriteArgs &a, int dtype, int batch,
                           int max_new, hipStream_t stream);
hipError_t launch_write_f16(const WriteArgs &a, int batch, int max_new, hipStream_t stream);
// dtype: kInt4, kInt4Affine or kInt2Affine (affine groups: unsigned codes,
// zero points beside the scales)
hipError_t launch_write_int4(const WriteArgs &a, int dtype, int batch, int max_new,
                             int max_flush_groups, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int dtype, int k_kind,
                         int v_kind, int batch, hipStream_t stream);

}  // namespace kvq
