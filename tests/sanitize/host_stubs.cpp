// Host-only stand-ins for the kernel launchers of libkvq, for a build of the
// host API (kvq_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer
// on a machine without a GPU.  Test infrastructure: the product library never
// links this file.
//
// Each launcher checks, on the host, what its kernels assume of the argument
// block the API built (pointers present, sizes positive, partition plan
// consistent, grids within the 32-bit work-item limit) and reports a
// violation by aborting; it launches nothing and returns success.
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "kvq_args.h"

namespace {

void require(bool ok, const char *what) {
  if (!ok) {
    fprintf(stderr, "host stub: %s\n", what);
    abort();
  }
}

}  // namespace

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace kvq {

hipError_t launch_decode(const DecodeArgs &a, int dtype, int k_kind, int v_kind, int batch,
                         hipStream_t stream) {
  (void)stream;
  require(dtype >= kInt8 && dtype <= kInt2Affine, "decode: dtype");
  require(k_kind >= kUniform && k_kind <= kToken && v_kind >= kUniform && v_kind <= kToken,
          "decode: scale kinds");
  require(a.k_codes && a.v_codes && a.q && a.block_tables && a.seq_lens && a.out,
          "decode: pointers");
  require(a.batch == batch && batch > 0, "decode: batch");
  require(a.group >= 1 && a.group <= 16 && a.cols == a.n_query * a.group && a.cols <= 16,
          "decode: query columns");
  require(a.num_q_heads == a.group * a.num_kv_heads, "decode: heads");
  require(a.slots >= 1 && a.num_parts >= 1, "decode: partition plan");
  if (a.balanced) {
    require(!is_kivi(dtype) && batch <= kMaxBalancedRows, "decode: balanced rows");
    require(a.wg_per_head == a.num_parts && a.slots == a.num_parts, "decode: balanced slots");
  } else {
    require(a.part_blocks >= 1 && a.slots == a.num_parts, "decode: per-row slots");
    require((long)a.num_parts * a.part_blocks * 16 >= a.max_seq_len - (is_kivi(dtype) ? a.residual : 0),
            "decode: partitions cover max_seq_len");
  }
  if (a.slots > 1 || a.balanced)
    require(a.ws_m && a.ws_l && a.ws_o, "decode: workspace");
  require((long)a.num_parts * batch * a.num_kv_heads * 256 < (1L << 32), "decode: grid");
  require(a.max_seq_len <= a.max_blocks_per_seq * 16, "decode: max_seq_len");
  return hipSuccess;
}

hipError_t launch_write_q8(const WriteArgs &a, int dtype, int batch, int max_new,
                           hipStream_t stream) {
  (void)stream;
  require(dtype == kInt8 || dtype == kFp8 || dtype == kFp8E5M2, "write q8: dtype");
  require(a.k_codes && a.v_codes && a.k_new && a.v_new && a.cu_new && a.block_tables &&
              a.seq_lens && a.k_scales && a.v_scales,
          "write q8: pointers");
  require(batch > 0 && max_new > 0 && max_new <= a.max_blocks_per_seq * 16, "write q8: sizes");
  return hipSuccess;
}

hipError_t launch_write_f16(const WriteArgs &a, int batch, int max_new, hipStream_t stream) {
  (void)stream;
  require(a.k_codes && a.v_codes && a.k_new && a.v_new && a.block_tables && a.seq_lens,
          "write f16: pointers");
  require(batch > 0 && max_new > 0, "write f16: sizes");
  return hipSuccess;
}

hipError_t launch_write_int4(const WriteArgs &a, int dtype, int batch, int max_new,
                             int max_flush_groups, hipStream_t stream) {
  (void)stream;
  require(is_kivi(dtype), "write int4: dtype");
  require(a.k_resid && a.v_resid && a.ring == a.residual + 64, "write int4: ring");
  require(batch > 0 && max_new > 0 && max_flush_groups == (max_new + 63) / 64,
          "write int4: flush groups");
  return hipSuccess;
}

hipError_t launch_calibrate(const CalibArgs &a, hipStream_t stream) {
  (void)stream;
  require(a.partial && a.n_tokens > 0 && a.n_chunks >= 1 && a.n_chunks <= 256,
          "calibrate: sizes");
  require((long)a.chunk_tokens * a.n_chunks >= a.n_tokens, "calibrate: chunks cover tokens");
  require(a.k || a.v, "calibrate: a tensor");
  return hipSuccess;
}

}  // namespace kvq

// Marks a host-only stub build: the driver of valid calls refuses to run
// against a library without it (valid calls on the real library launch
// kernels on its fake pointers).
extern "C" int kvq_host_stub_build(void) { return 1; }
