// kvq_write_decode_noalloc: the decode step of kvq_write_decode with its
// split-K partials in a library-owned device array instead of a caller
// workspace, for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host
// code never uses the variable's name as an address (on the host it only
// names the symbol); the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and is what the kernels
// receive, exactly as they receive a caller's workspace.
#include <mutex>

#include "kvq.h"
#include "kvq_args.h"

namespace {

constexpr size_t kScratchBytes = (size_t)KVQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device; null if the lookup fails.
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" kvq_status kvq_write_decode_noalloc(const kvq_layout *layout,
                                               const kvq_cache *cache,
                                               const uint16_t *k_new, const uint16_t *v_new,
                                               const uint16_t *q, const int32_t *block_tables,
                                               const int32_t *seq_lens, int32_t batch,
                                               int32_t max_seq_len, float softmax_scale,
                                               float *out, void *stream) {
  // every argument check of kvq_write_decode, before the size check and
  // before any HIP call
  const kvq_status st = kvq_validate(layout, cache, batch, max_seq_len);
  if (st != KVQ_OK) return st;
  if (batch == 0) return KVQ_OK;
  if (kvq_decode_workspace_bytes(layout, batch, max_seq_len) > kScratchBytes)
    return KVQ_ERR_WORKSPACE;
  void *ws = device_scratch();
  if (ws == nullptr) return KVQ_ERR_HIP;
  return kvq_write_decode(layout, cache, k_new, v_new, q, block_tables, seq_lens, batch,
                          max_seq_len, softmax_scale, out, ws, kScratchBytes, stream);
}
