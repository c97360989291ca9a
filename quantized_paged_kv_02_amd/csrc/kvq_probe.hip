// HBM bandwidth probes (measurement tooling, built as their own library
// libkvq_probe.so; not part of the libkvq ABI): read-only (the decode) and
// read-and-write at 2 : 1 (the bulk write).
//
// The read probe issues the decode kernel's access pattern without its
// arithmetic: every
// wavefront load is one 16-byte buffer load per lane, i.e. one 1 KiB chunk
// (an INT4 (block, head) code chunk, half an INT8 one), with the same
// non-temporal cache policy, eight chunks in flight per wavefront.  Chunk
// order: 0 = wavefront w takes chunks w, w + W, w + 2W, ... (W wavefronts in
// the grid), 1 = the same indices sent through a bijection of the chunk
// range (multiplication by an odd constant modulo a power of two), so
// consecutive loads of a wavefront land far apart, as paged blocks do.  The
// bytes a launch reads over its duration is the HBM read rate the chip
// reaches with this pattern: the "achievable" denominator beside the
// vendor's 8 TB/s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"

namespace {

constexpr int kInFlight = 8;

__global__ __launch_bounds__(1024) void kvq_probe_read_kernel(const uint8_t *src,
                                                             uint32_t chunk_mask,
                                                             int random_order,
                                                             uint32_t *sink) {
  using namespace kvq;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const uint32_t waves = (gridDim.x * blockDim.x) >> 6;
  const uint32_t n_chunks = chunk_mask + 1;
  uint32_t acc = 0;
  for (uint32_t c0 = wave; c0 < n_chunks; c0 += kInFlight * waves) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const uint32_t c = c0 + u * waves;
      const uint32_t idx = random_order ? (c * 0x9E3779B1u) & chunk_mask : c;
      // a chunk past the range reads through an empty resource: zeros
      const rsrc_t r = make_rsrc(src + (size_t)idx * 1024, c < n_chunks ? 1024u : 0u);
      v[u] = bld16(r, 16 * lane);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // keeps every load live; the buffer is filled so that this never holds
  if (acc == 0xFFFFFFFFu) sink[blockIdx.x] = acc;
}

// Read-and-write stream with the bulk write's 2 : 1 ratio (fp16 in, one
// byte per value out): wavefront w takes 1 KiB source chunks w, w + W, ...,
// one 16-byte load per lane (kInFlight chunks in flight), and stores 8 bytes
// per lane (the high byte of each fp16) to the chunk's 512-byte slot of
// `dst`: whole 512-byte runs of full lines, as the cache code chunks are
// written.
__global__ __launch_bounds__(1024) void kvq_probe_rw_kernel(const uint8_t *src, uint8_t *dst,
                                                           uint32_t n_chunks) {
  using namespace kvq;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const uint32_t waves = (gridDim.x * blockDim.x) >> 6;
  for (uint32_t c0 = wave; c0 < n_chunks; c0 += kInFlight * waves) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const uint32_t c = c0 + u * waves;
      const rsrc_t r = make_rsrc(src + (size_t)c * 1024, c < n_chunks ? 1024u : 0u);
      v[u] = bld16(r, 16 * lane);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const uint32_t c = c0 + u * waves;
      if (c < n_chunks) {
        const uint32_t lo = __builtin_amdgcn_perm(v[u][1], v[u][0], 0x07050301u);
        const uint32_t hi = __builtin_amdgcn_perm(v[u][3], v[u][2], 0x07050301u);
        *reinterpret_cast<uint2 *>(dst + (size_t)c * 512 + 8 * lane) = uint2{lo, hi};
      }
    }
  }
}

}  // namespace

// Read `bytes` (a power of two, at least 1 MiB, 1 KiB aligned) at the device
// pointer `src` once with `workgroups` workgroups of `threads` threads (64,
// 128, ..., 1024) on `stream`; `sink` is a device uint32 array of
// `workgroups` entries that the kernel may write.  Returns 0 on success, -1
// for bad arguments, -6 if the launch failed.
extern "C" int kvq_probe_read(const void *src, size_t bytes, int workgroups, int threads,
                              int random_order, uint32_t *sink, void *stream) {
  if (!src || !sink || workgroups < 1 || bytes < (1u << 20) || (bytes & (bytes - 1)) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 1023u) != 0 || bytes / 1024 > (1ull << 30) ||
      threads < 64 || threads > 1024 || threads % 64 != 0)
    return -1;
  const uint32_t mask = (uint32_t)(bytes / 1024 - 1);
  (void)hipGetLastError();
  hipLaunchKernelGGL(kvq_probe_read_kernel, dim3(workgroups), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(src), mask,
                     random_order, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Read `bytes` at `src` (a power of two, at least 1 MiB, 1 KiB aligned) and
// write bytes / 2 at `dst` (512-byte aligned) once, with `workgroups`
// workgroups of `threads` threads on `stream`.  Returns 0 on success, -1 for
// bad arguments, -6 if the launch failed.
extern "C" int kvq_probe_rw(const void *src, size_t bytes, void *dst, int workgroups,
                            int threads, void *stream) {
  if (!src || !dst || workgroups < 1 || bytes < (1u << 20) || (bytes & (bytes - 1)) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 1023u) != 0 ||
      (reinterpret_cast<uintptr_t>(dst) & 511u) != 0 || bytes / 1024 > (1ull << 30) ||
      threads < 64 || threads > 1024 || threads % 64 != 0)
    return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(kvq_probe_rw_kernel, dim3(workgroups), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(src),
                     static_cast<uint8_t *>(dst), (uint32_t)(bytes / 1024));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
