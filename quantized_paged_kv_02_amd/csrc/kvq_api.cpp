// Host side of libkvq: argument validation, partition sizing and kernel
// dispatch for the C ABI declared in include/kvq.h.  Everything here runs on
// the host before any launch; the library keeps no state.
#include "kvq.h"

#include <stdint.h>
#include <string.h>

#include <vector>

#include "kvq_args.h"

namespace {

constexpr int kBlock = 16;
constexpr int kHeadDim = 128;
constexpr int kGroup = 64;
// Partition sizing: decode workgroups (four wavefronts) resident at once
// on a 256-CU MI355X (kvq::decode_wg_per_cu per CU, the register budgets
// of the kernels) and the fixed cost of a workgroup (first-load latency,
// LDS merge, partial store) in blocks of streaming.
constexpr long kCUs = 256;
constexpr long kWgOverheadInt4 = 16;
constexpr long kWgOverheadQ8 = 8;
constexpr long kWgOverheadF16 = 4;  // a block streams twice the bytes of INT8
// Rows of at least this many blocks make a launch long enough that HBM
// efficiency, not fixed latency, decides the plan.
constexpr long kStreamMinBlocks = 256;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// KIVI-grouped INT4 cache (symmetric or affine)
bool kivi(const kvq_layout *L) {
  return L->dtype == KVQ_INT4 || L->dtype == KVQ_INT4_AFFINE || L->dtype == KVQ_INT2_AFFINE;
}

int kivi_len(int s, int residual) {
  const int n = s - residual;
  return n > 0 ? (n / kGroup) * kGroup : 0;
}

// Unquantized caches: fp16 or bf16 values, no scales, no residual ring.
bool unquantized(const kvq_layout *L) {
  return L->dtype == KVQ_FP16 || L->dtype == KVQ_BF16;
}

kvq_status check_layout(const kvq_layout *L) {
  if (!L) return KVQ_ERR_INVALID_ARG;
  if (L->struct_size != sizeof(kvq_layout)) return KVQ_ERR_INVALID_ARG;
  if (L->dtype != KVQ_INT8 && L->dtype != KVQ_FP8_E4M3 && L->dtype != KVQ_INT4 &&
      L->dtype != KVQ_FP16 && L->dtype != KVQ_INT4_AFFINE && L->dtype != KVQ_FP8_E5M2 &&
      L->dtype != KVQ_INT2_AFFINE && L->dtype != KVQ_BF16)
    return KVQ_ERR_INVALID_ARG;
  if (!unquantized(L)) {  // an FP16 / BF16 cache has no scales
    if (L->k_gran < KVQ_PER_TENSOR || L->k_gran > KVQ_PER_TOKEN) return KVQ_ERR_INVALID_ARG;
    if (L->v_gran < KVQ_PER_TENSOR || L->v_gran > KVQ_PER_TOKEN) return KVQ_ERR_INVALID_ARG;
  }
  if (L->num_kv_heads < 1 || L->num_q_heads < 1) return KVQ_ERR_INVALID_ARG;
  if (L->num_q_heads % L->num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
  if (L->num_blocks < 1 || L->max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
  if (L->split_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (L->partition != KVQ_PARTITION_PER_ROW && L->partition != KVQ_PARTITION_BALANCED)
    return KVQ_ERR_INVALID_ARG;
  if (L->head_dim != kHeadDim || L->block_size != kBlock) return KVQ_ERR_UNSUPPORTED;
  if (L->num_q_heads / L->num_kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
  if (kivi(L)) {
    if (L->k_gran != KVQ_PER_CHANNEL || L->v_gran != KVQ_PER_TOKEN) return KVQ_ERR_UNSUPPORTED;
    if (L->group_size != kGroup) return KVQ_ERR_UNSUPPORTED;
    if (L->residual_len < kGroup || L->residual_len % kGroup != 0) return KVQ_ERR_UNSUPPORTED;
    if (L->split_tokens % kGroup != 0) return KVQ_ERR_INVALID_ARG;
    if (L->partition == KVQ_PARTITION_BALANCED) return KVQ_ERR_UNSUPPORTED;
  } else if (L->split_tokens % kBlock != 0) {
    return KVQ_ERR_INVALID_ARG;
  }
  return KVQ_OK;
}

// Balanced partitions: workgroups per KV head (one per CU in all).
int balanced_wgs(const kvq_layout *L) {
  const long w = kCUs / L->num_kv_heads;
  return w > 1 ? (int)w : 1;
}

kvq_status check_cache(const kvq_layout *L, const kvq_cache *C, int32_t batch) {
  if (!C) return KVQ_ERR_INVALID_ARG;
  if (!C->k_codes || !C->v_codes) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(C->k_codes) || !aligned16(C->v_codes)) return KVQ_ERR_ALIGNMENT;
  if (unquantized(L)) return KVQ_OK;  // no scales, no ring
  if (!C->k_scales || !C->v_scales) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(C->k_scales) || !aligned16(C->v_scales)) return KVQ_ERR_ALIGNMENT;
  if (kivi(L)) {
    if (!C->k_resid || !C->v_resid) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(C->k_resid) || !aligned16(C->v_resid)) return KVQ_ERR_ALIGNMENT;
    if (C->ring_rows < batch) return KVQ_ERR_CAPACITY;
  }
  return KVQ_OK;
}

// Partition plan for a decode launch.
struct Plan {
  int part_blocks;  // blocks per main partition
  int num_parts;    // main partitions in the grid
  int slots;        // partial slots per (row, query head)
};

// Blocks of a row of length s that the decode streams.
int row_blocks(const kvq_layout *L, int32_t s) {
  return kivi(L) ? kivi_len(s, L->residual_len) / kBlock : (s + kBlock - 1) / kBlock;
}

// Partition length (blocks).  Long rows: the shortest length that keeps
// the launch to one workgroup per CU.  Short rows (the launch is bound by
// fixed latency): the length that minimises (dispatch rounds) x (blocks
// per workgroup + fixed cost), where a launch whose last round is nearly
// empty wastes a whole workgroup time and the longest workgroup sets the
// round's time.  With host_lens the workgroup count is the rows' own
// partitions; without, every row is taken to be max_blocks long.
int choose_part_blocks(const kvq_layout *L, int32_t batch, int max_blocks,
                       const int32_t *host_lens, int32_t n_query = 1) {
  const bool int4 = kivi(L);
  // a workgroup's four waves take units of 2 blocks (INT8/FP8) or one
  // 64-token group (INT4) in turn; partitions give each wave whole units
  const int quantum = int4 ? 16 : 8;
  const long resident =
      kCUs * kvq::decode_wg_per_cu(L->dtype, kvq::decode_scale_kind(L->k_gran),
                                   kvq::decode_scale_kind(L->v_gran));
  const long overhead = int4                       ? kWgOverheadInt4
                        : unquantized(L) ? kWgOverheadF16
                                               : kWgOverheadQ8;
  const long top = max_blocks > quantum ? max_blocks : quantum;
  // workgroups of a launch whose partitions hold c blocks
  auto workgroups = [&](long c) {
    long wgs = 0;
    if (host_lens != nullptr) {
      for (int32_t b = 0; b < batch; ++b) {
        const long nb = row_blocks(L, host_lens[b]);
        long pr = (nb + c - 1) / c;
        if (int4 && host_lens[b] > 0 && pr < 1) pr = 1;  // the fp16 window alone
        wgs += pr;
      }
      return wgs * L->num_kv_heads;
    }
    const long parts = (max_blocks + c - 1) / c;
    return (long)batch * L->num_kv_heads * (parts > 0 ? parts : 1);
  };
  if (L->dtype != KVQ_INT2_AFFINE && top >= kStreamMinBlocks) {
    // Long rows, HBM-bound formats: at most one workgroup per CU (the
    // dispatcher spreads up to one per CU before it doubles any), with the
    // shortest partitions that allow it.  Measured on the shapes of long
    // decode: more resident workgroups per CU contend for HBM and lose
    // 5-9 % (INT4 and FP8, 2-4 workgroups per CU), and a single partition
    // per row also drops the merge launch.  With more (row, head) pairs
    // than CUs, one partition per row.
    // The generic INT4 layout (more than four query heads per KV head, or
    // several queries per row) and the affine INT4 groups (zero-point
    // operands) are bound by their arithmetic instead: two workgroups per CU
    // hide more of it.  KIVI shape, 2 / 4 queries per row: 8192-token
    // partitions 116.9 / 120.8 us per launch, 16384: 125.8 / 128.0 us;
    // affine: 109.5 against 113.0 us (symmetric, compact: 104.8 against
    // 100.0 us, so one per CU there).
    const long per_cu = int4 && (L->dtype == KVQ_INT4_AFFINE ||
                                 L->num_q_heads / L->num_kv_heads > 4 || n_query > 1)
                            ? 2
                            : 1;
    for (long c = quantum; c < top; c += quantum)
      if (workgroups(c) <= per_cu * kCUs) return (int)c;
    return (int)((top + quantum - 1) / quantum * quantum);
  }
  // Workgroups that run as one round.  The 8-bit formats count one per CU:
  // a second or third resident workgroup on a CU adds no throughput there
  // (Llama-2-7B shape, INT8, 128 blocks per row, 128 (row, head) pairs:
  // 1024-token partitions, 256 workgroups, 19.6 us per launch against 20.3
  // us at 512 tokens and 21.3 us at 384, the round model at three per CU's
  // choice).  FP16 streams twice the bytes per block and does gain from a
  // second workgroup (512 tokens: 30.4 us; 1024: 37.3 us), as INT4 is
  // taken to.
  const bool one_per_cu = L->dtype == KVQ_INT8 || L->dtype == KVQ_FP8_E4M3 ||
                          L->dtype == KVQ_FP8_E5M2;
  const long round_wgs = one_per_cu ? kCUs : resident;
  long best_t = -1;
  int pb = quantum;
  for (long c = quantum; c <= top + quantum - 1; c += quantum) {
    const long parts = (max_blocks + c - 1) / c;
    if (parts > 4096) continue;
    const long wgs = workgroups(c);
    const long rounds = (wgs + round_wgs - 1) / round_wgs;
    const long t = (rounds > 0 ? rounds : 1) * (c + overhead);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      pb = (int)c;
    }
  }
  if (host_lens != nullptr) {
    // With real lengths the model can favour thousands of short workgroups
    // whose partials, merges and dispatch it prices too low: keep
    // partitions at least half of a balanced share of the work.
    long work = 0;
    for (int32_t b = 0; b < batch; ++b) work += row_blocks(L, host_lens[b]);
    work *= L->num_kv_heads;
    long floor_c = (work + 2 * round_wgs - 1) / (2 * round_wgs);
    floor_c = (floor_c + quantum - 1) / quantum * quantum;
    if (floor_c > top) floor_c = (top + quantum - 1) / quantum * quantum;
    if (pb < floor_c) pb = (int)floor_c;
  }
  return pb;
}

Plan make_plan(const kvq_layout *L, int32_t batch, int32_t max_seq_len, int32_t n_query = 1) {
  Plan p{};
  if (L->partition == KVQ_PARTITION_BALANCED) {
    // one partial slot per workgroup of a KV head: a row may meet them all
    p.part_blocks = 0;
    p.num_parts = balanced_wgs(L);
    p.slots = p.num_parts;
    return p;
  }
  const bool int4 = kivi(L);
  const int blocks = row_blocks(L, max_seq_len);
  int pb = L->split_tokens > 0 ? L->split_tokens / kBlock
                               : choose_part_blocks(L, batch, blocks, nullptr, n_query);
  if (pb < (int4 ? 4 : 1)) pb = int4 ? 4 : 1;
  p.part_blocks = pb;
  p.num_parts = blocks > 0 ? (blocks + pb - 1) / pb : 1;  // >= 1: empty rows, INT4 rings
  p.slots = p.num_parts;
  return p;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WorkspaceLayout {
  size_t m_off, l_off, o_off, total;
};

// Partials of every (row, query token, query head, partition slot); none
// when the plan has a single slot (the decode kernel then writes the output
// directly).
WorkspaceLayout workspace_layout(const kvq_layout *L, int32_t batch, const Plan &p,
                                 int32_t n_query = 1) {
  WorkspaceLayout w{};
  if (p.slots <= 1 && L->partition != KVQ_PARTITION_BALANCED) return w;
  const size_t rows = (size_t)batch * n_query * L->num_q_heads * p.slots;
  w.m_off = 0;
  w.l_off = w.m_off + round_up(rows * sizeof(float), 256);
  w.o_off = w.l_off + round_up(rows * sizeof(float), 256);
  w.total = w.o_off + round_up(rows * kHeadDim * sizeof(float), 256);
  return w;
}

}  // namespace

extern "C" {

const char *kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG: invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: configuration not supported";
    case KVQ_ERR_ALIGNMENT: return "KVQ_ERR_ALIGNMENT: device pointer not 16-byte aligned";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE: workspace too small or misaligned";
    case KVQ_ERR_CAPACITY: return "KVQ_ERR_CAPACITY: length exceeds the block table";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP: kernel launch failed";
  }
  return "KVQ_ERR_UNKNOWN";
}

kvq_status kvq_validate(const kvq_layout *layout, const kvq_cache *cache, int32_t batch,
                        int32_t max_seq_len) {
  kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (batch < 0 || max_seq_len < 0) return KVQ_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)layout->max_blocks_per_seq * kBlock) return KVQ_ERR_CAPACITY;
  if (layout->partition == KVQ_PARTITION_BALANCED && batch > kvq::kMaxBalancedRows)
    return KVQ_ERR_UNSUPPORTED;
  return check_cache(layout, cache, batch);
}

size_t kvq_decode_workspace_bytes(const kvq_layout *layout, int32_t batch,
                                  int32_t max_seq_len) {
  if (check_layout(layout) != KVQ_OK || batch < 0 || max_seq_len < 0) return 0;
  const Plan p = make_plan(layout, batch, max_seq_len);
  return workspace_layout(layout, batch, p).total;
}

kvq_status kvq_write(const kvq_layout *layout, const kvq_cache *cache, const uint16_t *k_new,
                     const uint16_t *v_new, const int32_t *cu_new,
                     const int32_t *block_tables, const int32_t *seq_lens, int32_t batch,
                     int32_t total_new, int32_t max_new_per_seq, void *stream) {
  kvq_status st = kvq_validate(layout, cache, batch, 0);
  if (st != KVQ_OK) return st;
  if (total_new < 0 || max_new_per_seq < 0) return KVQ_ERR_INVALID_ARG;
  if ((int64_t)max_new_per_seq > (int64_t)layout->max_blocks_per_seq * kBlock)
    return KVQ_ERR_CAPACITY;
  if (batch == 0 || total_new == 0 || max_new_per_seq == 0) return KVQ_OK;
  if (!k_new || !v_new || !cu_new || !block_tables || !seq_lens) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(cu_new) ||
      !aligned16(block_tables) || !aligned16(seq_lens))
    return KVQ_ERR_ALIGNMENT;

  kvq::WriteArgs a{};
  a.k_codes = static_cast<uint8_t *>(cache->k_codes);
  a.v_codes = static_cast<uint8_t *>(cache->v_codes);
  a.k_scales = cache->k_scales;
  a.v_scales = cache->v_scales;
  a.k_resid = cache->k_resid;
  a.v_resid = cache->v_resid;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cu_new = cu_new;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.num_kv_heads = layout->num_kv_heads;
  a.max_blocks_per_seq = layout->max_blocks_per_seq;
  a.k_gran = layout->k_gran;
  a.v_gran = layout->v_gran;
  a.residual = layout->residual_len;
  a.ring = layout->residual_len + kGroup;

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e;
  if (kivi(layout)) {
    // groups leaving the window when a row grows by n tokens to length S:
    // nq(S) - nq(S - n) = 64 (floor((S - 128) / 64) - floor((S - n - 128) /
    // 64)) <= 64 ceil(n / 64) (less while S - n < 128), so ceil(n / 64)
    const int max_groups = (max_new_per_seq + kGroup - 1) / kGroup;
    e = kvq::launch_write_int4(a, layout->dtype, batch, max_new_per_seq, max_groups, s);
  } else if (unquantized(layout)) {
    e = kvq::launch_write_f16(a, batch, max_new_per_seq, s);  // bits copied as they are
  } else {
    e = kvq::launch_write_q8(a, layout->dtype, batch, max_new_per_seq, s);
  }
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

// Host checks and kernel arguments of a decode launch; KVQ_OK with
// *launch == false when there is nothing to do (batch == 0).
static kvq_status decode_setup(const kvq_layout *layout, const kvq_cache *cache,
                               const uint16_t *q, const int32_t *block_tables,
                               const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                               float softmax_scale, float *out, void *workspace,
                               size_t workspace_bytes, kvq::DecodeArgs *a, bool *launch,
                               int32_t n_query = 1) {
  *launch = false;
  kvq_status st = kvq_validate(layout, cache, batch, max_seq_len);
  if (st != KVQ_OK) return st;
  if (batch == 0) return KVQ_OK;
  if (!q || !block_tables || !seq_lens || !out) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(block_tables) || !aligned16(seq_lens) || !aligned16(out))
    return KVQ_ERR_ALIGNMENT;
  if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
    return KVQ_ERR_INVALID_ARG;
  const Plan p = make_plan(layout, batch, max_seq_len, n_query);
  // one 256-thread workgroup per (partition, KV head, row) in a 1-D grid,
  // (row, partition) pairs padded to a multiple of 8: its work-item count
  // must fit in 32 bits
  // (a KIVI decode step adds 2 x batch x H flush workgroups)
  const int64_t pairs8 = ((int64_t)p.num_parts * batch + 7) / 8 * 8 + 2 * (int64_t)batch;
  if (pairs8 * layout->num_kv_heads * 256 >= ((int64_t)1 << 32)) return KVQ_ERR_UNSUPPORTED;
  const WorkspaceLayout w = workspace_layout(layout, batch, p, n_query);
  if (w.total > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
                      workspace_bytes < w.total))
    return KVQ_ERR_WORKSPACE;

  char *ws = static_cast<char *>(workspace);
  *a = kvq::DecodeArgs{};
  a->k_codes = static_cast<const uint8_t *>(cache->k_codes);
  a->v_codes = static_cast<const uint8_t *>(cache->v_codes);
  a->k_scales = cache->k_scales;
  a->v_scales = cache->v_scales;
  a->k_resid = cache->k_resid;
  a->v_resid = cache->v_resid;
  a->q = q;
  a->block_tables = block_tables;
  a->seq_lens = seq_lens;
  a->out = out;
  a->ws_m = reinterpret_cast<float *>(ws + w.m_off);
  a->ws_l = reinterpret_cast<float *>(ws + w.l_off);
  a->ws_o = reinterpret_cast<float *>(ws + w.o_off);
  a->batch = batch;
  a->num_q_heads = layout->num_q_heads;
  a->num_kv_heads = layout->num_kv_heads;
  a->group = layout->num_q_heads / layout->num_kv_heads;
  a->n_query = n_query;
  a->cols = n_query * a->group;
  a->max_blocks_per_seq = layout->max_blocks_per_seq;
  a->max_seq_len = max_seq_len;
  a->part_blocks = p.part_blocks;
  a->num_parts = p.num_parts;
  a->slots = p.slots;
  a->residual = layout->residual_len;
  a->ring = layout->residual_len + kGroup;
  a->k_head_stride = layout->k_gran == KVQ_PER_HEAD ? 1 : 0;
  a->v_head_stride = layout->v_gran == KVQ_PER_HEAD ? 1 : 0;
  // scale rows narrower or wider than a 128-byte line: per-token rows of
  // the 8-bit formats (64 bytes), affine KIVI rows (160 bytes).  Measured
  // on MI355X: Llama-2-7B INT8/token step 0.588 -> 0.577 ms, affine INT4
  // launch 134.2 -> 132.5 us with the heads of a (row, partition) on one
  // XCD; the symmetric INT4 step (128-byte rows) is 1.4 % slower that way.
  const bool q8 = layout->dtype == KVQ_INT8 || layout->dtype == KVQ_FP8_E4M3 ||
                  layout->dtype == KVQ_FP8_E5M2;
  a->xcd_heads = (q8 && (layout->k_gran == KVQ_PER_TOKEN || layout->v_gran == KVQ_PER_TOKEN)) ||
                 layout->dtype == KVQ_INT4_AFFINE || layout->dtype == KVQ_INT2_AFFINE;
  a->balanced = layout->partition == KVQ_PARTITION_BALANCED ? 1 : 0;
  a->wg_per_head = a->balanced ? p.num_parts : 0;
  a->qk_scale = softmax_scale * 1.4426950408889634f;
  *launch = true;
  return KVQ_OK;
}

static kvq_status decode_launch(const kvq_layout *layout, const kvq::DecodeArgs &a,
                                int32_t batch, void *stream) {
  (void)hipGetLastError();
  const hipError_t e = kvq::launch_decode(a, layout->dtype, kvq::decode_scale_kind(layout->k_gran),
                                          kvq::decode_scale_kind(layout->v_gran), batch,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_paged_decode(const kvq_layout *layout, const kvq_cache *cache,
                            const uint16_t *q, const int32_t *block_tables,
                            const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                            float softmax_scale, float *out, void *workspace,
                            size_t workspace_bytes, void *stream) {
  kvq::DecodeArgs a;
  bool launch;
  const kvq_status st = decode_setup(layout, cache, q, block_tables, seq_lens, batch, max_seq_len,
                                     softmax_scale, out, workspace, workspace_bytes, &a, &launch);
  if (st != KVQ_OK || !launch) return st;
  return decode_launch(layout, a, batch, stream);
}

kvq_status kvq_write_decode(const kvq_layout *layout, const kvq_cache *cache,
                            const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                            const int32_t *block_tables, const int32_t *seq_lens, int32_t batch,
                            int32_t max_seq_len, float softmax_scale, float *out,
                            void *workspace, size_t workspace_bytes, void *stream) {
  kvq::DecodeArgs a;
  bool launch;
  const kvq_status st = decode_setup(layout, cache, q, block_tables, seq_lens, batch, max_seq_len,
                                     softmax_scale, out, workspace, workspace_bytes, &a, &launch);
  if (st != KVQ_OK || !launch) return st;
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGNMENT;
  // The workgroup that streams a row's last partition stores the new token
  // first (INT8 / FP8 / FP16: its codes and scales in the last block; KIVI:
  // the fp16 ring); a KIVI step also flushes the group that leaves the
  // window at the next length, in workgroups of the same launch.
  a.k_new = k_new;
  a.v_new = v_new;
  return decode_launch(layout, a, batch, stream);
}

// ---- partition planning from host-known lengths ---------------------------------

int32_t kvq_plan_split_tokens(const kvq_layout *layout, const int32_t *host_seq_lens,
                              int32_t batch) {
  const kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (batch < 0 || (batch > 0 && host_seq_lens == nullptr)) return KVQ_ERR_INVALID_ARG;
  int32_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (host_seq_lens[b] < 0) return KVQ_ERR_INVALID_ARG;
    if (host_seq_lens[b] > max_len) max_len = host_seq_lens[b];
  }
  if ((int64_t)max_len > (int64_t)layout->max_blocks_per_seq * kBlock) return KVQ_ERR_CAPACITY;
  const int pb = choose_part_blocks(layout, batch, row_blocks(layout, max_len), host_seq_lens);
  return pb * kBlock;
}

// ---- choice between per-row and balanced partitions ---------------------------------

int32_t kvq_plan_partition(const kvq_layout *layout, const int32_t *host_seq_lens,
                           int32_t batch) {
  kvq_layout L = *layout;
  L.partition = KVQ_PARTITION_PER_ROW;
  const kvq_status st = check_layout(&L);
  if (st != KVQ_OK) return st;
  if (batch < 0 || (batch > 0 && host_seq_lens == nullptr)) return KVQ_ERR_INVALID_ARG;
  int32_t max_len = 0;
  long total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (host_seq_lens[b] < 0) return KVQ_ERR_INVALID_ARG;
    if (host_seq_lens[b] > max_len) max_len = host_seq_lens[b];
    total += row_blocks(&L, host_seq_lens[b]);
  }
  if ((int64_t)max_len > (int64_t)L.max_blocks_per_seq * kBlock) return KVQ_ERR_CAPACITY;
  if (kivi(&L) || batch == 0 || batch > kvq::kMaxBalancedRows || total == 0)
    return KVQ_PARTITION_PER_ROW;
  // Per-row partitions as kvq_plan_split_tokens would cut them: the launch
  // lasts about as long as its longest workgroup when the workgroups fit in
  // one round (one per CU), plus the merge when a row is split.
  const int pb = L.split_tokens > 0
                     ? L.split_tokens / kBlock
                     : choose_part_blocks(&L, batch, row_blocks(&L, max_len), host_seq_lens);
  long wgs = 0, longest = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const long nb = row_blocks(&L, host_seq_lens[b]);
    wgs += (nb + pb - 1) / pb;
    longest = nb < pb ? (nb > longest ? nb : longest) : (pb > longest ? pb : longest);
  }
  const long per_head = wgs;
  wgs *= L.num_kv_heads;
  if (wgs > kCUs) return KVQ_PARTITION_PER_ROW;  // several rounds: the rows' own split
  // The per-row launch is HBM-bound while its workgroups stream alike;
  // unequal rows leave its longest workgroup streaming alone at the end.
  // Balanced ranges pay the merge launch and a second segment per
  // workgroup: worth it only when the longest workgroup is well above the
  // mean (measured: Llama-3-8B GQA shape, rows U[1024, 16384], longest 1.9x
  // the mean: 110.6 against 115.6 us per launch; Llama-3-70B shape, equal
  // rows: FP8 135 against 127 us, so per row there).
  const long mean = (total + per_head - 1) / per_head;
  return 4 * longest > 5 * mean ? KVQ_PARTITION_BALANCED : KVQ_PARTITION_PER_ROW;
}

// ---- host-side check of block tables and lengths ------------------------------

kvq_status kvq_check_tables(const kvq_layout *layout, const int32_t *host_block_tables,
                            const int32_t *host_seq_lens, int32_t batch, int32_t max_seq_len,
                            int32_t *bad_row) {
  if (bad_row) *bad_row = -1;
  const kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (batch < 0 || max_seq_len < 0) return KVQ_ERR_INVALID_ARG;
  if (batch == 0) return KVQ_OK;
  if (!host_block_tables || !host_seq_lens) return KVQ_ERR_INVALID_ARG;
  const int64_t mbs = layout->max_blocks_per_seq;
  if ((int64_t)max_seq_len > mbs * kBlock) return KVQ_ERR_CAPACITY;
  // one bit per physical block: a block that two table entries name would
  // be written by both
  std::vector<uint8_t> used((size_t)layout->num_blocks, 0);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t s = host_seq_lens[b];
    if (s < 0) {
      if (bad_row) *bad_row = b;
      return KVQ_ERR_INVALID_ARG;
    }
    if (s > max_seq_len) {
      if (bad_row) *bad_row = b;
      return KVQ_ERR_CAPACITY;
    }
    // entries the kernels touch: every block of the row (INT8 / FP8 / FP16);
    // the INT4 blocks of a KIVI row, through the group the next token flushes
    const int64_t need = kivi(layout) ? kivi_len(s + 1, layout->residual_len) / kBlock
                                      : ((int64_t)s + kBlock - 1) / kBlock;
    for (int64_t j = 0; j < need; ++j) {
      const int32_t id = host_block_tables[(int64_t)b * mbs + j];
      if (id < 0 || id >= layout->num_blocks || used[(size_t)id]) {
        if (bad_row) *bad_row = b;
        return KVQ_ERR_INVALID_ARG;
      }
      used[(size_t)id] = 1;
    }
  }
  return KVQ_OK;
}

// ---- several query tokens per row ----------------------------------------------

static kvq_status check_mq(const kvq_layout *layout, int32_t n_query) {
  const kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (n_query < 1) return KVQ_ERR_INVALID_ARG;
  if ((int64_t)n_query * (layout->num_q_heads / layout->num_kv_heads) > 16)
    return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

size_t kvq_paged_decode_mq_workspace_bytes(const kvq_layout *layout, int32_t n_query,
                                           int32_t batch, int32_t max_seq_len) {
  if (check_mq(layout, n_query) != KVQ_OK || batch < 0 || max_seq_len < 0) return 0;
  const Plan p = make_plan(layout, batch, max_seq_len, n_query);
  return workspace_layout(layout, batch, p, n_query).total;
}

kvq_status kvq_paged_decode_mq(const kvq_layout *layout, const kvq_cache *cache,
                               const uint16_t *q, int32_t n_query, const int32_t *block_tables,
                               const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                               float softmax_scale, float *out, void *workspace,
                               size_t workspace_bytes, void *stream) {
  const kvq_status st0 = check_mq(layout, n_query);
  if (st0 != KVQ_OK) return st0;
  kvq::DecodeArgs a;
  bool launch;
  const kvq_status st = decode_setup(layout, cache, q, block_tables, seq_lens, batch,
                                     max_seq_len, softmax_scale, out, workspace,
                                     workspace_bytes, &a, &launch, n_query);
  if (st != KVQ_OK || !launch) return st;
  return decode_launch(layout, a, batch, stream);
}

// ---- static-scale calibration ------------------------------------------------

static int calib_chunks(int32_t n_tokens) {
  const int c = (n_tokens + 63) / 64;
  return c < 1 ? 1 : (c > 256 ? 256 : c);
}

static bool calib_dtype(const kvq_layout *L) {
  return L->dtype == KVQ_INT8 || L->dtype == KVQ_FP8_E4M3 || L->dtype == KVQ_FP8_E5M2;
}

size_t kvq_calibrate_workspace_bytes(const kvq_layout *layout, int32_t n_tokens) {
  if (check_layout(layout) != KVQ_OK || !calib_dtype(layout) || n_tokens <= 0) return 0;
  const size_t b = (size_t)calib_chunks(n_tokens) * 2 * layout->num_kv_heads * kHeadDim * 4;
  return round_up(b, 256);
}

kvq_status kvq_calibrate(const kvq_layout *layout, const uint16_t *k, const uint16_t *v,
                         int32_t n_tokens, float *k_scales, float *v_scales, int32_t accumulate,
                         void *workspace, size_t workspace_bytes, void *stream) {
  kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (!calib_dtype(layout)) return KVQ_ERR_UNSUPPORTED;  // no static scales
  if (layout->num_kv_heads > kvq::kMaxCalibHeads) return KVQ_ERR_UNSUPPORTED;
  if (n_tokens < 0) return KVQ_ERR_INVALID_ARG;
  const bool do_k = layout->k_gran != KVQ_PER_TOKEN, do_v = layout->v_gran != KVQ_PER_TOKEN;
  if (n_tokens == 0 || (!do_k && !do_v)) return KVQ_OK;
  if ((do_k && (!k || !k_scales)) || (do_v && (!v || !v_scales))) return KVQ_ERR_INVALID_ARG;
  if ((do_k && (!aligned16(k) || !aligned16(k_scales))) ||
      (do_v && (!aligned16(v) || !aligned16(v_scales))))
    return KVQ_ERR_ALIGNMENT;
  const size_t need = kvq_calibrate_workspace_bytes(layout, n_tokens);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      workspace_bytes < need)
    return KVQ_ERR_WORKSPACE;
  kvq::CalibArgs a{};
  a.k = do_k ? k : nullptr;
  a.v = do_v ? v : nullptr;
  a.k_scales = do_k ? k_scales : nullptr;
  a.v_scales = do_v ? v_scales : nullptr;
  a.partial = static_cast<float *>(workspace);
  a.n_tokens = n_tokens;
  a.num_kv_heads = layout->num_kv_heads;
  a.n_chunks = calib_chunks(n_tokens);
  a.chunk_tokens = (n_tokens + a.n_chunks - 1) / a.n_chunks;
  a.k_gran = layout->k_gran;
  a.v_gran = layout->v_gran;
  a.accumulate = accumulate ? 1 : 0;
  a.divisor = layout->dtype == KVQ_INT8 ? 127.0f
              : layout->dtype == KVQ_FP8_E4M3 ? 448.0f
                                              : 57344.0f;
  (void)hipGetLastError();
  const hipError_t e = kvq::launch_calibrate(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"
