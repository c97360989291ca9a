/*
 * kvq.h -- C ABI of libkvq: quantize-on-write and split-K paged decode
 * attention over an INT8, FP8 (OCP E4M3) or INT4 KV cache, for AMD MI355X
 * (gfx950).
 *
 * Method (from three web pages on KV-cache quantization):
 *   [yunthe]  "KV Cache量化压缩技术与vLLM推理引擎显存优化实战"
 *   [oh-bug]  "KV Cache Quantization 生产实战：用低精度缓存降低长上下文推理显存"
 *   [intelli] "大模型KV Cache显存优化与量化技术实践"
 *
 *  - Symmetric quantization: scale = max|x| / 127, q = clamp(round(x/scale),
 *    -128, 127)  ([intelli] §3.1 对称量化算法; [yunthe] section
 *    "KV Cache量化策略：INT8与FP8精度对比与选择").  Division is one IEEE fp32
 *    division, rounding is half-to-even.  FP8 uses scale = max|x| / 448 and
 *    round-to-nearest-even into E4M3 after clamping to +-448; E5M2 (the
 *    pages' other FP8 format) likewise with 57344 (its largest finite
 *    value).
 *  - Granularity of the scale: tensor, head, channel or token ([oh-bug]
 *    section "量化不是简单'截断精度'"); dynamic per-token scales are computed
 *    on write ([intelli] §3.2 动态量化策略), static ones are inputs.
 *  - Paged cache of 16-token blocks, dequantized inside the attention kernel
 *    ([yunthe] section "PagedAttention与KV Cache量化协同工作原理").
 *  - INT4 KIVI-style cache: K per channel, V per token, group 64, two codes
 *    per byte, the newest tokens kept in fp16 (residual 128) ([oh-bug]
 *    sections "Key 和 Value 的分布不一定相同" and "Transformers：适合实验和
 *    小规模验证").
 *  - Decode attention softmax(q K^T * softmax_scale) V over every cached token
 *    ([intelli] §6 Q1; [oh-bug] section "为什么长上下文更需要 KV Cache
 *    Quantization").
 *
 *  - An unquantized FP16 or BF16 cache through the same kernels, the
 *    baseline of the memory / latency comparison ([intelli] §5).
 *  - An asymmetric INT4 KIVI cache (the affine form with integer zero
 *    points of [oh-bug] section "量化不是简单'截断精度'") and static-scale
 *    calibration from calibration tokens ([yunthe] section "配置与启动参数").
 *
 * Conventions for every entry point:
 *  - All buffers are caller-owned DEVICE pointers except the kvq_layout and
 *    kvq_cache structs themselves, which are host memory read during the call
 *    only.  The library allocates, frees and synchronises nothing; it keeps no
 *    state between calls (except the per-GPU partials array of
 *    kvq_write_decode_noalloc) and may be called from several host threads.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Kernels run
 *    asynchronously on it, in call order.
 *  - Arguments are validated on the host before any launch; on error a
 *    negative kvq_status is returned and nothing is enqueued.  A failed launch
 *    returns KVQ_ERR_HIP (the HIP error state is cleared before launching).
 *  - Device pointers must be 16-byte aligned; fp16 data is IEEE binary16
 *    passed as uint16_t; fp32 is IEEE binary32.
 *  - Pool arrays may be of any size the device holds (byte offsets are
 *    formed in 64 bits; a layer's code arrays may pass 4 GiB); block ids
 *    and num_blocks are int32.
 *  - Host integers (batch, total_new, max_new_per_seq, max_seq_len) size the
 *    grids, because seq_lens lives on the device; they must bound the device
 *    values: seq_lens[b] <= max_seq_len for every row b of a decode
 *    (kvq_paged_decode, kvq_write_decode, kvq_paged_decode_mq), new tokens
 *    per sequence <= max_new_per_seq for kvq_write.  A decode row longer
 *    than max_seq_len gets NaN outputs (and, in kvq_write_decode, its token
 *    is not appended and, for KIVI caches, no group of it is flushed); a
 *    kvq_write row with more new tokens than max_new_per_seq is undefined.  Block ids in the
 *    tables must lie in [0, num_blocks): an id outside is an out-of-bounds
 *    access.  kvq_check_tables checks host copies of both.
 *  - Non-finite K/V inputs give unspecified codes.
 *  - Numerics of the decode: fp16 (bf16 for a BF16 cache) matrix operands
 *    with fp32 accumulation and an fp32 softmax.  Every finite V is safe:
 *    the running maximum lags a score by at most log2(65504 / s) for the
 *    largest per-token V scale s the format can hold, so weights times V
 *    scales stay finite in fp16.  Per-channel K scales (KIVI groups, static
 *    per-channel INT8/FP8) are folded into the query: |q_c| * s_c must stay
 *    below 65504 (e.g. K values within +-1000 and |q_c| < 450 for
 *    symmetric INT4, |q_c| < 98 for 2-bit affine groups).  The softmax
 *    weights (times per-token V scales) enter the value product as a pair
 *    of fp16 terms, hi and the rounded remainder (~22 significant bits), for
 *    the FP16 cache and the INT8/FP8 per-token V scales, and as one fp16
 *    term (11 bits) for static V scales and the KIVI formats.  The absolute
 *    error of an output scales with the magnitude of the values it
 *    averages.
 *
 * One kvq_cache describes ONE layer.  Shapes below use
 *   NB = num_blocks, H = num_kv_heads, Hq = num_q_heads, D = head_dim = 128,
 *   BS = block_size = 16, R = residual_len, G = group_size = 64,
 *   RING = R + G (fp16 ring slots per sequence and head, INT4 only).
 * Token t of batch row b lives in physical block block_tables[b*MBS + t/16],
 * slot t % 16 (MBS = max_blocks_per_seq).
 *
 * ---- INT8 / FP8 code layout: uint8 [NB][H][2048] for each of K and V ------
 * One (block, head) chunk holds 16 tokens x 128 channels.  Byte offset of
 * (slot s, channel c) inside the chunk:
 *   K: 1024*((c>>4)&1) + 256*(c>>5) + 16*s + (c&15)
 *   V: 1024*(c>>6) + 256*(s>>2) + 16*(c&15) + 4*((c>>4)&3) + (s&3)
 * INT8 codes are two's complement; FP8 codes are OCP E4M3 (0x7F/0xFF never
 * written) or, for KVQ_FP8_E5M2, OCP E5M2 (infinities and NaNs never
 * written).  The orders put each lane's matrix-core operand in one 16-byte
 * run so the decode kernel loads tiles straight into registers.
 *
 * ---- INT8 / FP8 scales (fp32), by granularity, for each of K and V ---------
 *   KVQ_PER_TENSOR : [1]            (input)
 *   KVQ_PER_HEAD   : [H]            (input)
 *   KVQ_PER_CHANNEL: [H][128]       (input)
 *   KVQ_PER_TOKEN  : [NB][H][16]    (written by kvq_write, max|x|/127, /448
 *                                    or /57344)
 * A zero scale quantizes every value to code 0.
 *
 * ---- INT4 (KIVI) layout ------------------------------------------------------
 * The first nq(S) = max(0, floor((S-R)/G))*G tokens of a sequence are INT4;
 * tokens nq(S) .. S-1 (R to R+G-1 of them once S >= R) stay fp16 in a ring.
 * A written sequence of length S also holds the INT4 blocks of the group
 * that leaves the window at length S+1 (groups 0 .. nq(S+1)-1 in all):
 * writes flush each group one token early, so that a one-token decode step
 * can flush concurrently with its attention, which does not read it.
 *   k_codes : uint8 [NB][H][1024]; (slot s, channel c) at byte
 *             256*(c>>5) + 16*s + ((c&31)>>1), low nibble for even c.
 *   v_codes : uint8 [NB][H][1024]; with j = c>>4, u = (c&15) + 16*(s>>2),
 *             w = j>>1, e = s&3, nibble p = 2*(j&1) + (e>>1) + 4*(e&1):
 *             byte 16*u + 4*w + (p>>1), low nibble when p is even.
 *   Codes are two's-complement nibbles in [-8, 7].
 *   k_scales: fp32 [NB][H][32]; the block at logical index j of a sequence
 *             holds the per-channel scales (max over the group's 64 tokens
 *             of |K| / 7) of channels 32*(j%4) .. 32*(j%4)+31 of group j/4.
 *   v_scales: fp32 [NB][H][16][2]; per token, channels 0..63 and 64..127
 *             (max over the 64 channels of |V| / 7).
 *   k_resid : fp16 [ring_rows][H][RING][128]; token t at slot t % RING.
 *   v_resid : fp16 [ring_rows][H][RING/4][128][4]; token t at slot
 *             s = t % RING is element [s>>2][c][s&3].
 * Both granularity fields must be KVQ_PER_CHANNEL (K) and KVQ_PER_TOKEN (V).
 *
 * ---- INT4 affine (KVQ_INT4_AFFINE) -------------------------------------------
 * The affine form of [oh-bug] section "量化不是简单'截断精度'": code =
 * clamp(round(x / scale) + zero_point, 0, 15), value = (code - zero_point) *
 * scale.  Per group the range is widened to contain zero: lo = min(min x,
 * 0), hi = max(max x, 0), scale = (hi - lo) / 15 and zero_point =
 * clamp(round(-lo / scale), 0, 15) (fp32, round half to even; a group of
 * zeros has scale 0, zero point 0, codes 0).  Groups, residual window, ring
 * and code positions are those of KVQ_INT4; codes are unsigned nibbles.
 *   k_scales: fp32 [NB][H][40]; floats 0..31 are the per-channel scales of
 *             the INT4 layout, the 32 bytes of floats 32..39 the uint8 zero
 *             points of the same channels (byte i: channel 32*(j%4)+i).
 *   v_scales: fp32 [NB][H][40]; floats 0..31 are [16][2] as for INT4, the
 *             32 bytes of floats 32..39 uint8 zero points, group-transposed:
 *             the zero point of channel group g of token 16*b + 4*u + e of
 *             a 64-token group is byte 8*b + 2*e + g of the row of the
 *             group's block u (b, u, e in 0..3), so one row holds what one
 *             lane row of the decode kernel needs.
 *
 * ---- 2-bit affine (KVQ_INT2_AFFINE) -------------------------------------------
 * The KVQ_INT4_AFFINE rule with codes 0..3 (scale = (hi - lo) / 3), the
 * 2-bit entry of [oh-bug] section "KV Cache 的基本内存模型" (0.25 byte per
 * value) and KIVI's asymmetric 2-bit scheme named in its references.
 * Groups, residual window, ring and the 40-float scale / zero-point rows
 * are those of KVQ_INT4_AFFINE.  Query groups and query counts as for the
 * other formats (n_query * Hq / H <= 16).
 *   k_codes : uint8 [NB][H][512]; (slot s, channel c) at byte
 *             128*(c>>5) + 8*s + ((c&31)>>2), bits 2*(c&3).
 *   v_codes : uint8 [NB][H][512]; with j = c>>4, e = s&3: byte
 *             8*((c&15) + 16*(s>>2)) + 4*((j&3)>>1) + 2*(j&1) + (e>>1),
 *             bits 2*(j>>2) + 4*(e&1) (a byte holds two consecutive tokens
 *             of two tiles, which the decode converts as FP4 nibbles).
 *
 * ---- FP16 (unquantized) layout: fp16 [NB][H][2048] for each of K and V ----
 * The baseline the quantized formats are measured against ([intelli] §5:
 * INT8 against FP16 memory and latency).  Values are stored as given; one
 * (block, head) chunk is 4096 bytes.  Byte offset of (slot s, channel c):
 *   K: 1024*((c>>3)&3) + 256*(c>>5) + 16*s + 2*(c&7)
 *   V: 1024*(c>>5) + 256*(s>>2) + 16*(c&15) + 8*((c>>4)&1) + 2*(s&3)
 * k_codes / v_codes point at these arrays.  There are no scales: the
 * granularity fields are ignored and k_scales / v_scales may be NULL.
 *
 * ---- BF16 (unquantized) layout: KVQ_FP16's with bf16 values ----
 * The other half-precision baseline ([intelli] §5 compares INT8 with the
 * 16-bit cache a model runs in; bf16 is the usual one for Llama-class
 * models).  Byte offsets, chunk size and the absent scales are those of
 * KVQ_FP16.  Every 16-bit input of the calls that take one (q, k_new, v_new)
 * is then bf16; scores use bf16 products with fp32 sums and the softmax
 * weights enter the value product as two bf16 terms, hi = bf16(p) and
 * lo = bf16(p - hi), about 16 significant bits (KVQ_FP16: two fp16 terms,
 * about 22 bits), so both meet the same output tolerance.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* null pointer, bad enum, bad count            */
  KVQ_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim != 128, g > 16 */
  KVQ_ERR_ALIGNMENT = -3,   /* a device pointer is not 16-byte aligned      */
  KVQ_ERR_WORKSPACE = -4,   /* decode workspace too small or misaligned     */
  KVQ_ERR_CAPACITY = -5,    /* a length exceeds max_blocks_per_seq * 16      */
  KVQ_ERR_HIP = -6          /* a kernel launch failed                       */
} kvq_status;

typedef enum kvq_dtype {
  KVQ_INT8 = 1,     /* 1 byte per value, symmetric, divisor 127             */
  KVQ_FP8_E4M3 = 2, /* 1 byte per value, OCP E4M3, divisor 448              */
  KVQ_INT4 = 3,     /* 0.5 byte per value, KIVI grouping, divisor 7         */
  KVQ_FP16 = 4,     /* 2 bytes per value, unquantized                       */
  KVQ_INT4_AFFINE = 5, /* INT4 KIVI grouping, asymmetric: codes 0..15 with a
                          zero point per group                              */
  KVQ_FP8_E5M2 = 6, /* 1 byte per value, OCP E5M2, divisor 57344            */
  KVQ_INT2_AFFINE = 7, /* 2-bit KIVI: 0.25 byte per value, codes 0..3 with a
                          zero point per group                              */
  KVQ_BF16 = 8      /* 2 bytes per value, unquantized bf16 (the FP16 layout);
                       q, k_new and v_new are bf16 for this dtype           */
} kvq_dtype;

typedef enum kvq_granularity {
  KVQ_PER_TENSOR = 0,
  KVQ_PER_HEAD = 1,
  KVQ_PER_CHANNEL = 2,
  KVQ_PER_TOKEN = 3
} kvq_granularity;

/* How a decode launch divides the work among its workgroups.
 *  KVQ_PARTITION_PER_ROW: every row is cut into partitions of split_tokens
 *    tokens; a workgroup streams one partition of one (row, KV head).
 *  KVQ_PARTITION_BALANCED: the blocks of all rows of a KV head, laid end to
 *    end in row order, are cut into one equal range per workgroup (one
 *    workgroup per CU: max(1, 256 / num_kv_heads) per KV head), so rows of
 *    unequal length leave no workgroup short of work ([oh-bug] section
 *    "为什么长上下文更需要 KV Cache Quantization": each step streams each
 *    row's whole history).  A range that crosses rows leaves one partial per
 *    row segment; the merge launch always runs.  INT8, FP8, FP16 and BF16 caches,
 *    batch <= 256; split_tokens is unused.  Results equal the per-row
 *    partitions' up to the order of the fp32 sums. */
typedef enum kvq_partition {
  KVQ_PARTITION_PER_ROW = 0,
  KVQ_PARTITION_BALANCED = 1
} kvq_partition;

/* Shape and quantization scheme of one layer's cache (host struct). */
typedef struct kvq_layout {
  uint32_t struct_size;       /* sizeof(kvq_layout)                          */
  int32_t dtype;              /* kvq_dtype                                   */
  int32_t k_gran;             /* kvq_granularity of K scales                 */
  int32_t v_gran;             /* kvq_granularity of V scales                 */
  int32_t group_size;         /* INT4: must be 64; ignored otherwise         */
  int32_t residual_len;       /* INT4: multiple of 64, >= 64; else ignored   */
  int32_t block_size;         /* must be 16                                  */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads              */
  int32_t num_kv_heads;       /* H; Hq / H must be 1..16                     */
  int32_t head_dim;           /* must be 128                                 */
  int32_t num_blocks;         /* NB, physical blocks in the pool             */
  int32_t max_blocks_per_seq; /* MBS, row length of block_tables             */
  int32_t split_tokens;       /* decode partition length in tokens; 0 picks
                                 one from the grid size.  Multiple of 16
                                 (INT4: of 64).                              */
  int32_t partition;          /* kvq_partition: how a decode launch divides
                                 the rows among workgroups                  */
} kvq_layout;

/* Device buffers of one layer's cache (host struct of device pointers). */
typedef struct kvq_cache {
  void *k_codes;      /* see the layout notes above                          */
  void *v_codes;
  float *k_scales;
  float *v_scales;
  uint16_t *k_resid;  /* INT4 only (else may be NULL)                        */
  uint16_t *v_resid;  /* INT4 only (else may be NULL)                        */
  int32_t ring_rows;  /* INT4: rows of the fp16 rings (>= batch)             */
} kvq_cache;

/* Human-readable name of a status code (static string, never NULL). */
const char *kvq_status_str(kvq_status status);

/* Host-only check of a layout, cache and call size, exactly the checks the
 * entry points run before launching.  Makes no HIP call.
 * batch == 0 is valid (the entry points then do nothing). */
kvq_status kvq_validate(const kvq_layout *layout, const kvq_cache *cache,
                        int32_t batch, int32_t max_seq_len);

/* Bytes of decode workspace for (layout, batch, max_seq_len); 0 if the
 * layout is invalid or if the launch needs none (a single partition per
 * row).  The workspace holds the split-K partials (running max, softmax sum
 * and unnormalised output per partition and query head); its contents need
 * no initialisation and are dead after the call. */
size_t kvq_decode_workspace_bytes(const kvq_layout *layout, int32_t batch,
                                  int32_t max_seq_len);

/* Quantize-on-write: append new K/V tokens to the cache.
 *   k_new, v_new : fp16 [total_new][H][128] (bf16 for a BF16 cache), the
 *                  new tokens of all rows
 *                  packed in row order.
 *   cu_new       : int32 [batch+1], row b's tokens are k_new[cu_new[b] ..
 *                  cu_new[b+1]-1]; cu_new[0] == 0, cu_new[batch] ==
 *                  total_new.
 *   block_tables : int32 [batch][MBS], physical block of each logical block.
 *   seq_lens     : int32 [batch], lengths AFTER this write; the new tokens
 *                  of row b take positions seq_lens[b]-n_b .. seq_lens[b]-1.
 *   max_new_per_seq: host bound on n_b.
 * INT8/FP8: writes codes (and per-token scales when the granularity is
 * KVQ_PER_TOKEN) into the block slots.  Static scales are read from the
 * cache's scale arrays.  FP16 / BF16: stores the values in the block
 * slots.
 * INT4: first quantizes the 64-token groups nq(S_old+1) .. nq(S_new+1)-1
 * (those that leave the fp16 window up to length S_new+1, see the INT4
 * layout; read from the ring or straight from k_new/v_new) into INT4 blocks
 * with their scales, then stores the new tokens from nq(S_new) on in the
 * ring (two launches, in that order, so a ring slot is read before it is
 * reused; one launch when every row takes at most one token).
 * Sequences must be extended in order; positions already written are
 * overwritten with the same values when rewritten. */
kvq_status kvq_write(const kvq_layout *layout, const kvq_cache *cache,
                     const uint16_t *k_new, const uint16_t *v_new,
                     const int32_t *cu_new, const int32_t *block_tables,
                     const int32_t *seq_lens, int32_t batch,
                     int32_t total_new, int32_t max_new_per_seq,
                     void *stream);

/* Decode attention over the quantized paged cache, one query per row:
 *   out[b][hq][:] = sum_t softmax_t(s_t) * v_hat[t],
 *   s_t = softmax_scale * dot(q[b][hq], k_hat[t]),  t < seq_lens[b],
 * with KV head hq / (Hq/H), k_hat/v_hat the dequantized values (code*scale,
 * or fp16 for INT4 residual tokens and for an FP16 cache; bf16 for BF16).
 *   q        : fp16 [batch][Hq][128] (bf16 for a BF16 cache)
 *   out      : fp32 [batch][Hq][128]; rows with seq_lens[b] == 0 get zeros.
 *   workspace: device buffer of at least kvq_decode_workspace_bytes(layout,
 *              batch, max_seq_len) bytes, 256-byte aligned (may be NULL when
 *              that size is 0).  Calls that share a workspace must not
 *              overlap in time (on one stream they never do).
 * Split-K: one launch computes partials per token partition (four
 * wavefronts per partition, merged in LDS), a second launch merges the
 * partitions of each (row, query head) by log-sum-exp in a fixed order, so
 * results are bitwise reproducible.  KVQ_ERR_UNSUPPORTED when the launch
 * would need 2^24 workgroups or more (partitions x rows, rounded up to a
 * multiple of 8, x KV heads); a larger split_tokens avoids it. */
kvq_status kvq_paged_decode(const kvq_layout *layout, const kvq_cache *cache,
                            const uint16_t *q, const int32_t *block_tables,
                            const int32_t *seq_lens, int32_t batch,
                            int32_t max_seq_len, float softmax_scale,
                            float *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* One decode step: quantize-on-write of ONE new token per row followed by
 * decode attention over the updated cache (the per-step append then read of
 * [yunthe] section "PagedAttention与KV Cache量化协同工作原理").  Same cache
 * contents and the same out, bit for bit, as kvq_write with one token per
 * row followed by kvq_paged_decode with these arguments.
 *   k_new, v_new : fp16 [batch][H][128] (bf16 for a BF16 cache); entry b is
 *                  row b's new token, at position seq_lens[b]-1 (seq_lens
 *                  count it).  Rows with seq_lens[b] == 0 take no token and
 *                  their entry is unread.
 *   q, block_tables, seq_lens, max_seq_len, softmax_scale, out, workspace,
 *   workspace_bytes: as for kvq_paged_decode.
 * INT8/FP8/FP16: a single launch (plus the partition merge when the launch
 * is split): the workgroup that streams a row's last partition quantizes
 * (FP16: copies) and stores the row's token (codes and per-token scales)
 * before streaming.
 * INT4: one decode launch (plus the merge) whose last-partition workgroup
 * of each row stores the token in the ring before reading the window, and
 * whose 2 x batch x H further workgroups flush the group that leaves the
 * window at length seq_lens[b]+1, if any; no workgroup of the launch reads
 * what those write.
 * Errors: as for kvq_paged_decode; additionally KVQ_ERR_INVALID_ARG when
 * k_new or v_new is NULL (batch > 0) and KVQ_ERR_ALIGNMENT when either is
 * not 16-byte aligned.  Nothing is enqueued on error. */
kvq_status kvq_write_decode(const kvq_layout *layout, const kvq_cache *cache,
                            const uint16_t *k_new, const uint16_t *v_new,
                            const uint16_t *q, const int32_t *block_tables,
                            const int32_t *seq_lens, int32_t batch,
                            int32_t max_seq_len, float softmax_scale,
                            float *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* kvq_write_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * hipMalloc): the same step, bit for bit, with the split-K partials in a
 * device array the library holds (KVQ_NOALLOC_SCRATCH_BYTES per GPU, kept
 * until the process ends) instead of a caller workspace.  Arguments as for
 * kvq_write_decode without workspace / workspace_bytes; the caller still
 * owns every other buffer.  The library allocates nothing: the array's
 * device address is looked up (hipGetSymbolAddress) on the first call on
 * each device, with the stream's device current.
 * Errors: as for kvq_write_decode; KVQ_ERR_WORKSPACE when the launch's
 * partials (kvq_decode_workspace_bytes) exceed KVQ_NOALLOC_SCRATCH_BYTES
 * (checked before any HIP call; a larger split_tokens needs fewer);
 * KVQ_ERR_HIP when the array's address cannot be found.
 * All calls on one GPU share its array, which keeps the last call's
 * partials (they need no clearing: every one read is written first by the
 * same call).  Calls that overlap in time on one GPU (several streams or
 * host threads) race on it and must be serialised by the caller. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_write_decode_noalloc(const kvq_layout *layout, const kvq_cache *cache,
                                    const uint16_t *k_new, const uint16_t *v_new,
                                    const uint16_t *q, const int32_t *block_tables,
                                    const int32_t *seq_lens, int32_t batch,
                                    int32_t max_seq_len, float softmax_scale, float *out,
                                    void *stream);

/* Partition length for a batch whose row lengths the caller knows on the
 * host (a serving scheduler does): the split_tokens value (tokens, a
 * multiple of 16; of 64 for INT4 caches) that the automatic plan's search
 * picks over the real lengths instead of taking every row to be
 * max_blocks_per_seq blocks long, raised to at least half of each
 * resident workgroup's balanced share of the blocks.  Equal lengths give
 * the automatic plan back; unequal ones get fewer, longer partitions, so
 * the short rows' workgroups leave less of the chip idle.  Set
 * layout->split_tokens to it before sizing the workspace and decoding.  host_seq_lens: HOST int32 [batch], the lengths the decode
 * will see.  Returns the length (> 0) or a negative kvq_status
 * (KVQ_ERR_INVALID_ARG: NULL lengths with batch > 0, a negative length;
 * KVQ_ERR_CAPACITY: a length beyond max_blocks_per_seq * 16; layout
 * errors as kvq_validate).  Host only, no HIP call. */
int32_t kvq_plan_split_tokens(const kvq_layout *layout, const int32_t *host_seq_lens,
                              int32_t batch);

/* The partition mode (kvq_partition) for a batch whose row lengths the
 * caller knows on the host, for the layout as given (its split_tokens, or
 * the automatic plan's when 0): KVQ_PARTITION_BALANCED when the per-row
 * partitions fit in one round of workgroups (one per CU) and their longest
 * workgroup streams more than 1.25 times the mean workgroup's blocks (rows
 * unequal enough that its tail outweighs the balanced launch's merge and
 * second segments); else KVQ_PARTITION_PER_ROW (always for KIVI caches,
 * batch 0 or more than 256 rows).  Set layout->partition to it before sizing the workspace.
 * Returns the mode (>= 0) or a negative kvq_status (as
 * kvq_plan_split_tokens).  Host only, no HIP call. */
int32_t kvq_plan_partition(const kvq_layout *layout, const int32_t *host_seq_lens,
                           int32_t batch);

/* Host-side check of block tables and row lengths, on HOST copies (the
 * entry points cannot check device data before launching; a block id out
 * of range there is an out-of-bounds access).  Checks, in row order:
 *   0 <= host_seq_lens[b] <= max_seq_len <= max_blocks_per_seq * 16;
 *   every table entry a kernel touches for row b is a block id in
 *   [0, num_blocks): entries 0 .. ceil(S_b / 16) - 1, or for KIVI caches
 *   the INT4 blocks 0 .. nq(S_b + 1) / 16 - 1 (see the INT4 layout);
 *   no block id appears twice among those entries of all rows (two rows
 *   sharing a block would overwrite each other's tokens).
 *   host_block_tables: HOST int32 [batch][max_blocks_per_seq];
 *   host_seq_lens    : HOST int32 [batch];
 *   bad_row          : optional (may be NULL); receives the first failing
 *                      row, or -1.
 * Returns KVQ_OK; KVQ_ERR_INVALID_ARG for a negative length, an id out of
 * range or repeated, or NULL arrays with batch > 0; KVQ_ERR_CAPACITY for a
 * length above max_seq_len or max_seq_len above the table's capacity;
 * layout errors as kvq_validate.  Host only, no HIP call; O(num_blocks)
 * host memory. */
kvq_status kvq_check_tables(const kvq_layout *layout, const int32_t *host_block_tables,
                            const int32_t *host_seq_lens, int32_t batch,
                            int32_t max_seq_len, int32_t *bad_row);

/* Decode attention for several new query tokens per row (speculative
 * verification of draft tokens, or a chunk of prefill, over the cache; the
 * whole-history read of [oh-bug] section "为什么长上下文更需要 KV Cache
 * Quantization" shared by n_query queries):
 *   q   : fp16 [batch][n_query][Hq][128] (bf16 for a BF16 cache); query j
 *         of row b sits at position seq_lens[b] - n_query + j (its K/V
 *         already written, e.g. by kvq_write) and attends to tokens
 *         0 .. seq_lens[b] - n_query + j.
 *   out : fp32 [batch][n_query][Hq][128]; a query with no visible token
 *         (seq_lens[b] - n_query + j < 0) gets zeros.
 *   workspace: kvq_paged_decode_mq_workspace_bytes(layout, n_query, batch,
 *         max_seq_len) bytes; otherwise as for kvq_paged_decode (n_query = 1
 *         gives exactly kvq_paged_decode's results).
 * The K/V stream is read once for all queries: the score product's 16
 * columns hold (query, head) pairs.  Errors: as for kvq_paged_decode;
 * KVQ_ERR_INVALID_ARG for n_query < 1; KVQ_ERR_UNSUPPORTED when n_query *
 * (Hq / H) > 16.  INT4 caches: the INT4 groups are seen by every query
 * (they end a residual window before the newest token); the fp16 window
 * is masked per query. */
size_t kvq_paged_decode_mq_workspace_bytes(const kvq_layout *layout, int32_t n_query,
                                           int32_t batch, int32_t max_seq_len);
kvq_status kvq_paged_decode_mq(const kvq_layout *layout, const kvq_cache *cache,
                               const uint16_t *q, int32_t n_query,
                               const int32_t *block_tables, const int32_t *seq_lens,
                               int32_t batch, int32_t max_seq_len, float softmax_scale,
                               float *out, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Static-scale calibration ([yunthe] sections "KV Cache量化策略" (scale =
 * max(abs(x)) / 127) and "配置与启动参数" (per-layer K and V scales computed
 * offline from calibration data); [oh-bug] vLLM section (per-tensor and
 * per-head FP8 scales from a random-token warmup or calibration data)).
 *   k, v         : fp16 [n_tokens][H][128] calibration tokens (e.g. a
 *                  layer's prefill K and V).
 *   k_scales, v_scales: the cache's static scale arrays for the layout's
 *                  granularity ([1], [H] or [H][128]), written as
 *                  max|x| / 127 (INT8), / 448 (E4M3) or / 57344 (E5M2),
 *                  max over the tokens and, per granularity, over the
 *                  head's channels or over everything.  A per-token
 *                  granularity has no static scale: that tensor's input
 *                  and output are unread and may be NULL.
 *   accumulate   : nonzero raises the existing scales to at least the new
 *                  ones (several calibration batches give the scale of all
 *                  of them); zero replaces them.
 *   workspace    : device buffer of kvq_calibrate_workspace_bytes(layout,
 *                  n_tokens) bytes, 256-byte aligned; contents need no
 *                  initialisation.
 * Two launches on `stream`.  Errors: KVQ_ERR_UNSUPPORTED for the KIVI
 * (INT4, affine INT4, 2-bit), FP16 and BF16 caches (no static scales) or
 * more than 256 KV heads; KVQ_ERR_INVALID_ARG
 * for n_tokens < 0 or a missing pointer of a calibrated tensor;
 * KVQ_ERR_ALIGNMENT, KVQ_ERR_WORKSPACE as elsewhere.  n_tokens == 0 does
 * nothing. */
size_t kvq_calibrate_workspace_bytes(const kvq_layout *layout, int32_t n_tokens);
kvq_status kvq_calibrate(const kvq_layout *layout, const uint16_t *k,
                         const uint16_t *v, int32_t n_tokens, float *k_scales,
                         float *v_scales, int32_t accumulate, void *workspace,
                         size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
