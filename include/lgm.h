/*
 * lgm.h — paged GQA/MQA single-token decode attention for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Sources the operations follow:
 *   [Loom]     Loom Kernels README (feichai0017/loom-kernels):
 *              "Supported operator paths" table, rows "Position and KV"
 *              (NeoX RoPE + native/static-FP8 paged-KV write over packed QKV
 *              into NHD cache views, static per-tensor/per-head FP8 E4M3
 *              scales, current-stream execution) and "Attention" (paged
 *              MQA/GQA decode, local split-K/LSE merge); "Next value program"
 *              (exact E4M3 cache bytes); "Architecture" (the backend accepts
 *              the exact contract or returns an error, borrowed pointers and
 *              the caller's stream).
 *   [mainarch] mainarch README (MaincodeHQ/mainarch), decode-attention
 *              section: FlashDecoding split-KV online softmax with a combine
 *              of partial results, paged KV through a block table, GQA reads
 *              the cache once per head group, OCP e4m3fn KV, every buffer in
 *              VRAM (a host-visible scratch buffer pinned the whole pipeline
 *              at 230 GB/s).
 *   [microLLM] microLLM-rocm README, "Detailed implementation and experiment
 *              ledger": split-half RoPE; positions-aware RoPE with mapped KV
 *              store and per-row-prefix cached attention; bf16 KV storage
 *              with fp32 accumulation.
 *
 * Conventions shared by every call
 * --------------------------------
 * Ownership: the caller owns all memory.  Every pointer is borrowed for the
 *   duration of the (asynchronous) work; the library allocates nothing, on
 *   the device or the host, and keeps no pointer after the call returns.
 * Device pointers: all tensor arguments are device (HBM) pointers.
 * Stream: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Work is enqueued on it; no call synchronises the host.
 * Validation: every host-visible argument (pointers for NULL, dims, dtypes,
 *   strides, partition size, workspace size, address-range aliasing) is
 *   checked before any HIP call.  On a violation the call returns a nonzero
 *   lgm_status, enqueues nothing, writes nothing, and lgm_last_error() names
 *   the function, the argument and what was expected.  Unsupported
 *   (dtype, head_dim, group, block_size) combinations return
 *   LGM_ERR_UNSUPPORTED; there is no fallback path.  A failed launch returns
 *   LGM_ERR_HIP.  Device-side faults surface at the caller's next sync.
 * Device-resident contents (context lengths, block-table entries) cannot be
 *   read by the host without a sync and are the caller's contract:
 *     - context_lens[b] is clamped to [0, max_blocks_per_seq * block_size]
 *       (and, for attention, to max_context_len); a sequence with length 0
 *       is inactive;
 *     - a block-table entry outside [0, num_blocks) is never dereferenced: the
 *       append skips that write and attention masks those 16 tokens.
 *   Entries for logical blocks at or beyond ceil(ctx / block_size) are never
 *   read, so they may hold anything.
 * Layouts (row-major, innermost last):
 *   packed QKV  [B][(Hq + 2*Hkv) * D] per row: Q heads, then K heads, then V
 *               heads, each D contiguous; rows qkv_row_stride elements apart.
 *   KV caches   NHD: [num_blocks][block_size][Hkv][D], K and V in separate
 *               pools with identical indexing and dtype.  With LGM_CACHE_HND
 *               the pools are [num_blocks][Hkv][block_size][D] instead.
 *   FP4 cache blocks (LGM_FP4_E2M1): block i of a pool is the byte range
 *               [i * S, (i + 1) * S), S = block_size * Hkv * (D/2 + D/32):
 *               first the codes, NHD [block_size][Hkv][D/2] bytes (element
 *               2k in the low nibble of byte k, 2k+1 in the high nibble),
 *               then the scales, [block_size][Hkv][D/32] E8M0 bytes (scale s
 *               of a row covers its elements 32s .. 32s+31).  With
 *               LGM_CACHE_HND both parts are head-major: [Hkv][block_size][..].  The scales
 *               travel with their block, so no scale pointer is passed.
 *   block table int32 [B][max_blocks_per_seq]: logical block -> physical.
 *   context len int32 [B]: tokens in the cache INCLUDING the new token, so
 *               the new token sits at position ctx - 1.
 *   q / out     [B][Hq][D]; q rows q_seq_stride elements apart, out dense.
 * Query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 */
#ifndef LGM_H_
#define LGM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LGM_ABI_VERSION 7

/* Bytes of int32 counters at the start of every nonzero attention workspace
 * (see lgm_paged_decode_workspace_size): zero on entry, left zero. */
#define LGM_COUNTER_SLOT_BYTES 4096u

typedef enum lgm_status {
  LGM_OK = 0,
  LGM_ERR_INVALID_ARGUMENT = 1,
  LGM_ERR_UNSUPPORTED = 2,
  LGM_ERR_WORKSPACE_TOO_SMALL = 3,
  LGM_ERR_HIP = 4
} lgm_status;

/* Element types.  LGM_FP8_E4M3 is OCP e4m3fn ([mainarch]): bias 7, largest
 * finite 448, 0x7F/0xFF NaN, no infinities.  LGM_FP4_E2M1 is a cache type
 * only ([mainarch] names an E2M1 KV cache with E8M0 block scales), in the OCP
 * Microscaling form: E2M1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), one
 * E8M0 scale byte 2^(byte - 127) per 32 consecutive head_dim elements of a
 * (token, kv head) row; see "FP4 cache blocks" above. */
/* A C caller may pass any int here; every call rejects values that are not
 * listed.  C++ sees the enum with a fixed 32-bit underlying type, so such a
 * value is an ordinary value of the type there too (without one, loading it
 * would be undefined behaviour in C++); the size and passing are the same. */
#ifdef __cplusplus
typedef enum lgm_dtype : int32_t { LGM_F32 = 0, LGM_BF16 = 1, LGM_FP8_E4M3 = 2, LGM_FP4_E2M1 = 3 } lgm_dtype;
#else
typedef enum lgm_dtype { LGM_F32 = 0, LGM_BF16 = 1, LGM_FP8_E4M3 = 2, LGM_FP4_E2M1 = 3 } lgm_dtype;
#endif

/* Contract-variant flags ([Loom] "Position and KV": NeoX/interleaved RoPE,
 * NHD/HND cache views, static per-tensor/per-head FP8 scales), OR-ed into
 * the `flags` argument; 0 selects NeoX RoPE, NHD caches and per-head scales.
 * Each call rejects bits it does not document with LGM_ERR_INVALID_ARGUMENT. */
#define LGM_ROPE_INTERLEAVED 0x1u /* append: rotate adjacent pairs (x[2i], x[2i+1]) */
#define LGM_CACHE_HND 0x2u        /* append and attention: caches stored head-major, see Layouts */
#define LGM_SCALE_PER_TENSOR 0x4u /* append and attention, FP8 caches: one K and one V scale */

/* Shapes shared by the calls.  num_seqs = B, num_q_heads = Hq,
 * num_kv_heads = Hkv (Hq % Hkv == 0), head_dim = D, block_size = tokens per
 * cache block, num_blocks = blocks in each pool, max_blocks_per_seq = block
 * table row length. */
typedef struct lgm_paged_dims {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
} lgm_paged_dims;

/*
 * Fused NeoX (or interleaved) RoPE + paged-KV append of the new token
 * ([Loom] "Position and KV"; [microLLM] split-half RoPE, mapped KV store).
 *
 * For each sequence b with ctx = context_lens[b] >= 1, pos = ctx - 1:
 *   every Q head and K head x of qkv row b is rotated split-half:
 *     pair i < D/2 is (x[i], x[i + D/2]), angle = pos * theta^(-2i/D),
 *     y[i] = x[i] cos - x[i+D/2] sin,  y[i+D/2] = x[i+D/2] cos + x[i] sin,
 *   (with LGM_ROPE_INTERLEAVED: pair i is (x[2i], x[2i+1]), same angle,
 *     y[2i] = x[2i] cos - x[2i+1] sin,  y[2i+1] = x[2i+1] cos + x[2i] sin),
 *   evaluated as: angle, cos and sin in fp64, cos and sin rounded once to
 *   fp32, then each product and each sum rounded to fp32 (no fused
 *   multiply-add);
 *   rotated Q -> q_out[b] (act dtype, round to nearest even);
 *   rotated K and the unrotated V head g -> slot (pos % block_size) of
 *   physical block block_tables[b][pos / block_size], kv head g, in the
 *   cache dtype: f32 as is, bf16 round to nearest even, FP8 E4M3 as
 *   E4M3(y / scale[g]) with an IEEE fp32 division, round to nearest even,
 *   magnitudes above 448 saturating to +-448, sign kept for zero.  FP4:
 *   each 32-element block of the row gets the scale exponent
 *   X = floor(log2(max |y|)) - 2 clamped to [-127, 127] (byte X + 127; an
 *   all-zero block gets byte 0), and each element the E2M1 code of
 *   y / 2^X (exact), rounded to nearest with ties to the even mantissa,
 *   magnitudes above 6 saturating to 6, sign kept for zero.
 * A sequence with ctx <= 0 writes nothing to the caches and its q_out row is
 * Q unrotated (angle 0).
 *
 *   qkv            [B][row] act dtype, row stride qkv_row_stride >= (Hq+2Hkv)*D
 *   q_out          [B][Hq][D] act dtype (dense); must not overlap any input
 *   k_cache,v_cache NHD (or HND) pools, cache dtype; written only at the B slots
 *   block_tables   int32 [B][max_blocks_per_seq]
 *   context_lens   int32 [B]
 *   k_scale,v_scale fp32 [Hkv] when cache_dtype is LGM_FP8_E4M3 ([1] with
 *                  LGM_SCALE_PER_TENSOR), else NULL
 *   rope_theta     > 0, finite
 *   flags          LGM_ROPE_INTERLEAVED | LGM_CACHE_HND | LGM_SCALE_PER_TENSOR
 *                  (the last for FP8 caches only)
 * Supported: (act, cache) in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 * (BF16, FP4_E2M1)}; head_dim even, 2..256 (a multiple of 32 for FP4);
 * block_size >= 1.  Append slots must be distinct
 * across the batch (the caller's contract; two sequences writing one slot
 * race).
 */
lgm_status lgm_rope_kv_append(const void* qkv, int64_t qkv_row_stride, void* q_out, void* k_cache,
                              void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const float* k_scale,
                              const float* v_scale, float rope_theta, lgm_paged_dims dims,
                              lgm_dtype act_dtype, lgm_dtype cache_dtype, uint32_t flags,
                              void* stream);

/*
 * The partition size the attention call will use, or 0 for equal ranges.
 * A positive partition_size must be a multiple of block_size and is returned
 * as is (clamped to the rounded-up max_context_len).  partition_size 0 lets
 * the library choose from the shapes alone (deterministic, no device query):
 *  - small jobs on the matrix-core shapes (bf16 activations, bf16 / FP8 /
 *    FP4 caches, head_dim 128): at most 1022 (sequence, kv head) streams and
 *    at most 16384 32-token tiles over them at max_context_len (32768 for
 *    FP8 caches).  One launch: plain ceil(L / partition) partitions of a
 *    multiple of 128 tokens (at most 64 per context, at most 1024 tokens per
 *    wave), the size that best balances the (sequence, kv head, partition)
 *    workgroups over 256 compute units, counting a fixed cost of 128 tokens
 *    per workgroup; the workgroup that finishes a context's last partition
 *    merges that context by log-sum-exp.  Returns the partition;
 *  - larger jobs on the matrix-core shapes: returns 0.  The 32-token tiles
 *    of all contexts, per head group (8 kv heads when 8 divide num_kv_heads
 *    and num_q_heads / num_kv_heads is at most 8, else 4 when 4 divide it,
 *    else 2 when 2 do, else 1), are cut into equal ranges, one per compute
 *    unit (256, fewer when a range would hold under 2 tiles); each workgroup
 *    reads whole KV rows of its head group (with a group of 2 or 1 kv heads
 *    its four waves take each head's tiles in 2 or 4 interleaved slices and
 *    combine them), and contexts split between ranges are merged by
 *    log-sum-exp;
 *  - other shapes: a size that gives about 8192 workgroups.
 * How contexts are cut into partitions:
 *  - the whole-row partition plan, taken when the matrix-core shapes have
 *    an even num_kv_heads and an explicit partition_size that is a
 *    multiple of 32 and at least 256 tokens, max_context_len holds at least
 *    64 partitions and the batch at least 256 (sequence, head group as
 *    above, partition) units: plain ceil(L / partition) partitions, run
 *    in equal numbers of whole partitions per workgroup (256 workgroups of
 *    whole KV rows);
 *  - every other partitioned plan: when max_context_len exceeds the
 *    partition size, each context is cut into floor(L / partition) full
 *    partitions followed by partitions of half that size (at least
 *    block_size) over the rest, which are processed last.
 * Returns -1 (and sets lgm_last_error) on invalid arguments.
 */
int32_t lgm_paged_decode_partition_size(lgm_paged_dims dims, int32_t max_context_len,
                                        int32_t partition_size, lgm_dtype cache_dtype);

/*
 * Bytes of device workspace lgm_paged_decode_attn needs for these
 * arguments, 0 when the plan needs none.  A nonzero workspace always starts
 * with the same slot of LGM_COUNTER_SLOT_BYTES (1024 int32 counters), which
 * must be zero on entry and which every plan leaves zero: the work-queue plan
 * uses words 0 and 1, the single-launch plan one arrival counter per
 * (sequence, kv head) stream from word 2 on, the other plans none.  After it come the plan's own
 * regions, each 256-byte aligned:
 *  - single launch (small jobs, see lgm_paged_decode_partition_size): when
 *    contexts are split, one record per (sequence, kv head, partition):
 *    fp32 outputs [B * Hkv][P][G][D], then natural-log LSEs [B * Hkv][P][G];
 *  - equal ranges (see lgm_paged_decode_partition_size): two records per
 *    range (fp32 outputs of the head group's HG * Hq / Hkv query heads, D
 *    each, and their natural-log LSEs; HG = 8, 4, 2 or 1 kv heads as in
 *    lgm_paged_decode_partition_size), then int32 context
 *    bookkeeping (two per context and head group);
 *  - partitions (the whole-row partition plan, the work-queue plan on the
 *    other matrix-core shapes, the vector-ALU plan on the rest): when
 *    contexts are split, fp32 partial outputs [B][Hq][P][D] and LSEs
 *    [B][Hq][P], P = the most partitions any context up to max_context_len
 *    is cut into.  Without a split the work-queue plan needs the slot alone
 *    and the other two plans need no workspace.
 * Returns 0 and sets lgm_last_error on invalid arguments (check it when 0
 * is unexpected).
 */
size_t lgm_paged_decode_workspace_size(lgm_paged_dims dims, int32_t max_context_len,
                                       int32_t partition_size, lgm_dtype cache_dtype);

/*
 * Paged GQA/MQA decode attention ([mainarch] decode attention; [Loom]
 * "Attention").  For each sequence b, query head h, kv head g = h / G,
 * L = min(context_lens[b], max_context_len):
 *   s_j = softmax_scale * <q[b][h], K_j>,  j < L, K_j = cache row of token j
 *         through the block table (FP8: decoded byte * k_scale[g]; FP4:
 *         each E2M1 code times its block's E8M0 scale),
 *   out[b][h] = sum_j softmax(s)_j V_j   (FP8: V_j = decoded byte * v_scale[g]),
 *   out_lse[b][h] = log(sum_j exp(s_j))  (natural log; -inf and out = 0 when L = 0).
 * Arithmetic is fp32 with one final rounding to the act dtype.  Contexts are
 * cut into partitions (see lgm_paged_decode_partition_size) processed in
 * parallel; partial results are merged by log-sum-exp (as lgm_lse_merge) on
 * the same stream, within this call.  A sequence that fits one partition is
 * written directly.  Small jobs take one launch, whose workgroups merge the
 * contexts they finish; the whole-row plan cuts equal tile ranges; the
 * work-queue plan runs as many workgroups as the device keeps resident, each
 * taking (sequence, partition, kv head) items from the workspace's work
 * counters until none is left.
 *
 *   out            [B][Hq][D] act dtype (dense)
 *   out_lse        optional fp32 [B][Hq] (NULL = not written)
 *   q              [B][Hq][D] act dtype, rows q_seq_stride >= Hq*D elements apart;
 *                  may be the q_out of lgm_rope_kv_append
 *   k_cache,v_cache NHD (or HND) pools (cache dtype), read only
 *   k_scale,v_scale fp32 [Hkv] for LGM_FP8_E4M3 caches ([1] with
 *                  LGM_SCALE_PER_TENSOR), else NULL
 *   softmax_scale  finite (normally 1/sqrt(D) rounded to fp32)
 *   partition_size 0 = library chooses; else a positive multiple of
 *                  block_size; >= max_context_len means no split
 *   max_context_len upper bound on context_lens, 0..max_blocks_per_seq*block_size
 *   workspace      device buffer of at least lgm_paged_decode_workspace_size()
 *                  bytes, 256-byte aligned (NULL allowed when that size is 0).
 *                  Its first LGM_COUNTER_SLOT_BYTES (the counters) must be zero
 *                  before the first call on it; every completed call, on any
 *                  plan, leaves them zero, so one buffer may serve calls with
 *                  different shapes and plans in turn.  Zero-fill it again
 *                  after a call on it failed to complete.  Calls sharing a
 *                  workspace must not overlap in time (one per stream).
 *   flags          LGM_CACHE_HND | LGM_SCALE_PER_TENSOR (the latter for FP8
 *                  caches only); LGM_ROPE_INTERLEAVED is rejected here
 * Supported: (act, cache) in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3)},
 * head_dim in {64, 128}, block_size 16, G = Hq/Hkv in 1..8; with bf16
 * activations at head_dim 128, G in 1..16 (matrix-core kernel); and
 * (BF16, FP4_E2M1) at head_dim 128, block_size 16, G in 1..16.  FP4 codes
 * and scales decode exactly; a scale byte 0xFF is NaN, as E8M0 defines.
 * out (16-byte aligned) must not overlap q, the caches or the workspace.
 */
lgm_status lgm_paged_decode_attn(void* out, float* out_lse, const void* q, int64_t q_seq_stride,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const float* k_scale, const float* v_scale, float softmax_scale,
                                 int32_t partition_size, int32_t max_context_len, void* workspace,
                                 size_t workspace_bytes, lgm_paged_dims dims, lgm_dtype act_dtype,
                                 lgm_dtype cache_dtype, uint32_t flags, void* stream);

/*
 * lgm_paged_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It computes exactly what
 * lgm_paged_decode_attn computes (same plans, same kernels, bitwise the same
 * results) and allocates nothing: its workspace is a device-resident array
 * of LGM_STATIC_SCRATCH_BYTES inside the library, one per GPU it runs on,
 * held until the process ends.
 *   - The first call on a device looks the array up on that device and
 *     clears its work-counter slot with a kernel on `stream`; every
 *     completed call leaves that slot zero again.
 *   - Calls whose lgm_paged_decode_workspace_size exceeds
 *     LGM_STATIC_SCRATCH_BYTES return LGM_ERR_WORKSPACE_TOO_SMALL and
 *     launch nothing (use lgm_paged_decode_attn with a workspace instead).
 *   - Every call on a GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (on different streams, or from different threads
 *     without ordering) race and give wrong results.  Order them, e.g. on
 *     one stream.
 * Arguments, layouts, validation and errors are those of
 * lgm_paged_decode_attn, less workspace and workspace_bytes.
 */
#define LGM_STATIC_SCRATCH_BYTES (32u << 20)
lgm_status lgm_paged_decode_attn_static(void* out, float* out_lse, const void* q, int64_t q_seq_stride,
                                        const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                        const int32_t* context_lens, const float* k_scale, const float* v_scale,
                                        float softmax_scale, int32_t partition_size, int32_t max_context_len,
                                        lgm_paged_dims dims, lgm_dtype act_dtype, lgm_dtype cache_dtype,
                                        uint32_t flags, void* stream);

/*
 * Log-sum-exp merge of split-K records ([mainarch] combine of split
 * partials; [Loom] local split-K/LSE merge).  For each (b, h) with
 * n = num_partitions[b] (clamped to [0, max_partitions]; NULL = all):
 *   M = max_p lse_p,  w_p = exp(lse_p - M),
 *   out[b][h] = sum_p w_p o_p / sum_p w_p,  out_lse[b][h] = M + log(sum_p w_p);
 * records with lse = -inf weigh 0 and their partial_out rows are not
 * used (they may hold anything, NaN or Inf included); n = 0 or all -inf
 * gives out = 0, out_lse = -inf.  Summation order is fixed (bitwise
 * reproducible).
 *
 *   out            [B][H][D] out_dtype (LGM_F32 or LGM_BF16), dense
 *   out_lse        optional fp32 [B][H]
 *   partial_out    fp32 [B][H][max_partitions][D], normalised partial outputs
 *   partial_lse    fp32 [B][H][max_partitions], natural log
 *   num_partitions optional int32 [B]
 * Supported: head_dim 64, 128 or 512 (the MLA latent).
 */
lgm_status lgm_lse_merge(void* out, float* out_lse, const float* partial_out,
                         const float* partial_lse, const int32_t* num_partitions,
                         int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                         int32_t max_partitions, lgm_dtype out_dtype, void* stream);

/*
 * Opt-in check of the block tables and context lengths (the debug check of
 * the paged-KV contract; the span check of the mainarch README's
 * troubleshooting section is its model).  The attention and append kernels
 * never dereference a table entry outside [0, num_blocks) and clamp context
 * lengths, silently; enqueued on the same stream before or after them, this
 * call reads the same device-resident entries with the same clamping and
 * raises counters in `status` where they would mask or clamp:
 *   status[0] += table entries of logical blocks < ceil(ctx / block_size)
 *                (ctx clamped to [0, max_blocks_per_seq * block_size]) that
 *                lie outside [0, num_blocks)
 *   status[1] += sequences whose context_lens[b] exceeds
 *                max_blocks_per_seq * block_size or max_context_len
 *   status[2]  = the largest 0x7FFFFFFF - (b * max_blocks_per_seq + lb) over
 *                bad entries: the first bad (sequence b, logical block lb) is
 *                0x7FFFFFFF - status[2] when status[0] > 0
 *   status[3]  unused (left as is)
 * status is int32 [4] device memory the caller zero-fills before the first
 * check; later checks only add to it.  Read it after synchronising.
 *   block_tables   int32 [B][max_blocks_per_seq];  context_lens  int32 [B]
 *   max_context_len the value the attention call is given (0..capacity)
 * dims.num_seqs <= 65535.  Nothing else is read or written.
 */
lgm_status lgm_check_block_tables(const int32_t* block_tables, const int32_t* context_lens, lgm_paged_dims dims,
                                  int32_t max_context_len, int32_t* status, void* stream);

/* Message of the last failed lgm_* call on this thread ("" if none).  Valid
 * until the next lgm_* call on the same thread. */
const char* lgm_last_error(void);

/* LGM_ABI_VERSION of the loaded library. */
int32_t lgm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LGM_H_ */
