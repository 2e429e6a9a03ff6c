/*
 * lgm_mla.h — paged multi-head latent attention (MLA) decode for AMD MI355X
 * (gfx950), beside the GQA calls of lgm.h and with the same conventions
 * (ownership, device pointers, stream, validation before any HIP call, error
 * text through lgm_last_error(), device-resident context lengths and block
 * tables as the caller's contract).
 *
 * Source: mainarch README (MaincodeHQ/mainarch), MLA section: the cache holds
 * one compressed latent per token instead of per-head K and V — a
 * 512-element FP8 E4M3 "ckv" beside a 64-element bf16 positional "kpe" —
 * and the per-head projections happen after the cache read, so all query
 * heads attend to the same latent rows; the kernel computes per-head dot
 * scores, a local softmax with exported LSE and softmax-weighted latent
 * output tiles, split-K across the sequence with a stage-2 merge of the
 * partial records.
 *
 * Layouts (row-major, innermost last):
 *   q_latent   [B][H][512] bf16, dense;  q_pe [B][H][64] bf16, dense
 *   ckv cache  [num_blocks][block_size][512] FP8 E4M3 codes
 *   kpe cache  [num_blocks][block_size][64] bf16
 *   block table int32 [B][max_blocks_per_seq], one table for both pools
 *   context len int32 [B] (clamped to [0, max_context_len])
 *   out        [B][H][512] bf16, dense;  out_lse fp32 [B][H]
 * A block-table entry outside [0, num_blocks) is never dereferenced: its
 * tokens are masked.
 */
#ifndef LGM_MLA_H
#define LGM_MLA_H

#include <stddef.h>
#include <stdint.h>

#include "lgm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* num_seqs = B, num_heads = H query heads, latent_dim (512) and rope_dim
 * (64) elements per token, block_size tokens per cache block, num_blocks
 * blocks in each pool, max_blocks_per_seq = block table row length. */
typedef struct lgm_mla_dims {
  int32_t num_seqs;
  int32_t num_heads;
  int32_t latent_dim;
  int32_t rope_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
} lgm_mla_dims;

/*
 * Partition size (tokens) lgm_paged_mla_decode uses for these arguments:
 * partition_size itself (capped to max_context_len rounded up to 32) when
 * positive, else one that gives about one workgroup per compute unit (256)
 * at max_context_len over the batch: ceil(B * max_context_len / 256)
 * rounded up to a multiple of 64 (the kernel's tile), at least 128, and
 * capped as above.  Returns -1 (and sets
 * lgm_last_error) on invalid arguments.
 */
int32_t lgm_paged_mla_partition_size(lgm_mla_dims dims, int32_t max_context_len, int32_t partition_size);

/*
 * Bytes of device workspace lgm_paged_mla_decode needs: with P =
 * ceil(max_context_len / partition) > 1, fp32 partial outputs
 * [B][H][P][512] then their natural-log LSEs [B][H][P] (each region 256-byte
 * aligned); 0 without a split.  Returns 0 and sets lgm_last_error on invalid
 * arguments.
 */
size_t lgm_paged_mla_workspace_size(lgm_mla_dims dims, int32_t max_context_len, int32_t partition_size);

/*
 * Paged MLA decode (mainarch README, MLA section).  For each sequence b,
 * query head h, L = min(context_lens[b], max_context_len), tokens j < L
 * through the block table, c_j = decode(ckv_j) * ckv_scale[0], r_j = kpe_j:
 *   s_j = softmax_scale * (<q_latent[b][h], c_j> + <q_pe[b][h], r_j>),
 *   out[b][h] = sum_j softmax(s)_j c_j,
 *   out_lse[b][h] = log(sum_j exp(s_j))   (natural log; -inf, out = 0 when L = 0).
 * Contexts are cut into partitions of lgm_paged_mla_partition_size tokens,
 * one workgroup each; a sequence with more than one writes fp32 records to
 * the workspace, merged by log-sum-exp (as lgm_lse_merge) on the same
 * stream within this call; a sequence in one partition is written directly.
 * Arithmetic: FP8 codes and query values enter the matrix cores as bf16
 * (exact for the codes), products accumulate in fp32, probabilities enter
 * the output product rounded to bf16; one final rounding to bf16.
 *
 *   out            [B][H][512] bf16, 16-byte aligned; must not overlap any input
 *   out_lse        optional fp32 [B][H] (NULL = not written)
 *   q_latent, q_pe bf16 [B][H][512] and [B][H][64], 16-byte aligned
 *   ckv_cache      FP8 E4M3 pool, 16-byte aligned, read only
 *   kpe_cache      bf16 pool, 16-byte aligned, read only
 *   ckv_scale      fp32 [1], the static per-tensor scale of the codes
 *   softmax_scale  finite
 *   partition_size 0 = library chooses; else a positive multiple of 32;
 *                  >= max_context_len means no split
 *   max_context_len upper bound on context_lens, 0..max_blocks_per_seq*block_size
 *   workspace      device buffer of lgm_paged_mla_workspace_size() bytes,
 *                  256-byte aligned (NULL allowed when that size is 0)
 *   ckv_dtype      LGM_FP8_E4M3
 * Supported: latent_dim 512, rope_dim 64, num_heads 1..16, block_size a
 * power of two, num_seqs <= 65535.
 */
lgm_status lgm_paged_mla_decode(void* out, float* out_lse, const void* q_latent, const void* q_pe,
                                const void* ckv_cache, const void* kpe_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const float* ckv_scale, float softmax_scale,
                                int32_t partition_size, int32_t max_context_len, void* workspace,
                                size_t workspace_bytes, lgm_mla_dims dims, lgm_dtype ckv_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LGM_MLA_H */
