/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged GQA attention library.
 *
 * Device entry points (decode, merge, prefill, cache writes; bf16, FP8 and
 * x-packed cache variants) plus host helpers.  All pointers to tensors are
 * DEVICE pointers owned by the caller; the library never allocates, frees or
 * synchronizes.  Work is enqueued on `stream` (a hipStream_t passed as void*;
 * NULL = the default stream).  Every entry point validates its scalar
 * arguments on the host first and returns a status without launching
 * anything on error; there is no fallback to another implementation.
 * Device-resident values (block ids, seq_lens, cu_seqlens) are not checked:
 * out-of-range values are undefined behaviour.
 *
 * Data types and layouts (row-major, contiguous):
 *   q, out       bf16  [num_seqs, H_q, D]           decode
 *                bf16  [total_q,  H_q, D]           prefill (packed ragged rows)
 *   k_cache,
 *   v_cache      bf16  [num_blocks, H_kv, block_size, D]
 *   block_tables int32 [num_seqs, max_blocks_per_seq]   logical -> physical block
 *   seq_lens     int32 [num_seqs]   KV length INCLUDING the current / new tokens
 *   cu_seqlens   int32 [num_seqs + 1]  cu[0] = 0, non-decreasing (prefill rows)
 *   max_logits,
 *   exp_sums     fp32  [num_seqs, H_q, max_num_partitions]
 *   tmp_out      fp32  [num_seqs, H_q, max_num_partitions, D]
 * The cache layout and the block-table walk are those of the RL.cu
 * "Add Cuda Kernel" page (include/kernels/attention.cuh, paged decode
 * launcher); the partial names follow the BI-V100 paged-attention design page,
 * section 2 "Level 3: Cross-Partition Coordination"; cu_seqlens is the
 * qo_indptr of the AstrAI "CUDA Kernels" page, "Q Scheduling and KV
 * Addressing".  Query head h reads kv head h / (H_q / H_kv).
 *
 * Supported: head_dim in {64, 128, 256}; block_size 16; H_q % H_kv == 0 with
 * H_q / H_kv <= 16; partition_size a multiple of block_size.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum paged_attn_status {
    PA_OK = 0,
    PA_ERR_NULL_POINTER = 1,  /* a required pointer is NULL */
    PA_ERR_BAD_SHAPE = 2,     /* non-positive size, H_q % H_kv, partition size, buffer too small */
    PA_ERR_UNSUPPORTED = 3,   /* head_dim, block_size or GQA group outside the supported set */
    PA_ERR_LAUNCH = 4,        /* the HIP runtime rejected a launch */
    PA_ERR_ALIGNMENT = 5,     /* a bf16 / fp32 tensor pointer is not 16-byte aligned */
    PA_ERR_BAD_VALUE = 6,     /* scale is not a positive finite number */
    PA_ERR_SCRATCH_LIMIT = 7  /* paged_attn_decode_fused_noalloc: the problem exceeds its fixed scratch */
};

/*
 * Paged GQA decode: for every sequence s and query head h,
 *   out[s,h,:] = softmax(scale * q[s,h,:] . K_s^T) V_s
 * over the seq_lens[s] tokens whose K/V rows are found through
 * block_tables[s, t / block_size], slot t % block_size (BI-V100 design page,
 * section 1 "Problem Definition"; RL.cu page, paged decode kernel).
 *
 * partition_size == 0: one pass per sequence; writes `out` (bf16, rounded to
 *   nearest even).  max_logits / exp_sums / tmp_out are ignored (may be NULL).
 * partition_size  > 0: split-KV.  Partition p of sequence s covers tokens
 *   [p*P, min((p+1)*P, L)).  For p < ceil(L / P) it writes
 *     max_logits[s,h,p] = exact max of the scaled scores (natural-log units),
 *     exp_sums[s,h,p]   = sum of exp(score - max_logits),
 *     tmp_out[s,h,p,:]  = sum exp(score - max_logits) v / exp_sums
 *   (the BI-V100 page's "attention_partial", with the weighted value sum
 *   stored normalized).  Partitions at or beyond ceil(L / P) are not written.
 *   `out` is ignored; paged_attn_decode_reduce merges the partials.
 *   max_num_partitions must be >= paged_attn_num_partitions(max_blocks_per_seq,
 *   block_size, partition_size).
 * A sequence with seq_lens[s] == 0 gets zeros (single pass) / no partials.
 * scale must be positive and finite (PA_ERR_BAD_VALUE otherwise), as for
 * every entry point that takes it.
 * num_seqs == 0 is a no-op returning PA_OK.
 */
int paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *seq_lens,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                      int partition_size, void *out, float *max_logits, float *exp_sums,
                      float *tmp_out, int max_num_partitions, void *stream);

/*
 * Cross-partition merge (BI-V100 design page, section 2 "combine" and
 * "Level 3"): for each (s, h), with n = ceil(seq_lens[s] / partition_size),
 *   M = max_{p<n} max_logits[s,h,p],  w_p = exp(max_logits[s,h,p] - M) * exp_sums[s,h,p],
 *   out[s,h,:] = bf16( sum_p w_p tmp_out[s,h,p,:] / sum_p w_p ).
 * A sequence with seq_lens[s] == 0 gets zeros.  Reads only p < n.
 */
int paged_attn_decode_reduce(const float *max_logits, const float *exp_sums,
                             const float *tmp_out, const int32_t *seq_lens, int num_seqs,
                             int num_q_heads, int head_dim, int partition_size,
                             int max_num_partitions, void *out, void *stream);

/*
 * Decode with the cross-partition merge fused into the partition kernel (the
 * BI-V100 design page, section 2 "Level 3", names two ways to merge: a
 * separate kernel, or whichever partition block finishes last -- this is the
 * second).  Same inputs and
 * partial buffers as paged_attn_decode with partition_size > 0, which here
 * are workspace (their contents are not partition partials); writes the bf16
 * `out` for every sequence in one launch, zero rows for zero-length
 * sequences.  Schedule: with up to 1024 sequences and max_num_partitions >= 2
 * (and ceil(max_blocks_per_seq / (max_num_partitions - 1)) <= 256), the
 * tiles of all (sequence, kv head) pairs are split evenly across the
 * workgroups (stream-K): each workgroup's share of a pair leaves one record,
 * at most max_num_partitions per pair; otherwise one record per partition of
 * partition_size tokens.  Each workgroup that writes a record increments the
 * arrival counter of its (sequence, kv head); the workgroup completing the
 * set merges the records in token order (deterministic) and resets the
 * counter.  A pair whose tokens form a single record writes `out` directly.
 *   counters  int32 [num_seqs * num_kv_heads], device memory, all zero on
 *             entry (e.g. cleared once after allocation); every completed call
 *             leaves them zero.  Calls that overlap in time must not share a
 *             counters buffer.
 * partition_size must be > 0 (a multiple of block_size).  Best when a
 * sequence has at most a few dozen partitions: the merge of one
 * (sequence, kv head) runs in a single workgroup.
 */
int paged_attn_decode_fused(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            int num_blocks, int max_blocks_per_seq, float scale,
                            int partition_size, void *out, float *max_logits, float *exp_sums,
                            float *tmp_out, int max_num_partitions, int32_t *counters,
                            void *stream);

/*
 * paged_attn_decode_fused without allocation, for callers that cannot call
 * hipMalloc or take a workspace from an allocator (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * computation, inputs, output (`out` for every sequence, zero rows for
 * zero-length sequences) and schedule as paged_attn_decode_fused with
 * max_num_partitions = paged_attn_num_partitions(max_blocks_per_seq,
 * block_size, partition_size); its workspace (partial records and arrival
 * counters) is instead a fixed 64 MiB device array inside the library, one
 * per GPU the library runs on, held until the process ends.  Limits: the
 * records, num_seqs * H_q * max_num_partitions * (D + 2) fp32 values in
 * 256-byte aligned sections, must fit in 64 MiB less 256 KiB of counters, and
 * num_seqs * H_kv <= 65536; beyond either the call returns
 * PA_ERR_SCRATCH_LIMIT without launching anything (a larger partition_size
 * needs fewer records).  The first call on a device takes the array's device
 * address and clears its counters (a fill kernel on `stream`); no call
 * allocates or frees memory.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and give wrong results; calls ordered on one stream are safe.
 * Errors: as paged_attn_decode_fused, plus PA_ERR_SCRATCH_LIMIT.
 */
int paged_attn_decode_fused_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *seq_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, int max_blocks_per_seq,
                                    float scale, int partition_size, void *out, void *stream);

/*
 * Paged GQA decode over an FP8 KV cache (the B200 page, "Stage D: FP8 Paged KV
 * Gather": FP8 codes gathered through the block table, a per-position dequant
 * scale applied after the gather).  Same computation, arguments, partials and
 * status codes as paged_attn_decode, with K and V taken as
 *   K[blk, h, slot, d] = e4m3(k_cache[blk, h, slot, d]) * k_scales[blk, h, slot]
 * (and V likewise), where
 *   k_cache, v_cache   uint8 [num_blocks, H_kv, block_size, D]  OCP FP8 E4M3
 *                      codes ("e4m3fn": bias 7, no infinities, 0x7F/0xFF NaN)
 *   k_scales, v_scales fp32  [num_blocks, H_kv, block_size]     dequant scales
 * as paged_attn_kv_append_fp8 writes them.  Slots past a sequence's length may
 * hold anything (NaN included); they are never used.  Partials merge with
 * paged_attn_decode_reduce.  k_cache, v_cache, k_scales and v_scales must be
 * 16-byte aligned.
 */
int paged_attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                          const float *k_scales, const float *v_scales,
                          const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, int max_blocks_per_seq, float scale, int partition_size,
                          void *out, float *max_logits, float *exp_sums, float *tmp_out,
                          int max_num_partitions, void *stream);

/*
 * Paged GQA decode over the BI-V100 page's cache layouts (section 3 "Paged
 * K/V Gather"): x-packed K and transposed V, bf16, x = 16 bytes / 2 = 8:
 *   k_cache  bf16 [num_blocks, H_kv, D / 8, block_size, 8]
 *   v_cache  bf16 [num_blocks, H_kv, D, block_size]
 * Element (block, h, slot, d) of K is k_cache[block, h, d / 8, slot, d % 8]
 * and of V is v_cache[block, h, d, slot].  Same computation, other arguments,
 * partials, merge and status codes as paged_attn_decode.
 */
int paged_attn_decode_xpacked(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq, float scale,
                              int partition_size, void *out, float *max_logits, float *exp_sums,
                              float *tmp_out, int max_num_partitions, void *stream);

/*
 * Paged GQA decode over a token-granular cache (the AstrAI page, "Attention
 * Backend" and "Q Scheduling and KV Addressing": decode with page_size=1,
 * kv_indptr giving each request's KV length, page indices translating logical
 * positions to physical slots):
 *   k_cache, v_cache  bf16 [num_slots, H_kv, D]
 *   kv_indptr         int32 [num_seqs + 1], non-decreasing; sequence s has
 *                     L = kv_indptr[s+1] - kv_indptr[s] tokens
 *   kv_indices        int32 [kv_indptr[num_seqs]]; token t of sequence s is
 *                     slot kv_indices[kv_indptr[s] + t]
 * Same computation, outputs, partials and status codes as paged_attn_decode.
 * max_kv_len (host) must be >= every L: it sizes the launch, and with
 * partition_size > 0 max_num_partitions must be >= ceil(max_kv_len / P)
 * rounded up to whole 16-token tiles, i.e. paged_attn_num_partitions(
 * ceil(max_kv_len / 16), 16, P).  Merge the partials with
 * paged_attn_decode_reduce_indptr.  Slot ids and offsets are device values,
 * not checked.
 */
int paged_attn_decode_tokens(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *kv_indptr, const int32_t *kv_indices, int num_seqs,
                             int num_q_heads, int num_kv_heads, int head_dim, int num_slots,
                             int max_kv_len, float scale, int partition_size, void *out,
                             float *max_logits, float *exp_sums, float *tmp_out,
                             int max_num_partitions, void *stream);

/* paged_attn_decode_reduce with each sequence's length taken from adjacent
 * kv_indptr entries (for the partials of paged_attn_decode_tokens). */
int paged_attn_decode_reduce_indptr(const float *max_logits, const float *exp_sums,
                                    const float *tmp_out, const int32_t *kv_indptr, int num_seqs,
                                    int num_q_heads, int head_dim, int partition_size,
                                    int max_num_partitions, void *out, void *stream);

/*
 * KV append: writes the K/V rows of new tokens into their cache slots -- the
 * cache write before decode and prefill (the AstrAI page's backend layer "owns
 * KV cache writes and reads").  Sequence s owns rows [cu_seqlens[s],
 * cu_seqlens[s+1]) of k_new / v_new (bf16 [num_tokens, H_kv, D]); they are the
 * LAST n = cu[s+1] - cu[s] of its seq_lens[s] tokens (seq_lens already counts
 * them), so row j goes to position c + j, c = seq_lens[s] - n: block
 * block_tables[s, (c + j) / block_size], slot (c + j) % block_size -- where
 * paged_attn_prefill_ragged reads its rows; a decode step has n = 1.
 *   k_cache, v_cache  bf16 [num_blocks, H_kv, block_size, D], updated in place
 *                     (only the new rows' slots are written).
 * max_new_tokens must be >= every n (it sizes the launch) and num_tokens must
 * equal cu_seqlens[num_seqs]; seq_lens[s] >= n and valid block ids for the
 * written positions are required (device values, not checked).  Two rows
 * written to the same slot (a block shared by two sequences) race.
 * num_seqs == 0 or num_tokens == 0 is a no-op.  Status codes as for decode.
 */
int paged_attn_kv_append(const void *k_new, const void *v_new, const int32_t *block_tables,
                         const int32_t *seq_lens, const int32_t *cu_seqlens, int num_seqs,
                         int num_tokens, int max_new_tokens, int num_kv_heads, int head_dim,
                         int block_size, int num_blocks, int max_blocks_per_seq, void *k_cache,
                         void *v_cache, void *stream);

/*
 * KV append into the x-packed K / transposed V layouts of
 * paged_attn_decode_xpacked: the same rows, placement, arguments and status
 * codes as paged_attn_kv_append.
 */
int paged_attn_kv_append_xpacked(const void *k_new, const void *v_new, const int32_t *block_tables,
                                 const int32_t *seq_lens, const int32_t *cu_seqlens, int num_seqs,
                                 int num_tokens, int max_new_tokens, int num_kv_heads, int head_dim,
                                 int block_size, int num_blocks, int max_blocks_per_seq,
                                 void *k_cache, void *v_cache, void *stream);

/*
 * KV append into an FP8 cache (the B200 page, "FP8 KV Quantize/Dequant", with
 * its per-position dequant scale): the same rows and placement as
 * paged_attn_kv_append, each (token, kv head) row of K and of V quantized on
 * its own:
 *   amax = max_d |x_d|,  scale = amax / 448  (fp32, correctly rounded),
 *   code_d = sign(x_d) | the E4M3 magnitude nearest to |x_d| / scale (fp32,
 *            correctly rounded), ties to the even code, saturating at 448;
 * a row of zeros gets scale 0 and zero codes.  Writes the codes to
 * k_cache / v_cache (uint8 [num_blocks, H_kv, block_size, D]) and the scales
 * to k_scales / v_scales (fp32 [num_blocks, H_kv, block_size]); dequantized
 * value = e4m3(code) * scale.  All four must be 16-byte aligned.
 */
int paged_attn_kv_append_fp8(const void *k_new, const void *v_new, const int32_t *block_tables,
                             const int32_t *seq_lens, const int32_t *cu_seqlens, int num_seqs,
                             int num_tokens, int max_new_tokens, int num_kv_heads, int head_dim,
                             int block_size, int num_blocks, int max_blocks_per_seq,
                             void *k_cache, void *v_cache, float *k_scales, float *v_scales,
                             void *stream);

/*
 * Ragged paged prefill with a causal mask.  Sequence s owns query rows
 * [cu_seqlens[s], cu_seqlens[s+1]) of q / out ([total_q, H_q, D]); its
 * n = cu[s+1] - cu[s] new tokens are the LAST n of its seq_lens[s] tokens,
 * whose K/V are already in the cache.  Row j (absolute position c + j,
 * c = seq_lens[s] - n) attends to keys t <= c + j (AstrAI page, "Q Scheduling
 * and KV Addressing"; causal rule of the RL.cu page's prefill kernel, aligned
 * to the end of the context).  max_q_len must be >= every n (it sizes the
 * launch); total_q must equal cu_seqlens[num_seqs].  Requires
 * seq_lens[s] >= n for every s.
 */
int paged_attn_prefill_ragged(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *seq_lens,
                              const int32_t *cu_seqlens, int num_seqs, int total_q,
                              int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, int max_blocks_per_seq,
                              float scale, void *out, void *stream);

/*
 * Ragged paged prefill, split-KV form: the same inputs, rows and output as
 * paged_attn_prefill_ragged, computed by cutting every (query tile, kv head)
 * into key chunks of kv_chunk tokens (the BI-V100 design page's partitioning,
 * section 2 "Level 3", applied to prefill) so that long contexts spread over
 * the whole GPU.  A persistent grid takes the chunks from a device counter;
 * rows whose keys all lie in the first chunk are written directly, the others
 * leave one fp32 partial record (running max, exp-sum, normalized output) per
 * chunk, merged by a second kernel with the page's combine rule.
 *   kv_chunk   0 = paged_attn_prefill_chunk_size(...); else a positive
 *              multiple of 64, at most 8192.
 *   workspace  device memory, 16-byte aligned, of at least
 *              paged_attn_prefill_workspace_size(...) bytes for the chunk in
 *              use.  Its first 8 bytes are two counters that must be zero
 *              before the first call (clear the buffer once after
 *              allocation); every completed call leaves them zero.  Calls
 *              that overlap in time must not share a workspace.
 * When the chunk list does not fit (more than 1024 sequences or (sequence,
 * query tile) pairs, or more than 128 query heads) or one chunk covers the
 * longest context, the call runs
 * the single-pass kernel and does not touch the workspace (it may then be
 * NULL).  Same status codes as paged_attn_prefill_ragged, plus
 * PA_ERR_BAD_SHAPE for a bad kv_chunk or a workspace that is too small.
 */
int paged_attn_prefill_ragged_split(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *seq_lens,
                                    const int32_t *cu_seqlens, int num_seqs, int total_q,
                                    int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, int max_blocks_per_seq,
                                    float scale, int kv_chunk, void *workspace,
                                    long long workspace_bytes, void *out, void *stream);

/* ---- host-only helpers (no device work) ---------------------------------- */

/* Key chunk the split-KV prefill uses when kv_chunk == 0: about 2.6 chunks
 * per CU of the current device if every (sequence, query tile) pair had the
 * longest context, a multiple of 256 in [512, 8192]; 0 when the single pass
 * is used instead (too many pairs or query heads, or one chunk covers the
 * longest context).
 * The pair count is bounded by ceil(total_q / (256 / G)) + num_seqs. */
int paged_attn_prefill_chunk_size(int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
                                  int max_blocks_per_seq, int block_size);

/* Workspace bytes of paged_attn_prefill_ragged_split for a chunk of kv_chunk
 * tokens: 256 + 2 * R4 + R4 * head_dim, R4 = total_q * num_q_heads *
 * ceil(max_blocks_per_seq * block_size / kv_chunk) * 4 bytes, each section
 * rounded up to 256 bytes; -1 for invalid arguments. */
long long paged_attn_prefill_workspace_size(int total_q, int num_q_heads, int head_dim,
                                            int max_blocks_per_seq, int block_size, int kv_chunk);

/* Partition count covering max_blocks_per_seq * block_size tokens; 1 when
 * partition_size == 0; -1 on a bad argument. */
int paged_attn_num_partitions(int max_blocks_per_seq, int block_size, int partition_size);

/* A partition size for paged_attn_decode: 0 (single pass) when one workgroup
 * per (sequence, kv head) already fills the GPU several times over, otherwise
 * a power of two >= 256 chosen so that the partition count is large enough to
 * keep all compute units busy.  total_kv_tokens may be 0 (unknown). */
int paged_attn_choose_partition_size(int num_seqs, int num_kv_heads, int max_seq_len,
                                     long total_kv_tokens);

/* Q-tile work map of a packed ragged batch (AstrAI page, "Q Scheduling and KV
 * Addressing"): from HOST cu_seqlens, tile k covers rows
 * [tile_to_index[k] * tile_rows, ...) of sequence tile_to_batch[k].  Writes at
 * most `capacity` entries and returns the number of tiles (or -1 on a bad
 * argument); a return value above capacity means the arrays were too small. */
int paged_attn_prefill_tile_map(const int32_t *cu_seqlens_host, int num_seqs, int tile_rows,
                                int32_t *tile_to_batch, int32_t *tile_to_index, int capacity);

/*
 * HBM read-stream probe: a measurement helper beside the attention path, not
 * a step of it.  The AstrAI "CUDA Kernels" page ("Known Optimization
 * Targets") rates its decode by achieved against theoretical bandwidth; this
 * call measures the achievable read rate on the device at hand, so a decode
 * can also be rated against that.  It reads each of the `bytes` bytes at
 * `buf` once (16-byte nontemporal loads, grid-stride over num_workgroups
 * workgroups of 256 threads) and writes to partial[w] the XOR of the 32-bit
 * words that workgroup w read: the XOR over all num_workgroups entries equals
 * the XOR of every 32-bit word of the buffer.
 *   buf             device memory, 16-byte aligned, read only.
 *   bytes           a positive multiple of 16.
 *   partial         device memory, uint32 [num_workgroups], written only.
 *   num_workgroups  >= 1 (the grid; a few times 256 CUs x 8 fills the chip).
 * Errors: PA_ERR_NULL_POINTER, PA_ERR_BAD_SHAPE (bytes, num_workgroups),
 * PA_ERR_ALIGNMENT (buf), PA_ERR_LAUNCH.  Enqueued on `stream`; the caller
 * owns both buffers.
 */
int paged_attn_read_probe(const void *buf, long long bytes, uint32_t *partial, int num_workgroups,
                          void *stream);

/*
 * Paged-gather read probe: a measurement helper beside the attention path,
 * not a step of it.  It reads exactly the K/V bytes one paged_attn_decode
 * of the batch reads -- every (block, kv head) tile of every used logical
 * block of every sequence, tail slots included -- through block_tables, with
 * the decode's 16-byte nontemporal loads, and nothing else, so it measures
 * the rate at which a paged cache can be gathered (the BI-V100 page, section
 * 3 "Paged K/V Gather", counts the gather's memory accesses; this times
 * them).  A piece is two 16 * head_dim * 2-byte tiles read by one wave,
 * two pieces in flight:
 *   whole_blocks 0: the K tile and the V tile of one (sequence, kv head,
 *                   block), pieces in (sequence, kv head, block) order -- the
 *                   decode's own walk over scattered tiles;
 *   whole_blocks 1: consecutive tile pairs of [K block | V block] of one
 *                   (sequence, block) -- each block's contiguous
 *                   H_kv * 16 * head_dim K and V rows read together;
 *   whole_blocks 2: the pieces of mode 0 read with load-to-LDS instructions
 *                   into a per-wave ring of two pieces in LDS and folded
 *                   from there -- the gather a direct-to-LDS tile ring sees.
 * All modes read the same bytes.  The grid's waves split the pieces into
 * equal consecutive runs.  partial[w] receives the XOR of the 32-bit words
 * workgroup w read; the XOR over all entries equals the XOR of every 32-bit
 * word of the K and V tiles of the used blocks (a block used twice cancels).
 *   k_cache, v_cache  bf16 [num_blocks, H_kv, block_size, head_dim], device,
 *                     16-byte aligned, read only.
 *   block_tables      int32 [num_seqs, max_blocks_per_seq], device.
 *   block_prefix      int32 [num_seqs + 1], device: block_prefix[0] = 0 and
 *                     block_prefix[s + 1] - block_prefix[s] = ceil(L_s / 16).
 *   partial           uint32 [num_workgroups], device, written only.
 * Limits: num_seqs <= 1024, head_dim in {64, 128, 256}, block_size 16.
 * Errors: PA_ERR_NULL_POINTER, PA_ERR_BAD_SHAPE (including whole_blocks
 * outside 0..2), PA_ERR_UNSUPPORTED, PA_ERR_ALIGNMENT, PA_ERR_LAUNCH.
 * Enqueued on `stream`.
 */
int paged_attn_gather_probe(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                            const int32_t *block_prefix, int num_seqs, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, int whole_blocks, uint32_t *partial,
                            int num_workgroups, void *stream);

/* Human-readable name of a status code. */
const char *paged_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
