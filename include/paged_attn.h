/*
 * paged_attn.h -- C ABI of libpagedattn.so, PagedAttention for AMD MI355X (gfx950).
 *
 * Attention for decode and chunked-prefill queries over a KV cache kept in
 * fixed-size physical blocks that each sequence reaches through its own
 * block table, plus the memory kernels that go with it: writing new K/V
 * rows into their slots, copying whole blocks for copy-on-write, and
 * swapping blocks between HBM and host memory.
 *
 * Sources (web pages on KV-cache management; sections named as on the page):
 *   [L7]  Lecture 7 "KV Cache Management: PagedAttention and Mooncake"
 *         (Stanford CS349E notes): §4.1 blocks and block table, §4.2
 *         blockwise attention, §4.3 the three fused kernels, §5.1 fork and
 *         copy-on-write.
 *   [M2]  Month 2 "PagedAttention" (infra learning path, memory chapter):
 *         §2.1 attention with a KV cache, §5.2 the per-layer block pool,
 *         §5.4 the kernel loop over logical blocks with online softmax.
 *   [L16] Lecture 16 "LLM Serving (1): Batching, PagedAttention,
 *         RadixAttention" (CMU 15-779 notes): §3.3 block table and
 *         blockwise attention merged by the online-softmax rule, §3.5
 *         sharing and copy-on-write.
 *   [L27] Lecture 27 "Better KV Caches: CacheGen, CacheBlend and LMCache"
 *         (CMU 11-868 notes): §1.1 new tokens' queries attend directly to
 *         cached K/V.
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers unless stated otherwise; the
 *     caller owns every buffer (the library never allocates, frees or
 *     synchronises).  Arrays are dense, row-major, in the layouts given,
 *     16-byte aligned, and do not alias one another.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; results are ready when the stream
 *     reaches that point.
 *   - dtype codes: PA_F32 (IEEE fp32) or PA_BF16 (bfloat16).  q, K and V
 *     share one dtype; accumulation is always fp32.  PA_FP8_E4M3 (8-bit
 *     codes, see the _fp8 calls) is a KV-cache storage format: the byte-moving
 *     calls (kv_cache_write as a plain copy, block_copy, the swaps) take it
 *     like any other dtype.
 *   - KV cache layout, one layer: [num_blocks][num_kv_heads][block_size][head_dim],
 *     K and V in separate arrays ([M2] §5.2; head-major inside a block so one
 *     (block, head) tile is contiguous).
 *   - Query head h reads KV head h / (num_heads / num_kv_heads) (contiguous
 *     GQA groups).
 *   - Return value: PA_OK, or a negative PA_ERR_* code.  Argument checks run
 *     on the host before anything is enqueued; a failed check enqueues
 *     nothing.  PA_ERR_LAUNCH reports a HIP launch error.  No exception
 *     crosses the ABI.  Calls are stateless and thread-safe.
 *   - Device-side contents (slots, block ids) are bounds-checked by the
 *     kernels: an out-of-range slot or pair is skipped and an out-of-range
 *     block-table entry is not dereferenced (its tokens contribute nothing),
 *     so bad ids never fault the GPU, but the result for that sequence is then
 *     unspecified.
 *   - The swap calls also take one HOST pointer (stated where it appears).
 *   - Supported shapes.  Attention calls: head_dim in {64, 128}, any
 *     block_size >= 1, num_heads % num_kv_heads == 0 (the MFMA kernels serve
 *     bf16 KV with head_dim 128 and block_size in {8, 16, 32, 64, 128},
 *     walking each sequence in 16-token tiles: prefill with any GQA group
 *     (as sub-groups whose size divides 16), decode with a group of at most
 *     16, or a larger one as sub-groups of at most 16 heads when its
 *     balanced split takes the call (num_seqs times the sub-group count at
 *     most 2048, and not a caller's partition_size of more than 16 pieces
 *     per row); other supported shapes run on plain vector kernels),
 *     one physical block of num_kv_heads * block_size * head_dim elements
 *     below 2^31 and a whole cache (num_blocks such blocks) below 2^41.
 *     kv_cache_write, block_copy and the swap calls: any block_size >= 1 and any head_dim whose row is a
 *     multiple of 16 bytes.  Anything else returns PA_ERR_UNSUPPORTED.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define PA_EXPORT __attribute__((visibility("default")))
#else
#define PA_EXPORT
#endif

enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 };

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  PA_ERR_SHAPE = -2,       /* negative or inconsistent sizes                    */
  PA_ERR_UNSUPPORTED = -3, /* valid but not implemented (head_dim, block size)  */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required        */
  PA_ERR_LAUNCH = -5,      /* HIP reported an error when launching              */
  PA_ERR_SCRATCH = -6      /* needs more than the built-in scratch buffer holds */
};

/* Static, NUL-terminated description of a status code (host). */
PA_EXPORT const char *pa_status_string(int status);

/* PA_ABI_VERSION of the built library (host). */
PA_EXPORT int pa_abi_version(void);

/*
 * pa_debug_flags -- what the kernels' bounds checks have masked since the
 * last clear (host; the debug build libpagedattn_debug.so only).  In every
 * build the kernels skip or mask out-of-range device-side ids without
 * dereferencing them; the debug build also records each kind it meets as a
 * bit of a per-device flag word, and checks two caller contracts the release
 * build trusts (no duplicate slots in one kv_cache_write, no conflicting
 * pairs in one block_copy).  Waits for the current device to finish
 * (hipDeviceSynchronize), stores the OR of the flags in *flags and clears
 * them if `clear` is nonzero.  The release build stores 0 and returns
 * PA_ERR_UNSUPPORTED.
 */
#define PA_DEBUG_SLOT_RANGE (1u << 0)     /* slot >= num_blocks * block_size (skipped)         */
#define PA_DEBUG_SLOT_DUP (1u << 1)       /* two tokens of one kv_cache_write share a slot      */
#define PA_DEBUG_BLOCK_RANGE (1u << 2)    /* block-table entry outside [0, num_blocks) (masked) */
#define PA_DEBUG_PAIR_RANGE (1u << 3)     /* block_copy id outside [0, num_blocks) (skipped)    */
#define PA_DEBUG_PAIR_CONFLICT (1u << 4)  /* a dst twice, or a dst that is another pair's src   */
#define PA_DEBUG_LEN_CLAMPED (1u << 5)    /* seq_lens < 0 or past the call's bound (clamped)    */
#define PA_DEBUG_QUERY_LOC (1u << 6)      /* query_start_loc not a partition of the query rows  */
#define PA_DEBUG_SWAP_RANGE (1u << 7)     /* swap id outside [0, num_blocks)                    */
#define PA_DEBUG_PLAN (1u << 8)           /* plan record outside the call's cache or rows       */
PA_EXPORT int pa_debug_flags(unsigned *flags, int clear);

/*
 * pa_timeline -- per-workgroup timestamps of the balanced decode's planned
 * kernels (host; the timestamp build libpagedattn_timeline.so only), for
 * breaking one call's time into its phases.  Each workgroup of the main
 * kernel records, by its hardware workgroup id, the s_memrealtime clock
 * (100 MHz; every XCD has its own, offset from the others, so only stamps
 * taken on one XCD compare) at 8 points:
 *   [0] start, [1] its range's plan records staged, [2..5] the stream end
 *   of waves 0..3, [6] the combine's start (after the barrier), [7] the end;
 * each merge-kernel workgroup records [0] start and [1] end.  A point a
 * workgroup does not reach stays 0.  Later calls overwrite earlier stamps.
 *
 *   main_stamps   host [rows][8] uint64 (written)
 *   merge_stamps  host [rows][2] uint64 (written)
 *   rows          workgroup ids 0 .. rows - 1 to copy, 1 <= rows <= PA_TIMELINE_ROWS
 * Waits for the current device to finish (hipDeviceSynchronize), copies the
 * stamps and sets them all to zero if `clear` is nonzero.  The release
 * build returns PA_ERR_UNSUPPORTED.
 */
#define PA_TIMELINE_ROWS 4096
PA_EXPORT int pa_timeline(uint64_t *main_stamps, uint64_t *merge_stamps, int32_t rows, int32_t clear);

/*
 * kv_cache_write -- scatter new K/V rows into their cache slots
 * ([L7] §4.3 first fused kernel; [L7] §4.1 and [L16] §3.3: a token lands in
 * the next free slot of its sequence's last block).
 *
 *   key, value    [num_tokens][num_kv_heads][head_dim], dtype
 *   k_cache, v_cache  [num_blocks][num_kv_heads][block_size][head_dim], dtype (written)
 *   slot_mapping  [num_tokens] int64: slot = block * block_size + offset;
 *                 slot < 0 skips the token (padding); slot >= num_blocks*block_size
 *                 is out of range and skipped.
 * For every token t with a valid slot s and every KV head h:
 *   K[s / bs][h][s % bs][:] = key[t][h][:];  V likewise.
 * A bit-exact copy.  Two tokens with the same slot in one call: which one
 * wins is unspecified.  num_tokens == 0 is a no-op.
 */
PA_EXPORT int kv_cache_write(const void *key, const void *value, void *k_cache, void *v_cache,
                   const int64_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                   int32_t num_kv_heads, int32_t block_size, int32_t head_dim, int32_t dtype,
                   void *stream);

/*
 * paged_attn_decode_workspace_size -- bytes of device workspace that
 * paged_attn_decode needs for these sizes (host, pure function; an upper
 * bound over the kernels the call may pick).  partition_size as in
 * paged_attn_decode.  0 means no workspace is needed.  Returns 0 for invalid
 * sizes as well.
 */
PA_EXPORT size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                                  int32_t num_kv_heads, int32_t head_dim,
                                                  int32_t block_size, int32_t max_seq_len,
                                                  int32_t partition_size);

/*
 * paged_attn_decode -- one query token per sequence attends to all of its
 * cached tokens through the block table ([M2] §2.1 and §5.4; [L7] §4.2).
 *
 *   out           [num_seqs][num_heads][head_dim], out_dtype (PA_F32 or PA_BF16,
 *                 rounded to nearest even once at the end)
 *   q             [num_seqs][num_heads][head_dim], kv_dtype
 *   k_cache, v_cache  [num_blocks][num_kv_heads][block_size][head_dim], kv_dtype
 *   block_tables  [num_seqs][max_blocks_per_seq] int32: logical block j of
 *                 sequence b lives in physical block block_tables[b][j]; only
 *                 the first ceil(seq_lens[b] / block_size) entries are read.
 *   seq_lens      [num_seqs] int32: tokens in the cache for each sequence,
 *                 the current token included (its K/V are written first).
 *                 Must be <= max_seq_len and <= max_blocks_per_seq*block_size;
 *                 larger values are clamped to those bounds.  0 gives a zero row.
 *   max_seq_len   host-side upper bound of seq_lens (sizes the launch grid).
 *   scale         multiplies q.k (normally 1/sqrt(head_dim)); finite and > 0,
 *                 else PA_ERR_SHAPE.
 *   partition_size  split-K granularity in tokens, a multiple of block_size,
 *                 or 0 for the library's choice.  The KV blocks of all
 *                 (sequence, KV head) rows are split into contiguous pieces of
 *                 this many tokens (0: as many equal pieces as keep the GPU
 *                 busy); each piece of a row is reduced to (max, sum of
 *                 exponentials, unnormalised output) and the pieces are merged
 *                 by the online-softmax rule ([L16] §3.3) in a fixed order, so
 *                 results are bit-identical for any physical block permutation
 *                 and agree to rounding for any partition_size.  On the
 *                 MFMA kernels a piece is a whole number of 16-token tiles:
 *                 partition_size is rounded down to one (at least one tile).
 *   workspace     device scratch of at least
 *                 paged_attn_decode_workspace_size(...) bytes (may be NULL when
 *                 that size is 0).  Contents on entry are ignored.  Two calls
 *                 that may run at the same time need separate workspaces.
 * out[b][h] = sum_t softmax_t(scale * q[b][h] . K_t) V_t over the
 * seq_lens[b] tokens of KV head h / (num_heads / num_kv_heads).
 */
PA_EXPORT int paged_attn_decode(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                      const void *v_cache, int32_t kv_dtype, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * paged_attn_prefill_chunk -- causal attention of a chunk of new query
 * tokens per sequence over the cached prefix plus the chunk itself
 * ([L27] §1.1: the new tokens' queries attend to the cached K/V directly;
 * the chunk's own K/V must already be in the cache, e.g. via kv_cache_write).
 *
 *   out           [num_query_tokens][num_heads][head_dim], out_dtype
 *   q             [num_query_tokens][num_heads][head_dim], kv_dtype
 *   query_start_loc [num_seqs + 1] int32, non-decreasing, query_start_loc[0] == 0:
 *                 sequence b owns query rows query_start_loc[b] ..
 *                 query_start_loc[b+1]-1 (n_b rows, n_b <= seq_lens[b]).
 *   num_query_tokens  rows of q and out; rows at or beyond it are never read
 *                 or written, whatever query_start_loc says.
 *   seq_lens      [num_seqs] int32: tokens in the cache after the chunk.
 *   max_query_len host-side upper bound of n_b (rows beyond it are not
 *                 computed); max_seq_len bounds seq_lens.  scale as in
 *                 paged_attn_decode.
 * Row i of sequence b sits at position seq_lens[b] - n_b + i and attends to
 * tokens 0 .. that position (inclusive).  The prefix need not end on a block
 * boundary.
 * Precision (bf16 caches, head_dim 128): the softmax weights enter the PV
 * product rounded once to fp16 and V is widened to fp16, so V entries must
 * not exceed 65504 in magnitude (larger ones overflow to infinity); the
 * rounding moves an output by at most 2^-11 * max |v| over its keys.
 */
PA_EXPORT int paged_attn_prefill_chunk(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                             const void *v_cache, int32_t kv_dtype, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *query_start_loc,
                             const int32_t *seq_lens, int32_t num_seqs, int32_t num_query_tokens,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_query_len,
                             int32_t max_seq_len, float scale, void *stream);

/*
 * FP8 KV cache ([L7] §10: storing KV in 8 bits shrinks its memory and the
 * bandwidth attention needs by the bit count; the pages fix neither format
 * nor scaling, so this library's convention is):
 *   - codes are E4M3 as in the OCP 8-bit floating-point formats: sign, 4
 *     exponent bits (bias 7), 3 mantissa bits, subnormals, no infinities,
 *     S.1111.111 = NaN, largest magnitude 448;
 *   - one fp32 scale per tensor: K = value(code) * k_scale and
 *     V = value(code) * v_scale (scales finite and > 0, else PA_ERR_SHAPE);
 *   - attention reads bf16 q and computes exactly as on a bf16 cache holding
 *     value(code) (every E4M3 value is a bf16 value), with k_scale folded into
 *     the score scale and v_scale into the final normalisation;
 *   - the FP8 attention calls serve head_dim 128, block_size in
 *     {8, 16, 32, 64, 128} and the GQA groups of the MFMA kernels above
 *     (prefill: any; decode: at most 16, or larger where it takes the
 *     balanced split); other shapes return PA_ERR_UNSUPPORTED.
 *
 * kv_cache_write_fp8 -- kv_cache_write into FP8 caches: key and value rows
 * ([num_tokens][num_kv_heads][head_dim], src_dtype PA_F32 or PA_BF16) are
 * quantised on the way: element x of a key row becomes the code nearest to
 * the fp32 quotient x / k_scale (IEEE division, round to nearest), ties to
 * the even code, magnitudes beyond 448 saturated to 448 (values likewise
 * with v_scale); a NaN element gives an unspecified code.  Caches
 * [num_blocks][num_kv_heads][block_size][head_dim] bytes.  head_dim must be
 * a multiple of 16 (else PA_ERR_UNSUPPORTED).  Slots as in kv_cache_write.
 */
PA_EXPORT int kv_cache_write_fp8(const void *key, const void *value, int32_t src_dtype, void *k_cache,
                                 void *v_cache, const int64_t *slot_mapping, int32_t num_tokens,
                                 int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                                 int32_t head_dim, float k_scale, float v_scale, void *stream);

/*
 * Decode plans.  Which blocks each part of the balanced split reads depends
 * only on seq_lens, the block tables and the sizes, not on the layer, so a
 * plan computed once per decode step serves the attention of every layer
 * (all layers of a step share the block tables; [L7] §4.5).  A planned
 * decode starts streaming K/V after one memory round trip instead of
 * computing its part of the split from seq_lens and the tables first.
 *
 * paged_attn_decode_plan_size -- bytes of the plan buffer for these sizes
 * (host, pure function).  0: this shape is not split by the balanced path
 * and needs no plan (the planned call then behaves as the plain one).
 */
PA_EXPORT size_t paged_attn_decode_plan_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                             int32_t max_seq_len, int32_t partition_size, int32_t kv_dtype);

/*
 * paged_attn_decode_plan -- enqueue the computation of a plan into `plan`
 * (DEVICE, plan_bytes >= paged_attn_decode_plan_size(...), else
 * PA_ERR_WORKSPACE) from block_tables and seq_lens, as paged_attn_decode
 * would read them.  Nothing else is read or written.  A no-op when the size
 * is 0.
 */
PA_EXPORT int paged_attn_decode_plan(void *plan, size_t plan_bytes, int32_t kv_dtype,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, int32_t max_seq_len, int32_t partition_size,
                                     void *stream);

/*
 * paged_attn_decode_planned -- paged_attn_decode (kv_dtype PA_F32 / PA_BF16)
 * or paged_attn_decode_fp8 (kv_dtype PA_FP8_E4M3; k_scale and v_scale are
 * ignored otherwise) reading its split from `plan`.  The plan must have been
 * made by paged_attn_decode_plan with the same kv_dtype, sizes,
 * max_blocks_per_seq, max_seq_len and partition_size, from block_tables and
 * seq_lens whose contents have not changed since (the call still reads
 * seq_lens, for sequences with no tokens); otherwise the result is
 * unspecified.  Results are bit-identical to the unplanned call.
 */
PA_EXPORT int paged_attn_decode_planned(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                                        const void *v_cache, int32_t kv_dtype, float k_scale, float v_scale,
                                        const void *plan, size_t plan_bytes, const int32_t *block_tables,
                                        int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                        int32_t partition_size, void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * paged_attn_decode_append -- one layer of a decode step: every sequence's
 * new token is written into its slot and the sequence's query then attends
 * to its cache, new token included ([L7] §4.3: the KV write and the
 * attention through the block table are the fused kernels of the pages'
 * design; [L7] §4.1: a decode step appends one token to each sequence's last
 * block).  The result, output and caches, is bit for bit that of
 * kv_cache_write(key, value, slot_mapping) followed by
 * paged_attn_decode_planned with the same arguments, provided every
 * slot_mapping[b] is negative (no write) or the slot that the block table
 * gives position seq_lens[b] - 1 of sequence b (the append itself), and no
 * other sequence's first seq_lens tokens use that slot (a shared last block
 * is copied before it is written, [L7] §5.1).  Otherwise the output is
 * unspecified (the caches are still written as kv_cache_write would).
 *
 *   key, value    [num_seqs][num_kv_heads][head_dim]: the new token's K and V
 *                 rows; bf16 for PA_BF16 and PA_FP8_E4M3 caches (quantised
 *                 as kv_cache_write_fp8 does), fp32 for PA_F32 caches.
 *   slot_mapping  [num_seqs] int64: the new token's slot (< 0: none).
 *   k_cache, v_cache  written.  All other arguments, the plan, the workspace
 *                 and the guarantees as in paged_attn_decode_planned.
 * On the balanced split with a bf16 cache the write costs no launch of its
 * own: the attention kernel reads the new rows in place of position
 * seq_lens[b] - 1 and the split-merge kernel, after every read, stores them.
 * Other shapes run kv_cache_write(_fp8) and then the decode.
 */
PA_EXPORT int paged_attn_decode_append(void *out, int32_t out_dtype, const void *q, const void *key,
                                       const void *value, const int64_t *slot_mapping, void *k_cache,
                                       void *v_cache, int32_t kv_dtype, float k_scale, float v_scale,
                                       const void *plan, size_t plan_bytes, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                       int32_t partition_size, void *workspace, size_t workspace_bytes,
                                       void *stream);

/*
 * paged_attn_decode_fp8 -- paged_attn_decode over FP8 caches (q bf16
 * [num_seqs][num_heads][head_dim], out PA_F32 or PA_BF16).  All other
 * arguments, the workspace (paged_attn_decode_workspace_size covers it) and
 * the guarantees are those of paged_attn_decode.
 */
PA_EXPORT int paged_attn_decode_fp8(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                                    const void *v_cache, float k_scale, float v_scale,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t max_seq_len, float scale,
                                    int32_t partition_size, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same call, arguments (kv_dtype PA_F32 or
 * PA_BF16), kernels and results, bit for bit, but with no workspace
 * argument.  The workspace is a fixed device array inside the library,
 * PA_NOALLOC_SCRATCH_BYTES bytes, one copy on every GPU the library runs on,
 * held until the process ends.  The call itself allocates nothing and calls
 * no allocating routine; its first call on a device looks up the array's
 * device address there (once per device).
 *   - A call whose kernel needs more workspace than PA_NOALLOC_SCRATCH_BYTES
 *     returns PA_ERR_SCRATCH and enqueues nothing.  The need never exceeds
 *     paged_attn_decode_workspace_size(...) for the same sizes; the library's
 *     default split needs about 1 MB for 64 sequences of an 8-KV-head,
 *     128-dim layer and 4 MB for eight 32K-token sequences, and 512-token
 *     partitions of eight 32K-token, 64-head rows need about 17 MB.
 *   - Every call on one GPU shares that GPU's array: two calls that may run
 *     at the same time on one GPU (different streams, or different host
 *     threads) race and give unspecified results.  Calls ordered on one
 *     stream are safe.  Nothing in the array needs to start at zero; it
 *     keeps whatever the last call left.
 *   - The device is the stream's (the current device for the null stream).
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
PA_EXPORT int paged_attn_decode_noalloc(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                                        const void *v_cache, int32_t kv_dtype, const int32_t *block_tables,
                                        int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                                        int32_t partition_size, void *stream);

/*
 * paged_attn_prefill_chunk_fp8 -- paged_attn_prefill_chunk over FP8 caches
 * (q bf16 [num_query_tokens][num_heads][head_dim]); otherwise as
 * paged_attn_prefill_chunk.
 */
PA_EXPORT int paged_attn_prefill_chunk_fp8(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                                           const void *v_cache, float k_scale, float v_scale,
                                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *query_start_loc, const int32_t *seq_lens,
                                           int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_query_len, int32_t max_seq_len,
                                           float scale, void *stream);

/*
 * block_copy -- batched copy of whole physical blocks for copy-on-write
 * ([L7] §4.3 third fused kernel: the copies copy-on-write needs are gathered
 * and done in one launch; [L7] §5.1 and [L16] §3.5: a shared block is copied
 * before a sequence writes into it).
 *
 *   pairs  [num_pairs][2] int64 (src, dst): K[dst] = K[src] and V[dst] = V[src]
 *          over all num_kv_heads heads of the block.  Pairs with an id outside
 *          [0, num_blocks) are skipped; src == dst is a no-op.  A dst may not
 *          appear twice and no dst may be another pair's src in the same call
 *          (the copies run concurrently).
 * Bit-exact.  num_pairs == 0 is a no-op.
 */
PA_EXPORT int block_copy(void *k_cache, void *v_cache, const int64_t *pairs, int32_t num_pairs,
               int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
               int32_t dtype, void *stream);

/*
 * kv_swap_out -- copy whole physical blocks of one layer from the K and V
 * caches to host memory, for preemption by swapping ([L7] §6.2: a preempted
 * sequence group's blocks are copied to CPU memory and back, at the cost of
 * PCIe bandwidth plus a fixed cost per copy; [M2] §8.1: a 4K-token sequence
 * is swapped as one unit and the swap should run ahead, asynchronously).
 *
 *   block_ids  [num_ids] int64, DEVICE: the physical blocks to copy out, in
 *              the order they are packed.  An id outside [0, num_blocks)
 *              yields a zero-filled piece.
 *   host_dst   HOST memory of num_ids * 2 * block_bytes bytes, where
 *              block_bytes = num_kv_heads * block_size * head_dim * elem:
 *              piece i holds K[block_ids[i]] then V[block_ids[i]].  Pinned
 *              memory (hipHostMalloc) keeps the call asynchronous; pageable
 *              memory works but the copies then block the host.
 *   staging    DEVICE scratch of staging_bytes >= 2 * block_bytes (else
 *              PA_ERR_WORKSPACE).  The listed blocks are packed into it with
 *              one kernel per chunk of floor(staging_bytes / (2 * block_bytes))
 *              ids (at most 65535), and each chunk goes to the host with one
 *              DMA copy, so the per-copy cost is paid per chunk, not per
 *              block.  Contents on entry are ignored; two calls that may run
 *              at the same time need separate staging buffers.
 * Bit-exact.  num_ids == 0 is a no-op.  Host memory and the caches may be
 * reused once the stream has passed the call.
 */
PA_EXPORT int kv_swap_out(const void *k_cache, const void *v_cache, const int64_t *block_ids,
                          int32_t num_ids, void *host_dst, void *staging, size_t staging_bytes,
                          int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                          int32_t head_dim, int32_t dtype, void *stream);

/*
 * kv_swap_in -- the reverse of kv_swap_out: piece i of host_src (K then V,
 * as kv_swap_out packs them) is written to physical block block_ids[i] of
 * the K and V caches ([L7] §6.2: swapped-in blocks may land in any free
 * physical blocks; the block table is updated by the caller).  An id outside
 * [0, num_blocks) is skipped.  No id may appear twice.  Same staging rules.
 * Bit-exact.  num_ids == 0 is a no-op.
 */
PA_EXPORT int kv_swap_in(void *k_cache, void *v_cache, const int64_t *block_ids, int32_t num_ids,
                         const void *host_src, void *staging, size_t staging_bytes,
                         int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                         int32_t head_dim, int32_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
