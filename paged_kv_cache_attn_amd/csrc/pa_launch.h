// pa_launch.h -- host-side launchers of the gfx950 kernels (internal to
// libpagedattn; the public C ABI is include/paged_attn.h).  Arguments are
// assumed validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Waves per decode workgroup (they split each segment's blocks round-robin).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif

namespace pa {

// Block sizes the MFMA kernels take (they walk rows in 16-token tiles; a
// tile is a whole block, part of one, or two blocks of 8).
inline bool mfma_block_size(int bs) { return bs == 8 || bs == 16 || bs == 32 || bs == 64 || bs == 128; }

// Balanced (stream-K) decode: largest batch whose per-sequence prefix fits the
// workgroup's LDS, and the number of ranges the library picks by default.
constexpr int kStreamKMaxSeqs = 2048;
#ifndef PA_STREAMK_RANGES
#define PA_STREAMK_RANGES 512
#endif
constexpr int kStreamKRanges = PA_STREAMK_RANGES;
// Largest range (in blocks) a balanced-decode workgroup stages in LDS.
constexpr int kStreamKTabCache = 1024;

hipError_t launch_kv_cache_write(const void *key, const void *value, void *k_cache, void *v_cache,
                                 const int64_t *slot_mapping, int num_tokens, int num_blocks,
                                 int num_kv_heads, int block_size, int head_dim, int elem_bytes,
                                 hipStream_t stream);
// Quantising write into FP8 E4M3 caches; src_bf16: key/value are bf16 (else fp32).
hipError_t launch_kv_cache_write_fp8(const void *key, const void *value, int src_bf16, void *k_cache,
                                     void *v_cache, const int64_t *slot_mapping, int num_tokens,
                                     int num_blocks, int num_kv_heads, int block_size, int head_dim,
                                     float k_scale, float v_scale, hipStream_t stream);

// gather (true): ids[0..n) of the K and V caches -> staging [n][2][block];
// scatter (false): the reverse.  block_chunks = 16-byte chunks per block.
hipError_t launch_swap_blocks(bool gather, void *k_cache, void *v_cache, const int64_t *ids, int n,
                              void *staging, int num_blocks, int block_chunks, hipStream_t stream);
hipError_t launch_block_copy(void *k_cache, void *v_cache, const int64_t *pairs, int num_pairs,
                             int num_blocks, int num_kv_heads, int block_size, int head_dim,
                             int elem_bytes, hipStream_t stream);

// Everything one decode launch needs.  Sizes are validated; pointers are device.
// Bit of a plan record's block count marking a tile whose block a neighbouring
// row also uses (its loads keep the tile in the L2).
constexpr int kKeepTile = 1 << 30;

struct DecodeParams {
  void *out;
  int out_bf16;            // 0: fp32 output, 1: bf16 output
  const void *q;           // [B][Hq][D]
  const void *k_cache;     // [NB][Hkv][bs][D]
  const void *v_cache;
  int kv_bf16;             // 0: fp32 KV, 1: bf16 KV (q has the KV dtype)
  int kv_fp8;              // 1: FP8 E4M3 KV codes with bf16 q (kv_bf16 is then 0)
  float k_scale, v_scale;  // FP8: K = value(code) * k_scale, V likewise; 1 otherwise
  const int32_t *block_tables;
  int max_blocks_per_seq;
  const int32_t *seq_lens;
  int num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks;
  int max_len_cap;         // min(max_seq_len, max_blocks_per_seq * block_size)
  float scale;
  int head_split;          // balanced path: hs >= 1 sub-groups per GQA group, each g / hs heads,
                           //   each its own row; the rows of sequence b are those of b * hs .. + hs - 1
  int tile_tokens;         // tokens per unit of part_blocks / the flat space: 16 on the MFMA
                           // path (16-token tiles), block_size on the vector path
  int part_blocks;         // units per split-K partition
  int nparts_max;          // ceil(ceil(max_len_cap / bs) / part_blocks), >= 1
  float *ws_o;             // [B][Hq][nparts_max][D]   (unused when nparts_max == 1)
  float *ws_ml;            // [B][Hq][nparts_max][2]   (max in log2 units, sum)
  // balanced (stream-K) path
  int sk_ranges;           // workgroups = ranges of the flat block space
  int sk_range_blocks;     // 0: T / sk_ranges blocks each (balanced); > 0: fixed
  float *sk_part;          // [ranges][2][g][D] partial outputs
  float *sk_ml;            // [ranges][2][g][2] partial (max, sum)
  int4 *sk_desc;           // [ranges] the split row under the range's first position
                           //   (workspace; for a planned call, the plan's copy):
                           // {row or -1, its first range, slot of its first piece, its last range}
  // a decode plan (balanced path; nullptr: each launch stages its own range)
  int4 *plan_hdr;          // [ranges] {range start, range end, total blocks T, ranges used G}
  int4 *plan_rec;          // [ranges][plan_stride] {tile row 0 / 1024, tile row 8 / 1024, row, j}
  int2 *plan_rec2;         // [ranges][plan_stride] {sequence length, blocks of the row
                           //   | kKeepTile if a neighbouring row uses the tile's block}
  int plan_stride;         // positions per range in the plan (>= every range's size)
  // the step's write folded into a planned bf16 call (nullptr: none)
  const void *new_k;       // [B][Hkv][D] bf16: the new token's K row of every sequence
  const void *new_v;       // [B][Hkv][D]
  const int64_t *slot_mapping;  // [B]: its slot (< 0: none)
};

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_streamk(const DecodeParams &p, hipStream_t stream);
// Writes the plan of p's balanced split (p.plan_* set, the attention fields unused).
hipError_t launch_decode_streamk_plan(const DecodeParams &p, hipStream_t stream);

struct PrefillParams {
  void *out;
  int out_bf16;
  const void *q;           // [Tq][Hq][D]
  const void *k_cache;
  const void *v_cache;
  int kv_bf16;
  int kv_fp8;              // as in DecodeParams
  float k_scale, v_scale;
  const int32_t *block_tables;
  int max_blocks_per_seq;
  const int32_t *query_start_loc;  // [B+1]
  const int32_t *seq_lens;         // [B]
  int num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks;
  int max_query_len;
  int num_query_tokens;    // rows of q / out; rows at or beyond are never touched
  int max_len_cap;
  float scale;
  int head_split;          // MFMA kernels: hs sub-groups per GQA group, each g / hs heads (a
                           //   divisor of 16) served as if by a KV head of its own
};

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream);

#ifndef PAGED_ATTN_DEBUG
#define PAGED_ATTN_DEBUG 0
#endif
#if PAGED_ATTN_DEBUG
// Device addresses of the debug flag words of the four kernel files (debug
// build only; see pa_device.h).
hipError_t debug_word_ops(void **p);
hipError_t debug_word_decode(void **p);
hipError_t debug_word_streamk(void **p);
hipError_t debug_word_prefill(void **p);
#endif

#ifndef PAGED_ATTN_TIMELINE
#define PAGED_ATTN_TIMELINE 0
#endif
#if PAGED_ATTN_TIMELINE
// Device addresses of the balanced decode's timestamp arrays (timestamp build
// only): [PA_TIMELINE_ROWS][8] for the main kernel, [PA_TIMELINE_ROWS][2] for
// the merge kernel, uint64 each.
hipError_t timeline_symbols(void **main_stamps, void **merge_stamps);
#endif

}  // namespace pa
