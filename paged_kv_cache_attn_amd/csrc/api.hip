// api.hip -- the C ABI of libpagedattn (declared in include/paged_attn.h):
// host-side argument checks, kernel selection and launch.  Every check runs
// before anything is enqueued; a failed check returns its code and launches
// nothing.  No exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "paged_attn.h"
#include "pa_launch.h"

namespace {

constexpr int kDefaultPartitionTokens = 256;
constexpr int64_t kStreamKMaxPiecesPerRow = 16;  // a caller's fixed pieces per row on the balanced path
constexpr int kMaxGridYZ = 65535;

int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 1; }
// dtypes attention computes in (q, out, and the KV of the plain calls)
bool dtype_ok(int32_t dtype) { return dtype == PA_F32 || dtype == PA_BF16; }
// dtypes the byte-moving calls store
bool storage_dtype_ok(int32_t dtype) { return dtype_ok(dtype) || dtype == PA_FP8_E4M3; }
bool scale_ok(float s) { return s > 0.f && s <= 3.4e38f; }  // finite and positive (false for NaN)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// A GQA group of more than 16 query heads (one MFMA tile's columns) is served
// by the balanced decode as hs sub-groups of g / hs <= 16 heads, each its own
// row over the same K/V: hs is the smallest divisor of g that is at least
// ceil(g / 16).  1 for g <= 16.
int head_split(int g) {
  int hs = (g + 15) / 16;
  while (g % hs != 0) ++hs;
  return hs;
}

// Partition size (tokens) the decode call uses; 0 selects the default,
// rounded up to a whole number of blocks.
int64_t effective_partition(int32_t partition_size, int32_t block_size) {
  if (partition_size > 0) return partition_size;
  return ceil_div(kDefaultPartitionTokens, block_size) * block_size;
}

// The vector kernels' pieces when the caller leaves the size to the library:
// the longest power of two from 256 to 4096 tokens that still gives about
// 1,024 workgroups with keys (four per CU, over two rounds) when every row is
// max_seq_len long.  A long piece spreads a workgroup's fixed cost (its q
// loads, the merge of its waves, its share of the merge launch) over more
// keys.  It depends only on arguments the workspace query also takes, so
// that query's answer covers every call it was made for.
int64_t vec_default_partition(int64_t rows, int64_t max_seq_len, int32_t block_size) {
  int64_t P = kDefaultPartitionTokens;
  while (P < 4096 && rows * ceil_div(std::max<int64_t>(max_seq_len, 1), 2 * P) >= 1024) P *= 2;
  return ceil_div(P, block_size) * block_size;
}

// Shape checks shared by both attention calls.
int check_attention_shapes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_seq_len, int32_t kv_dtype,
                           int32_t out_dtype) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0)
    return PA_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!dtype_ok(kv_dtype) || !dtype_ok(out_dtype)) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  // one physical block (all KV heads) is addressed with 32-bit element offsets
  if ((int64_t)num_kv_heads * block_size * head_dim > 0x7fffffff) return PA_ERR_UNSUPPORTED;
  // ... and a whole cache with 8-row offsets in 31 bits (2^41 elements: terabytes)
  if ((int64_t)num_blocks * num_kv_heads * block_size * head_dim >= ((int64_t)1 << 41)) return PA_ERR_UNSUPPORTED;
  if (num_seqs > kMaxGridYZ || num_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// How a decode call splits its work, and where its workspace pieces live.
struct DecodePlan {
  bool streamk = false;
  bool too_large = false;
  bool grid_mfma = false;                // partition grid on the MFMA kernels (else the vector ones)
  int head_split = 1;                    // balanced path: sub-groups of a large GQA group
  int ranges = 0, range_blocks = 0;      // balanced path
  int part_blocks = 0, nparts = 1;       // partition-grid path
  size_t off_part = 0, off_ml = 0, off_desc = 0, workspace_bytes = 0;
  // the balanced path's plan buffer: header, records, records2
  int plan_stride = 0;
  size_t plan_off_rec = 0, plan_off_rec2 = 0, plan_off_desc = 0, plan_bytes = 0;
};

DecodePlan plan_decode(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                       int max_seq_len, int64_t cap, int partition_size, bool mfma_shape) {
  DecodePlan pl;
  const int g = num_heads / num_kv_heads;
  const int64_t rows = (int64_t)num_seqs * num_kv_heads;
  // balanced path: a large group's sub-groups are rows of their own
  const int hs = mfma_shape ? head_split(g) : 1, gv = g / hs;
  // the unit of the split: 16-token tiles on the MFMA path, blocks otherwise
  const int unit = mfma_shape ? 16 : block_size;
  const int64_t part_units = partition_size > 0 ? std::max<int64_t>(1, partition_size / unit) : 0;
  const int64_t blocks_per_row = cap > 0 ? ceil_div(cap, unit) : 0;
  const int64_t t_upper = rows * hs * blocks_per_row;  // flat blocks, at most
  // balanced ranges: the default count, or more when that keeps every range
  // within the blocks a workgroup can stage (t_upper bounds the real total).
  // Rows of more than 8 query heads park so much in LDS that one workgroup
  // fits per CU: half the ranges, so that they all run in one round.
  const int64_t nr = gv > 8 ? pa::kStreamKRanges / 2 : pa::kStreamKRanges;
  const int64_t sk_ranges_default = std::max<int64_t>(
      {1, std::min<int64_t>(nr, t_upper), ceil_div(t_upper, pa::kStreamKTabCache)});
  // The library's own split is always the balanced one on the MFMA path (its
  // merge shares a row cut into many pieces out over the row's ranges).  A
  // caller's fixed pieces take fixed-size ranges when they are few per row;
  // more per row, the partition grid, whose pieces are the row's own.
  const bool fixed_ok = partition_size == 0 ||
                        (part_units <= pa::kStreamKTabCache &&
                         ceil_div(std::max<int64_t>(blocks_per_row, 1), part_units) <= kStreamKMaxPiecesPerRow);
  if (mfma_shape && (int64_t)num_seqs * hs <= pa::kStreamKMaxSeqs && t_upper <= 0x7fffffff && fixed_ok) {
    pl.streamk = true;
    pl.head_split = hs;
    if (partition_size > 0) {
      pl.range_blocks = (int)part_units;
      pl.ranges = (int)std::max<int64_t>(1, ceil_div(t_upper, pl.range_blocks));
    } else {
      pl.range_blocks = 0;
      pl.ranges = (int)sk_ranges_default;
    }
    const size_t part = (size_t)pl.ranges * 2 * gv * head_dim * sizeof(float);
    const size_t ml = (size_t)pl.ranges * 2 * gv * 2 * sizeof(float);
    pl.off_part = 0;
    pl.off_ml = align256(part);
    pl.off_desc = pl.off_ml + align256(ml);
    pl.workspace_bytes = pl.off_desc + align256((size_t)pl.ranges * 4 * sizeof(int));
    // a range holds at most ceil(T / G) <= ceil(t_upper / ranges) positions
    // (or range_blocks), and never more than the staging cache
    pl.plan_stride = pl.range_blocks > 0
                         ? pl.range_blocks
                         : (int)std::min<int64_t>(ceil_div(t_upper, pl.ranges) + 1, pa::kStreamKTabCache);
    pl.plan_off_rec = align256((size_t)pl.ranges * 4 * sizeof(int));
    pl.plan_off_rec2 = pl.plan_off_rec + align256((size_t)pl.ranges * pl.plan_stride * 4 * sizeof(int));
    pl.plan_off_desc = pl.plan_off_rec2 + align256((size_t)pl.ranges * pl.plan_stride * 2 * sizeof(int));
    pl.plan_bytes = pl.plan_off_desc + align256((size_t)pl.ranges * 4 * sizeof(int));
    return pl;
  }
  // the partition grid: MFMA kernels up to 16 query heads per KV head,
  // the vector kernels beyond
  pl.grid_mfma = mfma_shape && g <= 16;
  const int gunit = pl.grid_mfma ? 16 : block_size;
  const int64_t P = !pl.grid_mfma && partition_size <= 0 ? vec_default_partition(rows, max_seq_len, block_size)
                                                         : effective_partition(partition_size, block_size);
  const int64_t pu = std::max<int64_t>(1, P / gunit);  // units per partition
  const int64_t nparts = cap > 0 ? ceil_div(ceil_div(cap, gunit), pu) : 1;
  if (nparts > 0x7fffffff) {
    pl.too_large = true;
    return pl;
  }
  pl.part_blocks = (int)pu;
  pl.nparts = (int)nparts;
  if (nparts > 1) {
    const size_t o = (size_t)num_seqs * num_heads * nparts * head_dim * sizeof(float);
    pl.off_part = 0;
    pl.off_ml = align256(o);
    pl.workspace_bytes = pl.off_ml + align256((size_t)num_seqs * num_heads * nparts * 2 * sizeof(float));
  }
  return pl;
}

}  // namespace

extern "C" {

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "negative or inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, block size or grid size";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "HIP kernel launch failed";
    case PA_ERR_SCRATCH: return "the call needs more scratch than the library's built-in buffer holds";
    default: return "unknown status";
  }
}

int pa_abi_version(void) { return PA_ABI_VERSION; }

int pa_debug_flags(unsigned *flags, int clear) {
#if PAGED_ATTN_DEBUG
  if (!flags) return PA_ERR_NULL;
  if (hipDeviceSynchronize() != hipSuccess) return PA_ERR_LAUNCH;
  hipError_t (*const words[])(void **) = {pa::debug_word_ops, pa::debug_word_decode, pa::debug_word_streamk,
                                          pa::debug_word_prefill};
  unsigned all = 0;
  for (auto word : words) {
    void *p = nullptr;
    unsigned v = 0;
    if (word(&p) != hipSuccess || hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost) != hipSuccess)
      return PA_ERR_LAUNCH;
    all |= v;
    if (clear && hipMemset(p, 0, sizeof v) != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (clear && hipDeviceSynchronize() != hipSuccess) return PA_ERR_LAUNCH;
  *flags = all;
  return PA_OK;
#else
  (void)clear;
  if (flags) *flags = 0;
  return PA_ERR_UNSUPPORTED;
#endif
}

int pa_timeline(uint64_t *main_stamps, uint64_t *merge_stamps, int32_t rows, int32_t clear) {
#if PAGED_ATTN_TIMELINE
  if (!main_stamps || !merge_stamps) return PA_ERR_NULL;
  if (rows < 1 || rows > PA_TIMELINE_ROWS) return PA_ERR_SHAPE;
  if (hipDeviceSynchronize() != hipSuccess) return PA_ERR_LAUNCH;
  void *m = nullptr, *g = nullptr;
  if (pa::timeline_symbols(&m, &g) != hipSuccess) return PA_ERR_LAUNCH;
  if (hipMemcpy(main_stamps, m, (size_t)rows * 8 * sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(merge_stamps, g, (size_t)rows * 2 * sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess)
    return PA_ERR_LAUNCH;
  if (clear) {
    if (hipMemset(m, 0, (size_t)PA_TIMELINE_ROWS * 8 * sizeof(uint64_t)) != hipSuccess ||
        hipMemset(g, 0, (size_t)PA_TIMELINE_ROWS * 2 * sizeof(uint64_t)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
      return PA_ERR_LAUNCH;
  }
  return PA_OK;
#else
  (void)main_stamps;
  (void)merge_stamps;
  (void)rows;
  (void)clear;
  return PA_ERR_UNSUPPORTED;
#endif
}

int kv_cache_write(const void *key, const void *value, void *k_cache, void *v_cache,
                   const int64_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                   int32_t num_kv_heads, int32_t block_size, int32_t head_dim, int32_t dtype,
                   void *stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
    return PA_ERR_SHAPE;
  if (!storage_dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if ((head_dim * elem_bytes(dtype)) % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  return launch_status(pa::launch_kv_cache_write(key, value, k_cache, v_cache, slot_mapping,
                                                 num_tokens, num_blocks, num_kv_heads, block_size,
                                                 head_dim, elem_bytes(dtype),
                                                 static_cast<hipStream_t>(stream)));
}

int kv_cache_write_fp8(const void *key, const void *value, int32_t src_dtype, void *k_cache, void *v_cache,
                       const int64_t *slot_mapping, int32_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                       int32_t block_size, int32_t head_dim, float k_scale, float v_scale, void *stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
    return PA_ERR_SHAPE;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PA_ERR_SHAPE;
  if (!dtype_ok(src_dtype) || head_dim % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  return launch_status(pa::launch_kv_cache_write_fp8(key, value, src_dtype == PA_BF16, k_cache, v_cache,
                                                     slot_mapping, num_tokens, num_blocks, num_kv_heads,
                                                     block_size, head_dim, k_scale, v_scale,
                                                     static_cast<hipStream_t>(stream)));
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                        int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_seq_len < 0 || partition_size < 0 || num_heads % num_kv_heads != 0)
    return 0;
  if (partition_size > 0 && partition_size % block_size != 0) return 0;
  // the larger of the two kernels' needs: the dtype is not an argument here
  DecodePlan a = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                             max_seq_len, partition_size, true);
  DecodePlan b = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                             max_seq_len, partition_size, false);
  return std::max(a.workspace_bytes, b.workspace_bytes);
}

}  // extern "C"

namespace {

bool mfma_decode_shape(int32_t kv_dtype, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size) {
  return (kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3) && head_dim == 128 && pa::mfma_block_size(block_size);
}

// The new token of every sequence for a decode step that also writes it:
// key/value [num_seqs][num_kv_heads][head_dim] (bf16 for bf16 and FP8
// caches, fp32 for fp32 caches), slot_mapping [num_seqs].
struct AppendRows {
  const void *key, *value;
  const int64_t *slot_mapping;
};

// Every decode entry point.  kv_dtype PA_FP8_E4M3: the caches hold E4M3
// codes read as value * k_scale / v_scale, q is bf16, and only the MFMA
// shapes are served.  plan (may be NULL): a plan from
// paged_attn_decode_plan for the same sizes, block tables and seq_lens.
int decode_impl(void *out, int32_t out_dtype, const void *q, const void *k_cache, const void *v_cache,
                int32_t kv_dtype, float k_scale, float v_scale, const int32_t *block_tables,
                int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                int32_t max_seq_len, float scale, int32_t partition_size, void *workspace,
                size_t workspace_bytes, void *stream, bool planned = false, const void *plan_buf = nullptr,
                size_t plan_bytes = 0, const AppendRows *append = nullptr) {
  const bool fp8 = kv_dtype == PA_FP8_E4M3;
  int st = check_attention_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                  max_blocks_per_seq, max_seq_len, fp8 ? PA_BF16 : kv_dtype, out_dtype);
  if (st != PA_OK) return st;
  if (!scale_ok(scale)) return PA_ERR_SHAPE;  // the kernels scale after taking the max
  if (fp8 && !scale_ok(k_scale)) return PA_ERR_SHAPE;
  if (fp8 && !scale_ok(v_scale)) return PA_ERR_SHAPE;
  if (fp8 && !(head_dim == 128 && pa::mfma_block_size(block_size))) return PA_ERR_UNSUPPORTED;
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size != 0))
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_NULL;

  const int64_t cap = std::min<int64_t>(max_seq_len, (int64_t)max_blocks_per_seq * block_size);
  const bool mfma_shape = mfma_decode_shape(kv_dtype, num_heads, num_kv_heads, head_dim, block_size);
  DecodePlan plan = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                                cap, partition_size, mfma_shape);
  if (plan.too_large) return PA_ERR_UNSUPPORTED;
  // FP8 caches have MFMA kernels only: a group above 16 needs the balanced path
  if (fp8 && !plan.streamk && !plan.grid_mfma) return PA_ERR_UNSUPPORTED;
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return PA_ERR_WORKSPACE;
  if (planned && plan.streamk && (!plan_buf || plan_bytes < plan.plan_bytes)) return PA_ERR_WORKSPACE;
  // the step's write: folded into the planned bf16 balanced kernels (the
  // main kernel reads the new rows in place of position L - 1, the merge
  // kernel writes them to their slots), otherwise written first
  const bool fold = append && planned && plan.streamk && kv_dtype == PA_BF16 && plan.head_split == 1;
  if (append) {
    if (!append->key || !append->value || !append->slot_mapping) return PA_ERR_NULL;
    if (!fold) {
      void *kcw = const_cast<void *>(k_cache), *vcw = const_cast<void *>(v_cache);
      const int ws = fp8 ? kv_cache_write_fp8(append->key, append->value, PA_BF16, kcw, vcw, append->slot_mapping,
                                              num_seqs, num_blocks, num_kv_heads, block_size, head_dim, k_scale,
                                              v_scale, stream)
                         : kv_cache_write(append->key, append->value, kcw, vcw, append->slot_mapping, num_seqs,
                                          num_blocks, num_kv_heads, block_size, head_dim, kv_dtype, stream);
      if (ws != PA_OK) return ws;
    }
  }

  pa::DecodeParams p = {};
  p.out = out;
  p.out_bf16 = out_dtype == PA_BF16;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.kv_fp8 = fp8;
  p.k_scale = fp8 ? k_scale : 1.f;
  p.v_scale = fp8 ? v_scale : 1.f;
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.seq_lens = seq_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_len_cap = (int)cap;
  p.scale = scale;
  p.head_split = plan.streamk ? plan.head_split : 1;
  char *ws = static_cast<char *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.streamk) {
    p.sk_ranges = plan.ranges;
    p.sk_range_blocks = plan.range_blocks;
    p.sk_part = reinterpret_cast<float *>(ws + plan.off_part);
    p.sk_ml = reinterpret_cast<float *>(ws + plan.off_ml);
    p.sk_desc = reinterpret_cast<int4 *>(ws + plan.off_desc);
    if (planned) {
      char *pb = static_cast<char *>(const_cast<void *>(plan_buf));
      p.plan_hdr = reinterpret_cast<int4 *>(pb);
      p.plan_rec = reinterpret_cast<int4 *>(pb + plan.plan_off_rec);
      p.plan_rec2 = reinterpret_cast<int2 *>(pb + plan.plan_off_rec2);
      p.sk_desc = reinterpret_cast<int4 *>(pb + plan.plan_off_desc);  // the plan's merge descriptors
      p.plan_stride = plan.plan_stride;
    }
    if (fold) {
      p.new_k = append->key;
      p.new_v = append->value;
      p.slot_mapping = append->slot_mapping;
    }
    return launch_status(pa::launch_decode_streamk(p, s));
  }
  p.tile_tokens = plan.grid_mfma ? 16 : block_size;
  p.part_blocks = plan.part_blocks;
  p.nparts_max = plan.nparts;
  p.ws_o = plan.workspace_bytes > 0 ? reinterpret_cast<float *>(ws + plan.off_part) : nullptr;
  p.ws_ml = plan.workspace_bytes > 0 ? reinterpret_cast<float *>(ws + plan.off_ml) : nullptr;
  return launch_status(pa::launch_decode(p, s));
}

}  // namespace

extern "C" {

int paged_attn_decode(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                      const void *v_cache, int32_t kv_dtype, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *stream) {
  if (!dtype_ok(kv_dtype)) return PA_ERR_UNSUPPORTED;
  return decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, 1.f, 1.f, block_tables, max_blocks_per_seq,
                     seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len,
                     scale, partition_size, workspace, workspace_bytes, stream);
}

size_t paged_attn_decode_plan_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len,
                                   int32_t partition_size, int32_t kv_dtype) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || max_seq_len < 0 || partition_size < 0 || num_heads % num_kv_heads != 0)
    return 0;
  if (partition_size > 0 && partition_size % block_size != 0) return 0;
  const int64_t cap = std::min<int64_t>(max_seq_len, (int64_t)max_blocks_per_seq * block_size);
  DecodePlan plan = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len, cap,
                                partition_size, mfma_decode_shape(kv_dtype, num_heads, num_kv_heads, head_dim,
                                                                  block_size));
  return plan.streamk ? plan.plan_bytes : 0;
}

int paged_attn_decode_plan(void *plan_buf, size_t plan_bytes, int32_t kv_dtype, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_seq_len, int32_t partition_size, void *stream) {
  const bool fp8 = kv_dtype == PA_FP8_E4M3;
  if (!fp8 && !dtype_ok(kv_dtype)) return PA_ERR_UNSUPPORTED;
  int st = check_attention_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                  max_blocks_per_seq, max_seq_len, fp8 ? PA_BF16 : kv_dtype, PA_F32);
  if (st != PA_OK) return st;
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size != 0)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  const int64_t cap = std::min<int64_t>(max_seq_len, (int64_t)max_blocks_per_seq * block_size);
  DecodePlan plan = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len, cap,
                                partition_size,
                                mfma_decode_shape(kv_dtype, num_heads, num_kv_heads, head_dim, block_size));
  if (!plan.streamk) return PA_OK;  // this shape is not split by ranges: nothing to plan
  if (!plan_buf || plan_bytes < plan.plan_bytes) return PA_ERR_WORKSPACE;
  if (!block_tables || !seq_lens) return PA_ERR_NULL;
  pa::DecodeParams p = {};
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.seq_lens = seq_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_len_cap = (int)cap;
  p.head_split = plan.head_split;
  p.sk_ranges = plan.ranges;
  p.sk_range_blocks = plan.range_blocks;
  char *pb = static_cast<char *>(plan_buf);
  p.plan_hdr = reinterpret_cast<int4 *>(pb);
  p.plan_rec = reinterpret_cast<int4 *>(pb + plan.plan_off_rec);
  p.plan_rec2 = reinterpret_cast<int2 *>(pb + plan.plan_off_rec2);
  p.sk_desc = reinterpret_cast<int4 *>(pb + plan.plan_off_desc);
  p.plan_stride = plan.plan_stride;
  return launch_status(pa::launch_decode_streamk_plan(p, static_cast<hipStream_t>(stream)));
}

int paged_attn_decode_planned(void *out, int32_t out_dtype, const void *q, const void *k_cache, const void *v_cache,
                              int32_t kv_dtype, float k_scale, float v_scale, const void *plan_buf,
                              size_t plan_bytes, const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                              float scale, int32_t partition_size, void *workspace, size_t workspace_bytes,
                              void *stream) {
  if (kv_dtype != PA_FP8_E4M3 && !dtype_ok(kv_dtype)) return PA_ERR_UNSUPPORTED;
  return decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_seq_len, scale, partition_size, workspace, workspace_bytes, stream, true,
                     plan_buf, plan_bytes);
}

int paged_attn_decode_append(void *out, int32_t out_dtype, const void *q, const void *key, const void *value,
                             const int64_t *slot_mapping, void *k_cache, void *v_cache, int32_t kv_dtype,
                             float k_scale, float v_scale, const void *plan_buf, size_t plan_bytes,
                             const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *seq_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                             int32_t partition_size, void *workspace, size_t workspace_bytes, void *stream) {
  if (kv_dtype != PA_FP8_E4M3 && !dtype_ok(kv_dtype)) return PA_ERR_UNSUPPORTED;
  const AppendRows rows = {key, value, slot_mapping};
  return decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_seq_len, scale, partition_size, workspace, workspace_bytes, stream, true,
                     plan_buf, plan_bytes, &rows);
}

int paged_attn_decode_fp8(void *out, int32_t out_dtype, const void *q, const void *k_cache, const void *v_cache,
                          float k_scale, float v_scale, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                          float scale, int32_t partition_size, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return decode_impl(out, out_dtype, q, k_cache, v_cache, PA_FP8_E4M3, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_seq_len, scale, partition_size, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

int prefill_impl(void *out, int32_t out_dtype, const void *q, const void *k_cache, const void *v_cache,
                 int32_t kv_dtype, float k_scale, float v_scale, const int32_t *block_tables,
                 int32_t max_blocks_per_seq, const int32_t *query_start_loc, const int32_t *seq_lens,
                 int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_query_len,
                 int32_t max_seq_len, float scale, void *stream) {
  const bool fp8 = kv_dtype == PA_FP8_E4M3;
  int st = check_attention_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                  max_blocks_per_seq, max_seq_len, fp8 ? PA_BF16 : kv_dtype, out_dtype);
  if (st != PA_OK) return st;
  if (!scale_ok(scale)) return PA_ERR_SHAPE;  // the kernels scale after taking the max
  if (fp8 && !scale_ok(k_scale)) return PA_ERR_SHAPE;
  if (fp8 && !scale_ok(v_scale)) return PA_ERR_SHAPE;
  const int g = num_heads / num_kv_heads;
  const bool mfma = (kv_dtype == PA_BF16 || fp8) && head_dim == 128 && pa::mfma_block_size(block_size);
  if (fp8 && !mfma) return PA_ERR_UNSUPPORTED;
  // MFMA kernels: a column group is 16 / gs tokens x gs heads, gs the largest
  // power of two up to 16 that divides g; g / gs sub-groups per KV head
  int gs = 16;
  while (g % gs != 0) gs >>= 1;
  if (max_query_len < 0 || num_query_tokens < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_query_len == 0 || num_query_tokens == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !seq_lens)
    return PA_ERR_NULL;
  const int64_t cap = std::min<int64_t>(max_seq_len, (int64_t)max_blocks_per_seq * block_size);
  pa::PrefillParams p = {};
  p.out = out;
  p.out_bf16 = out_dtype == PA_BF16;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.kv_bf16 = kv_dtype == PA_BF16;
  p.kv_fp8 = fp8;
  p.k_scale = fp8 ? k_scale : 1.f;
  p.v_scale = fp8 ? v_scale : 1.f;
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.query_start_loc = query_start_loc;
  p.seq_lens = seq_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_query_len = max_query_len;
  p.num_query_tokens = num_query_tokens;
  p.max_len_cap = (int)cap;
  p.scale = scale;
  p.head_split = mfma ? g / gs : 1;
  return launch_status(pa::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int paged_attn_prefill_chunk(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                             const void *v_cache, int32_t kv_dtype, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *query_start_loc,
                             const int32_t *seq_lens, int32_t num_seqs, int32_t num_query_tokens,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_query_len,
                             int32_t max_seq_len, float scale, void *stream) {
  if (!dtype_ok(kv_dtype)) return PA_ERR_UNSUPPORTED;
  return prefill_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, 1.f, 1.f, block_tables, max_blocks_per_seq,
                      query_start_loc, seq_lens, num_seqs, num_query_tokens, num_heads, num_kv_heads, head_dim,
                      block_size, num_blocks, max_query_len, max_seq_len, scale, stream);
}

int paged_attn_prefill_chunk_fp8(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                                 const void *v_cache, float k_scale, float v_scale, const int32_t *block_tables,
                                 int32_t max_blocks_per_seq, const int32_t *query_start_loc,
                                 const int32_t *seq_lens, int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t max_query_len, int32_t max_seq_len, float scale,
                                 void *stream) {
  return prefill_impl(out, out_dtype, q, k_cache, v_cache, PA_FP8_E4M3, k_scale, v_scale, block_tables,
                      max_blocks_per_seq, query_start_loc, seq_lens, num_seqs, num_query_tokens, num_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_query_len, max_seq_len, scale, stream);
}

int block_copy(void *k_cache, void *v_cache, const int64_t *pairs, int32_t num_pairs,
               int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
               int32_t dtype, void *stream) {
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
    return PA_ERR_SHAPE;
  if (!storage_dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if ((head_dim * elem_bytes(dtype)) % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_NULL;
  if ((int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype) / 16 > 0x7fff0000)
    return PA_ERR_UNSUPPORTED;  // chunk indexes (plus a slice) stay within int
  return launch_status(pa::launch_block_copy(k_cache, v_cache, pairs, num_pairs, num_blocks,
                                             num_kv_heads, block_size, head_dim, elem_bytes(dtype),
                                             static_cast<hipStream_t>(stream)));
}

namespace {

// Shared by both swap directions: checks, then per chunk of staging-sized
// id runs, the gather kernel + a device-to-host copy, or a host-to-device
// copy + the scatter kernel, all on `stream`.
int swap_blocks(bool out, void *k_cache, void *v_cache, const int64_t *block_ids, int32_t num_ids,
                void *host, void *staging, size_t staging_bytes, int32_t num_blocks, int32_t num_kv_heads,
                int32_t block_size, int32_t head_dim, int32_t dtype, void *stream) {
  if (num_ids < 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
    return PA_ERR_SHAPE;
  if (!storage_dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if ((head_dim * elem_bytes(dtype)) % 16 != 0) return PA_ERR_UNSUPPORTED;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes / 16 > 0x7fffffff) return PA_ERR_UNSUPPORTED;
  if (num_ids == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_ids || !host) return PA_ERR_NULL;
  const int64_t per_id = 2 * block_bytes;
  if (!staging || staging_bytes < (size_t)per_id) return PA_ERR_WORKSPACE;
  const int64_t chunk = std::min<int64_t>({(int64_t)(staging_bytes / per_id), num_ids, 65535});
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t i0 = 0; i0 < num_ids; i0 += chunk) {
    const int n = (int)std::min<int64_t>(chunk, num_ids - i0);
    uint8_t *h = static_cast<uint8_t *>(host) + i0 * per_id;
    hipError_t e;
    if (out) {
      e = pa::launch_swap_blocks(true, k_cache, v_cache, block_ids + i0, n, staging, num_blocks,
                                 (int)(block_bytes / 16), s);
      if (e == hipSuccess) e = hipMemcpyAsync(h, staging, n * per_id, hipMemcpyDeviceToHost, s);
    } else {
      e = hipMemcpyAsync(staging, h, n * per_id, hipMemcpyHostToDevice, s);
      if (e == hipSuccess)
        e = pa::launch_swap_blocks(false, k_cache, v_cache, block_ids + i0, n, staging, num_blocks,
                                   (int)(block_bytes / 16), s);
    }
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

}  // namespace

int kv_swap_out(const void *k_cache, const void *v_cache, const int64_t *block_ids, int32_t num_ids,
                void *host_dst, void *staging, size_t staging_bytes, int32_t num_blocks, int32_t num_kv_heads,
                int32_t block_size, int32_t head_dim, int32_t dtype, void *stream) {
  return swap_blocks(true, const_cast<void *>(k_cache), const_cast<void *>(v_cache), block_ids, num_ids,
                     host_dst, staging, staging_bytes, num_blocks, num_kv_heads, block_size, head_dim, dtype,
                     stream);
}

int kv_swap_in(void *k_cache, void *v_cache, const int64_t *block_ids, int32_t num_ids, const void *host_src,
               void *staging, size_t staging_bytes, int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
               int32_t head_dim, int32_t dtype, void *stream) {
  return swap_blocks(false, k_cache, v_cache, block_ids, num_ids, const_cast<void *>(host_src), staging,
                     staging_bytes, num_blocks, num_kv_heads, block_size, head_dim, dtype, stream);
}

}  // extern "C"

// -- Decode without allocation -------------------------------------------------
// For callers that cannot allocate (code under graph capture, tight serving
// loops): paged_attn_decode with its workspace in a fixed device array of
// this library instead of a caller buffer.  Each GPU the library runs on
// holds its own copy of the array until the process ends.  Host code never
// passes the array's name to a kernel (on the host that name is only a
// stand-in): its device address is looked up once per device, with that
// device current, and kept.  The decode kernels need no part of their
// workspace cleared (every piece the merge reads is written earlier in the
// same call), so the array is never initialised.
namespace {

static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on `dev` (nullptr on failure), looked up on
// first use with `dev` current; the caller's current device is restored.
void *scratch_on_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return nullptr;
  if (prev != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void *found = nullptr;
  const hipError_t e = hipGetSymbolAddress(&found, HIP_SYMBOL(scratch));
  if (prev != dev) (void)hipSetDevice(prev);
  if (e != hipSuccess || !found) {
    (void)hipGetLastError();  // clear the sticky error of the failed lookup
    return nullptr;
  }
  g_scratch_ptr[dev].store(found, std::memory_order_release);
  return found;
}

}  // namespace

extern "C" {

int paged_attn_decode_noalloc(void *out, int32_t out_dtype, const void *q, const void *k_cache,
                              const void *v_cache, int32_t kv_dtype, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_seq_len, float scale, int32_t partition_size,
                              void *stream) {
  if (!dtype_ok(kv_dtype)) return PA_ERR_UNSUPPORTED;
  // every argument check of paged_attn_decode first, with an empty
  // workspace: a call that needs none is served as is, one that needs some
  // fails only with PA_ERR_WORKSPACE
  int st = decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, 1.f, 1.f, block_tables, max_blocks_per_seq,
                       seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len,
                       scale, partition_size, nullptr, 0, stream);
  if (st != PA_ERR_WORKSPACE) return st;
  // the workspace of the kernel this call picks (the arguments are valid here)
  const int64_t cap = std::min<int64_t>(max_seq_len, (int64_t)max_blocks_per_seq * block_size);
  const DecodePlan plan = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len, cap,
                                      partition_size,
                                      mfma_decode_shape(kv_dtype, num_heads, num_kv_heads, head_dim, block_size));
  if (plan.workspace_bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return PA_ERR_LAUNCH;
  void *ws = scratch_on_device(dev);
  if (!ws) return PA_ERR_LAUNCH;
  return decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, 1.f, 1.f, block_tables, max_blocks_per_seq,
                     seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len,
                     scale, partition_size, ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
