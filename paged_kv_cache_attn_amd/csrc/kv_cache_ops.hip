// kv_cache_ops.hip -- the two memory kernels around paged attention:
//   kv_cache_write: scatter new K/V rows into their slots (Lecture 7 "KV Cache
//     Management" §4.3, first fused kernel; slots follow the fill rule of
//     §4.1 and of Lecture 16 "LLM Serving (1)" §3.3);
//   block_copy: batched whole-block copies for copy-on-write (Lecture 7 §4.3,
//     third fused kernel, and §5.1).
//   swap gather / scatter: the listed blocks of one layer packed into (or
//     unpacked from) a contiguous staging buffer, so a swap between HBM and
//     host memory is one DMA copy per chunk instead of one per block
//     (Lecture 7 §6.2: swapping costs PCIe bandwidth plus a fixed cost per
//     copy; Month 2 §8.1: a 4K-token sequence's blocks are swapped together).
// Both are pure HBM streams: each thread moves 16-byte chunks with
// global_load_dwordx4 / global_store_dwordx4, consecutive threads take
// consecutive chunks of a row so every wave touches whole 256-byte rows.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// One thread per 16-byte chunk of one (token, head) row; K and V handled by
// the same thread.  row_chunks = head_dim * elem_bytes / 16.
// I: the index type of the chunk arithmetic (32-bit whenever the counts fit,
// which keeps the divisions short).  The key/value chunk is loaded before the
// slot is known (its address does not depend on it), so the slot load and the
// data loads share one memory round trip.
template <typename I>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const uint8_t *__restrict__ key, const uint8_t *__restrict__ value,
    uint8_t *__restrict__ k_cache, uint8_t *__restrict__ v_cache,
    const int64_t *__restrict__ slot_mapping, I total_chunks, int num_kv_heads,
    int block_size, int row_chunks, int64_t num_slots) {
  const I gid = (I)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_chunks) return;
  const I chunk = gid % (I)row_chunks;
  const I row = gid / (I)row_chunks;  // t * num_kv_heads + h
  const I h = row % (I)num_kv_heads;
  const I t = row / (I)num_kv_heads;
  const int64_t row_bytes = (int64_t)row_chunks * 16;
  const int64_t src = (int64_t)row * row_bytes + (int64_t)chunk * 16;
  const u32x4 kv = ld16(key + src);
  const u32x4 vv = ld16(value + src);
  const int64_t slot = slot_mapping[t];
  // Consume all three loads before the slot test, so the compiler cannot sink
  // the data loads behind it: they are issued together, one round trip.
  asm volatile("" ::"v"(kv), "v"(vv), "v"(slot));
  debug_report(slot >= num_slots, kDbgSlotRange);
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int off = (int)(slot - blk * block_size);
  const int64_t dst_row = (blk * num_kv_heads + h) * block_size + off;
  const int64_t dst = dst_row * row_bytes + (int64_t)chunk * 16;
  st16(k_cache + dst, kv);
  st16(v_cache + dst, vv);
}

// Quantising write into FP8 E4M3 caches (Lecture 7 §10: KV stored in 8 bits
// halves its memory and bandwidth).  One thread per 16 codes (16 bytes) of
// one (token, head) row, K and V: the 16 source values (bf16 or fp32) are
// loaded with the slot, divided by the tensor's scale (IEEE fp32 division,
// round to nearest) and rounded to the nearest code with ties to even,
// saturating at +-448.  row_chunks = head_dim / 16.
template <typename I, bool SRC_BF16>
__global__ __launch_bounds__(256) void kv_cache_write_fp8_kernel(
    const uint8_t *__restrict__ key, const uint8_t *__restrict__ value, uint8_t *__restrict__ k_cache,
    uint8_t *__restrict__ v_cache, const int64_t *__restrict__ slot_mapping, I total_chunks, int num_kv_heads,
    int block_size, int row_chunks, int64_t num_slots, float k_scale, float v_scale) {
  constexpr int kSrcLoads = SRC_BF16 ? 2 : 4;  // 16-byte loads for 16 source values
  const I gid = (I)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_chunks) return;
  const I chunk = gid % (I)row_chunks;
  const I row = gid / (I)row_chunks;  // t * num_kv_heads + h
  const I h = row % (I)num_kv_heads;
  const I t = row / (I)num_kv_heads;
  const int64_t src = ((int64_t)row * row_chunks + chunk) * 16 * (SRC_BF16 ? 2 : 4);
  u32x4 ks[kSrcLoads], vs[kSrcLoads];
#pragma unroll
  for (int i = 0; i < kSrcLoads; ++i) {
    ks[i] = ld16(key + src + 16 * i);
    vs[i] = ld16(value + src + 16 * i);
  }
  const int64_t slot = slot_mapping[t];
  asm volatile("" ::"v"(ks[0]), "v"(vs[0]), "v"(slot));
  debug_report(slot >= num_slots, kDbgSlotRange);
  if (slot < 0 || slot >= num_slots) return;
  // source value j (0..15) of a row piece
  auto val = [&](const u32x4 *s, int j) -> float {
    if (SRC_BF16) {
      const uint32_t w = s[j >> 3][(j >> 1) & 3];
      return bf16_bits_to_float((j & 1) ? w >> 16 : w & 0xffffu);
    }
    return __uint_as_float(s[j >> 2][j & 3]);
  };
  u32x4 kq, vq;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kq[i] = pack_fp8x4(__fdiv_rn(val(ks, 4 * i), k_scale), __fdiv_rn(val(ks, 4 * i + 1), k_scale),
                       __fdiv_rn(val(ks, 4 * i + 2), k_scale), __fdiv_rn(val(ks, 4 * i + 3), k_scale));
    vq[i] = pack_fp8x4(__fdiv_rn(val(vs, 4 * i), v_scale), __fdiv_rn(val(vs, 4 * i + 1), v_scale),
                       __fdiv_rn(val(vs, 4 * i + 2), v_scale), __fdiv_rn(val(vs, 4 * i + 3), v_scale));
  }
  const int64_t blk = slot / block_size;
  const int off = (int)(slot - blk * block_size);
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * (int64_t)row_chunks * 16 + (int64_t)chunk * 16;
  st16(k_cache + dst, kq);
  st16(v_cache + dst, vq);
}

#if PAGED_ATTN_DEBUG
PA_DEBUG_WORD_ACCESSOR(debug_word_ops)

// Debug build: thread t compares its slot with those of the later tokens.
__global__ __launch_bounds__(256) void debug_dup_slots_kernel(const int64_t *__restrict__ slots, int n,
                                                              int64_t num_slots) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;
  bool dup = false;
  for (int u = t + 1; u < n; ++u) dup |= slots[u] == s;
  debug_report(dup, kDbgSlotDup);
}

// Debug build: pair i against every other pair j: a dst used twice, or a dst
// that is another pair's src (the copies run concurrently).
__global__ __launch_bounds__(256) void debug_pair_conflicts_kernel(const int64_t *__restrict__ pairs, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t src = pairs[2 * (int64_t)i], dst = pairs[2 * (int64_t)i + 1];
  if (src == dst) return;  // a no-op
  bool bad = false;
  for (int j = 0; j < n; ++j) {
    const int64_t s2 = pairs[2 * (int64_t)j], d2 = pairs[2 * (int64_t)j + 1];
    if (j == i || s2 == d2) continue;  // itself, or another no-op
    bad |= d2 == dst || s2 == dst || d2 == src;
  }
  debug_report(bad, kDbgPairConflict);
}
#endif

hipError_t launch_kv_cache_write_fp8(const void *key, const void *value, int src_bf16, void *k_cache,
                                     void *v_cache, const int64_t *slot_mapping, int num_tokens,
                                     int num_blocks, int num_kv_heads, int block_size, int head_dim,
                                     float k_scale, float v_scale, hipStream_t stream) {
  const int row_chunks = head_dim / 16;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * row_chunks;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const uint8_t *k8 = (const uint8_t *)key, *v8 = (const uint8_t *)value;
  uint8_t *kc = (uint8_t *)k_cache, *vc = (uint8_t *)v_cache;
  const bool narrow = total < INT32_MAX && num_slots < INT32_MAX;
#if PAGED_ATTN_DEBUG
  hipLaunchKernelGGL(debug_dup_slots_kernel, dim3((num_tokens + 255) / 256), dim3(256), 0, stream, slot_mapping,
                     num_tokens, num_slots);
#endif
  if (narrow && src_bf16)
    hipLaunchKernelGGL((kv_cache_write_fp8_kernel<uint32_t, true>), dim3((unsigned)grid), dim3(256), 0, stream,
                       k8, v8, kc, vc, slot_mapping, (uint32_t)total, num_kv_heads, block_size, row_chunks,
                       num_slots, k_scale, v_scale);
  else if (narrow)
    hipLaunchKernelGGL((kv_cache_write_fp8_kernel<uint32_t, false>), dim3((unsigned)grid), dim3(256), 0, stream,
                       k8, v8, kc, vc, slot_mapping, (uint32_t)total, num_kv_heads, block_size, row_chunks,
                       num_slots, k_scale, v_scale);
  else if (src_bf16)
    hipLaunchKernelGGL((kv_cache_write_fp8_kernel<int64_t, true>), dim3((unsigned)grid), dim3(256), 0, stream,
                       k8, v8, kc, vc, slot_mapping, total, num_kv_heads, block_size, row_chunks, num_slots,
                       k_scale, v_scale);
  else
    hipLaunchKernelGGL((kv_cache_write_fp8_kernel<int64_t, false>), dim3((unsigned)grid), dim3(256), 0, stream,
                       k8, v8, kc, vc, slot_mapping, total, num_kv_heads, block_size, row_chunks, num_slots,
                       k_scale, v_scale);
  return hipGetLastError();
}

// grid.x = pair, grid.y = 0 (K) / 1 (V); each workgroup copies one block of
// one cache: block_chunks 16-byte chunks, strided over 256 threads.
__global__ __launch_bounds__(256) void block_copy_kernel(uint8_t *__restrict__ k_cache,
                                                         uint8_t *__restrict__ v_cache,
                                                         const int64_t *__restrict__ pairs,
                                                         int64_t num_blocks, int block_chunks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.x];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  debug_report(threadIdx.x == 0 && (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks), kDbgPairRange);
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks || src == dst) return;
  uint8_t *cache = blockIdx.y == 0 ? k_cache : v_cache;
  const int64_t bytes = (int64_t)block_chunks * 16;
  const uint8_t *s = cache + src * bytes;
  uint8_t *d = cache + dst * bytes;
  // 4 chunks in flight per thread before the stores
  int i = threadIdx.x;
  for (; i + 3 * 256 < block_chunks; i += 4 * 256) {
    u32x4 a = ld16(s + (int64_t)i * 16), b = ld16(s + (int64_t)(i + 256) * 16);
    u32x4 c = ld16(s + (int64_t)(i + 512) * 16), e = ld16(s + (int64_t)(i + 768) * 16);
    st16(d + (int64_t)i * 16, a);
    st16(d + (int64_t)(i + 256) * 16, b);
    st16(d + (int64_t)(i + 512) * 16, c);
    st16(d + (int64_t)(i + 768) * 16, e);
  }
  for (; i < block_chunks; i += 256) st16(d + (int64_t)i * 16, ld16(s + (int64_t)i * 16));
}

// Swap staging.  Gather: staging piece (i, kv) = block ids[i] of the K
// (kv = 0) or V (kv = 1) cache; an id outside [0, num_blocks) gives a zero
// piece.  Scatter: the reverse, skipping such ids.  One workgroup per piece,
// grid (n, 2); `ids` points at the first id of this chunk.
template <bool kGather>
__global__ __launch_bounds__(256) void swap_blocks_kernel(uint8_t *__restrict__ k_cache,
                                                          uint8_t *__restrict__ v_cache,
                                                          const int64_t *__restrict__ ids,
                                                          uint8_t *__restrict__ staging,
                                                          int64_t num_blocks, int block_chunks) {
  const int64_t id = ids[blockIdx.x];
  const bool ok = id >= 0 && id < num_blocks;
  debug_report(threadIdx.x == 0 && !ok, kDbgSwapRange);
  if (!kGather && !ok) return;
  const int64_t bytes = (int64_t)block_chunks * 16;
  uint8_t *blk = (blockIdx.y == 0 ? k_cache : v_cache) + (ok ? id : 0) * bytes;
  uint8_t *stg = staging + ((int64_t)blockIdx.x * 2 + blockIdx.y) * bytes;
  const uint8_t *s = kGather ? blk : stg;
  uint8_t *d = kGather ? stg : blk;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  int i = threadIdx.x;
  for (; i + 3 * 256 < block_chunks; i += 4 * 256) {
    u32x4 a = ld16(s + (int64_t)i * 16), b = ld16(s + (int64_t)(i + 256) * 16);
    u32x4 c = ld16(s + (int64_t)(i + 512) * 16), e = ld16(s + (int64_t)(i + 768) * 16);
    st16(d + (int64_t)i * 16, ok ? a : zero);
    st16(d + (int64_t)(i + 256) * 16, ok ? b : zero);
    st16(d + (int64_t)(i + 512) * 16, ok ? c : zero);
    st16(d + (int64_t)(i + 768) * 16, ok ? e : zero);
  }
  for (; i < block_chunks; i += 256) {
    const u32x4 a = ld16(s + (int64_t)i * 16);
    st16(d + (int64_t)i * 16, ok ? a : zero);
  }
}

hipError_t launch_swap_blocks(bool gather, void *k_cache, void *v_cache, const int64_t *ids, int n,
                              void *staging, int num_blocks, int block_chunks, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (gather)
    hipLaunchKernelGGL(swap_blocks_kernel<true>, dim3((unsigned)n, 2), dim3(256), 0, stream, (uint8_t *)k_cache,
                       (uint8_t *)v_cache, ids, (uint8_t *)staging, (int64_t)num_blocks, block_chunks);
  else
    hipLaunchKernelGGL(swap_blocks_kernel<false>, dim3((unsigned)n, 2), dim3(256), 0, stream, (uint8_t *)k_cache,
                       (uint8_t *)v_cache, ids, (uint8_t *)staging, (int64_t)num_blocks, block_chunks);
  return hipGetLastError();
}

hipError_t launch_kv_cache_write(const void *key, const void *value, void *k_cache, void *v_cache,
                                 const int64_t *slot_mapping, int num_tokens, int num_blocks,
                                 int num_kv_heads, int block_size, int head_dim, int elem_bytes,
                                 hipStream_t stream) {
  const int row_chunks = head_dim * elem_bytes / 16;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * row_chunks;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
#if PAGED_ATTN_DEBUG
  hipLaunchKernelGGL(debug_dup_slots_kernel, dim3((num_tokens + 255) / 256), dim3(256), 0, stream, slot_mapping,
                     num_tokens, num_slots);
#endif
  if (total < INT32_MAX && num_slots < INT32_MAX)
    hipLaunchKernelGGL(kv_cache_write_kernel<uint32_t>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t *)key, (const uint8_t *)value, (uint8_t *)k_cache, (uint8_t *)v_cache,
                       slot_mapping, (uint32_t)total, num_kv_heads, block_size, row_chunks, num_slots);
  else
    hipLaunchKernelGGL(kv_cache_write_kernel<int64_t>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t *)key, (const uint8_t *)value, (uint8_t *)k_cache, (uint8_t *)v_cache,
                       slot_mapping, total, num_kv_heads, block_size, row_chunks, num_slots);
  return hipGetLastError();
}

hipError_t launch_block_copy(void *k_cache, void *v_cache, const int64_t *pairs, int num_pairs,
                             int num_blocks, int num_kv_heads, int block_size, int head_dim,
                             int elem_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int block_chunks = (int)((int64_t)num_kv_heads * block_size * head_dim * elem_bytes / 16);
#if PAGED_ATTN_DEBUG
  hipLaunchKernelGGL(debug_pair_conflicts_kernel, dim3((num_pairs + 255) / 256), dim3(256), 0, stream, pairs,
                     num_pairs);
#endif
  hipLaunchKernelGGL(block_copy_kernel, dim3((unsigned)num_pairs, 2), dim3(256), 0, stream,
                     (uint8_t *)k_cache, (uint8_t *)v_cache, pairs, (int64_t)num_blocks,
                     block_chunks);
  return hipGetLastError();
}

}  // namespace pa
