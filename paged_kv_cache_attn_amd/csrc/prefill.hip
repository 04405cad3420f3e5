// prefill.hip -- causal attention of a chunk of new queries over the paged
// cache (cached prefix + the chunk itself) on gfx950.
//
// What is computed (Lecture 27 "Better KV Caches" §1.1: the new tokens'
// queries attend directly to the cached K/V; Lecture 7 "KV Cache Management"
// §8.3: only the uncached suffix is computed): sequence b has seq_lens[b]
// tokens in the cache after its chunk of n_b rows was written; chunk row i
// sits at position pos = seq_lens[b] - n_b + i and attends to tokens
// 0 .. pos through the block table.
//
// MFMA kernel: one wave serves 16 columns = (16 / g) consecutive chunk
// tokens x the g query heads of one KV head, so every K/V tile it reads is
// shared by the whole GQA group; key blocks are visited in ascending order
// with a per-column causal bound (the same tile step as decode).
#include "attn_core.h"
#include "pa_launch.h"

namespace pa {

namespace {

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

__device__ __forceinline__ void store_out(void *out, int out_bf16, int64_t idx, float v) {
  if (out_bf16) {
    reinterpret_cast<__bf16 *>(out)[idx] = (__bf16)v;
  } else {
    reinterpret_cast<float *>(out)[idx] = v;
  }
}

// bf16 KV, head_dim 128, block_size 16, g in {1, 2, 4, 8, 16}.
// grid = (ceil(max_query_len / (16 / g)), Hkv, B), one wave per workgroup.
__global__ __launch_bounds__(64) void prefill_mfma_d128_kernel(PrefillParams p) {
  constexpr int D = 128;
  constexpr int BS = 16;
  const int tile = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int g = p.num_heads / p.num_kv_heads;
  const int tpw = 16 / g;  // chunk tokens per wave
  const int q0 = p.query_start_loc[b];
  const int n_b = p.query_start_loc[b + 1] - q0;
  if (tile * tpw >= n_b) return;
  const int S = clamp_len(p.seq_lens[b], p.max_len_cap);

  const int lane = threadIdx.x & 63;
  const int r = lane >> 4, c = lane & 15;
  const int ti = c / g, hh = c - (c / g) * g;
  const int qi = tile * tpw + ti;  // row inside the chunk
  const bool col_ok = ti < tpw && qi < n_b && q0 >= 0 && (int64_t)q0 + qi < p.num_query_tokens;
  const int lim = col_ok ? S - n_b + qi + 1 : 0;  // keys < lim are visible
  const int last_qi = min(tile * tpw + tpw, n_b) - 1;
  int kend = S - n_b + last_qi + 1;  // wave-wide key bound
  kend = kend < 0 ? 0 : kend;
  const int nblk = (kend + BS - 1) / BS;

  bf16x8 qb[4];
  load_q_operand_d128(qb,
                      col_ok ? reinterpret_cast<const uint16_t *>(p.q) +
                                   ((int64_t)(q0 + qi) * p.num_heads + (int64_t)kh * g + hh) * D
                             : nullptr,
                      r);

  const float sl2 = p.scale * kLog2e;
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
  const uint16_t *kbase = reinterpret_cast<const uint16_t *>(p.k_cache) + (int64_t)kh * BS * D;
  const uint16_t *vbase = reinterpret_cast<const uint16_t *>(p.v_cache) + (int64_t)kh * BS * D;
  const int64_t blk_stride = (int64_t)p.num_kv_heads * BS * D;

  MfmaAttnState st;
  st.init();
  auto load = [&](int j, KVTile &t, bool &ok) {
    int phys = table[j];
    ok = (unsigned)phys < (unsigned)p.num_blocks;
    phys = ok ? phys : 0;
    load_kv_tile_d128(t, kbase + phys * blk_stride, vbase + phys * blk_stride, r, c);
  };
  if (nblk > 0) {
    KVTile cur;
    bool ok;
    load(0, cur, ok);
    for (int j = 0;; ++j) {
      if (j + 1 < nblk) {
        KVTile nxt;
        bool okn;
        load(j + 1, nxt, okn);
        st.step(qb, cur, j * BS, ok ? lim : 0, sl2, r);
        cur = nxt;
        ok = okn;
      } else {
        st.step(qb, cur, j * BS, ok ? lim : 0, sl2, r);
        break;
      }
    }
  }
  const float l = row_sum4(st.l);
  if (!col_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t row = (int64_t)(q0 + qi) * p.num_heads + (int64_t)kh * g + hh;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      store_out(p.out, p.out_bf16, row * D + 32 * r + 8 * i + jj, st.acc[jj][i] * inv);
}

// Generic VALU kernel: any dtype / head_dim 64 or 128 / group size / block
// size.  One wave per (chunk row, query head, sequence).
template <int D, bool BF16>
__global__ __launch_bounds__(64) void prefill_valu_kernel(PrefillParams p) {
  constexpr int DPL = D / 64;
  const int qi = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int q0 = p.query_start_loc[b];
  const int n_b = p.query_start_loc[b + 1] - q0;
  if (qi >= n_b || q0 < 0 || (int64_t)q0 + qi >= p.num_query_tokens) return;
  const int g = p.num_heads / p.num_kv_heads;
  const int kh = h / g;
  const int bs = p.block_size;
  const int S = clamp_len(p.seq_lens[b], p.max_len_cap);
  int nkeys = S - n_b + qi + 1;
  nkeys = nkeys < 0 ? 0 : (nkeys > S ? S : nkeys);
  const int lane = threadIdx.x;
  auto ld = [&](const void *base, int64_t idx) -> float {
    if (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t *>(base)[idx]);
    return reinterpret_cast<const float *>(base)[idx];
  };
  const int64_t row = (int64_t)(q0 + qi) * p.num_heads + h;
  float qv[DPL], acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    qv[i] = ld(p.q, row * D + lane * DPL + i);
    acc[i] = 0.f;
  }
  const float sl2 = p.scale * kLog2e;
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
  float m = kNegInf, l = 0.f;
  for (int t = 0; t < nkeys; ++t) {
    const int phys = table[t / bs];
    if ((unsigned)phys >= (unsigned)p.num_blocks) continue;
    const int64_t base = (((int64_t)phys * p.num_kv_heads + kh) * bs + t % bs) * D + lane * DPL;
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) dot += qv[i] * ld(p.k_cache, base + i);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) dot += __shfl_xor(dot, s, 64);
    const float x = dot * sl2;
    const float m_new = fmaxf(m, x);
    const float corr = fast_exp2(m - m_new);
    const float e = fast_exp2(x - m_new);
    l = l * corr + e;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = acc[i] * corr + e * ld(p.v_cache, base + i);
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) store_out(p.out, p.out_bf16, row * D + lane * DPL + i, acc[i] * inv);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_query_len == 0) return hipSuccess;
  const int g = p.num_heads / p.num_kv_heads;
  const bool mfma = p.kv_bf16 && p.head_dim == 128 && p.block_size == 16 && g <= 16 && (16 % g) == 0;
  if (mfma) {
    const int tpw = 16 / g;
    dim3 grid((p.max_query_len + tpw - 1) / tpw, p.num_kv_heads, p.num_seqs);
    hipLaunchKernelGGL(prefill_mfma_d128_kernel, grid, dim3(64), 0, stream, p);
  } else {
    dim3 grid(p.max_query_len, p.num_heads, p.num_seqs);
    if (p.head_dim == 64) {
      if (p.kv_bf16)
        hipLaunchKernelGGL((prefill_valu_kernel<64, true>), grid, dim3(64), 0, stream, p);
      else
        hipLaunchKernelGGL((prefill_valu_kernel<64, false>), grid, dim3(64), 0, stream, p);
    } else {
      if (p.kv_bf16)
        hipLaunchKernelGGL((prefill_valu_kernel<128, true>), grid, dim3(64), 0, stream, p);
      else
        hipLaunchKernelGGL((prefill_valu_kernel<128, false>), grid, dim3(64), 0, stream, p);
    }
  }
  return hipGetLastError();
}

}  // namespace pa
