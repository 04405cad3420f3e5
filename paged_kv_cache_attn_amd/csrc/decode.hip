// decode.hip -- paged attention for decode queries on gfx950.
//
// What is computed (Month 2 "PagedAttention" §2.1 and §5.4; Lecture 7 "KV
// Cache Management" §4.2): for sequence b and query head h,
//   out[b][h] = sum_t softmax_t(scale * q[b][h] . K_t) V_t
// over the seq_lens[b] cached tokens of KV head h / g, where token t lives at
// offset t % bs of physical block block_tables[b][t / bs].
//
// How (MI355X design, not the pages' CUDA kernel):
//   * one workgroup per (split-K partition, KV head, sequence); the whole GQA
//     group of g query heads is served by the same workgroup, so each K/V
//     tile is read from HBM once per group, not once per query head;
//   * inside a wave, the g query heads are the 16 "columns" of 16x16 MFMA
//     tiles: S^T = K_blk * Q^T (v_mfma_f32_16x16x32_bf16, K straight from
//     global memory, 16 tokens x 128 dims per block), then
//     O^T += V_blk^T * P^T (v_mfma_f32_16x16x16_bf16); the V^T operand is
//     formed in registers with v_perm from 16-byte row loads, no LDS;
//   * online softmax per column in the exp2 domain (scale*log2e folded in),
//     the running max/sum kept per lane, so the rescale of the output tile
//     needs no lane exchange;
//   * the waves of a workgroup take the partition's blocks round-robin and
//     are merged through LDS; partitions are merged by a second kernel in a
//     fixed order (Lecture 16 "LLM Serving (1)" §3.3: the merge rule of the
//     online softmax), so the result depends only on logical positions and
//     is bit-identical under any physical block permutation.
#include "attn_core.h"
#include "attn_vec.h"
#include "pa_launch.h"

namespace pa {

namespace {

// Vector kernels: waves per workgroup, and query heads served per pass.
constexpr int kVecWaves = 4;

__device__ __forceinline__ void store_out(void *out, int out_bf16, int64_t idx, float v) {
  if (out_bf16) {
    reinterpret_cast<__bf16 *>(out)[idx] = (__bf16)v;
  } else {
    reinterpret_cast<float *>(out)[idx] = v;
  }
}

// ----------------------------------------------------------------------------
// MFMA kernel: bf16 (or FP8 E4M3, FP8) KV with bf16 q, head_dim 128, block
// size 8, 16, 32, 64 or 128 (walked in 16-token tiles), g <= 16.
// Lane (r, c) = (lane >> 4, lane & 15); column c is query head kh*g + c.
// The block size BSZ is a template argument so the table walk folds to
// constants for each supported size.  FP8 tiles travel through the pipeline
// as loaded (half the registers) and are expanded to bf16 just before their
// step; k_scale is folded into the score scale and v_scale into the final
// normalisation.
// ----------------------------------------------------------------------------
template <int NW, int BSZ, bool FP8>
__global__ __launch_bounds__(64 * NW) void decode_mfma_d128_kernel(DecodeParams p) {
  using F = KVFormat<FP8>;
  constexpr int D = 128;
  constexpr int BS = 16;
  const int part = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int g = p.num_heads / p.num_kv_heads;
  const int L = clamp_len(p.seq_lens[b], p.max_len_cap);
  const int nblk = (L + BS - 1) / BS;
  const int nparts = nblk == 0 ? 1 : (nblk + p.part_blocks - 1) / p.part_blocks;
  if (part >= nparts) return;
  const int j0 = part * p.part_blocks;
  const int j1 = min(j0 + p.part_blocks, nblk);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4, c = lane & 15;
  const bool col_ok = c < g;

  bf16x8 qb[4];
  F::load_q(qb,
            col_ok ? reinterpret_cast<const uint16_t *>(p.q) + ((int64_t)b * p.num_heads + (int64_t)kh * g + c) * D
                   : nullptr,
            r);

  const float sl2 = p.scale * p.k_scale * kLog2e;
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
  const typename F::Elem *kc = reinterpret_cast<const typename F::Elem *>(p.k_cache);
  const typename F::Elem *vc = reinterpret_cast<const typename F::Elem *>(p.v_cache);
  const int nblk_tab = (L + BSZ - 1) / BSZ;
  const TileMap map(BSZ, p.num_kv_heads, p.num_blocks);

  MfmaAttnState st;
  st.init();

  // The row's tiles stream through the caches (non-temporal loads) unless
  // the previous or the next sequence starts with the same block (forked or
  // prefix-sharing sequences sit next to each other in a batch): then they
  // are loaded so that they stay in the L2 for those rows.
  bool keep = false;
  if (nblk_tab > 0) {
    const int t0 = table[0];
    if (b > 0 && clamp_len(p.seq_lens[b - 1], p.max_len_cap) > 0) keep |= table[-p.max_blocks_per_seq] == t0;
    if (b + 1 < p.num_seqs && clamp_len(p.seq_lens[b + 1], p.max_len_cap) > 0)
      keep |= table[p.max_blocks_per_seq] == t0;
  }
  const bool stream = !__builtin_amdgcn_readfirstlane((int)keep);

  // 16-token tile j (any supported block size).  An out-of-range table entry
  // is never dereferenced: the tile is read from block 0 and fully masked.
  auto load = [&](int j, typename F::Raw &t, int &lim) {
    int e0, e1;
    const bool ok = map.entries(table, j, nblk_tab, e0, e1);
    debug_report(!ok, kDbgBlockRange);
    lim = ok ? L : 0;
    F::load(t, kc, vc, map.rows(e0, e1, kh), r, c, stream);
  };

  // Two-deep software pipeline: the next tile's loads are in flight while
  // the current one is multiplied.
  int j = j0 + w;
  if (j < j1) {
    typename F::Raw cur;
    int lim;
    load(j, cur, lim);
    while (true) {
      const int jn = j + NW;
      if (jn < j1) {
        typename F::Raw nxt;
        int limn;
        load(jn, nxt, limn);
        st.step(qb, F::expand(cur), j * BS, lim, sl2, r);
        cur = nxt;
        lim = limn;
        j = jn;
      } else {
        st.step(qb, F::expand(cur), j * BS, lim, sl2, r);
        break;
      }
    }
  }
  float m = st.m, l = st.l;
  floatx4 *acc = st.acc;

  // Per-lane l covers this lane's tokens; sum the four rows.
  l = row_sum4(l);
  // acc[jj][i] = O[column c][dim 32r + 8i + jj], relative to max m.

  const int64_t row = (int64_t)b * p.num_heads + (int64_t)kh * g + c;  // valid when col_ok
  if (NW == 1) {
    if (!col_ok) return;
    if (nparts == 1) {
      const float inv = l > 0.f ? p.v_scale / l : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          store_out(p.out, p.out_bf16, row * D + 32 * r + 8 * i + jj, acc[jj][i] * inv);
    } else {
      float *wo = p.ws_o + (row * p.nparts_max + part) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) wo[32 * r + 8 * i + jj] = acc[jj][i];
      if (r == 0) {
        p.ws_ml[(row * p.nparts_max + part) * 2 + 0] = m;
        p.ws_ml[(row * p.nparts_max + part) * 2 + 1] = l;
      }
    }
    return;
  }

  // Merge the NW wave states of this workgroup through LDS.
  __shared__ float sm_o[NW][16][D];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  if (col_ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sm_o[w][c][32 * r + 8 * i + jj] = acc[jj][i];
    if (r == 0) {
      sm_m[w][c] = m;
      sm_l[w][c] = l;
    }
  }
  __syncthreads();
  const int total = g * D;
  for (int idx = threadIdx.x; idx < total; idx += 64 * NW) {
    const int cc = idx / D, d = idx - cc * D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][cc]);
    const float M_use = M == kNegInf ? 0.f : M;
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float wgt = fast_exp2(sm_m[ww][cc] - M_use);
      lsum += sm_l[ww][cc] * wgt;
      o += sm_o[ww][cc][d] * wgt;
    }
    const int64_t rr = (int64_t)b * p.num_heads + (int64_t)kh * g + cc;
    if (nparts == 1) {
      store_out(p.out, p.out_bf16, rr * D + d, lsum > 0.f ? o * p.v_scale / lsum : 0.f);
    } else {
      p.ws_o[(rr * p.nparts_max + part) * D + d] = o;
      if (d == 0) {
        p.ws_ml[(rr * p.nparts_max + part) * 2 + 0] = M;
        p.ws_ml[(rr * p.nparts_max + part) * 2 + 1] = lsum;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Vector kernel: fp32 or bf16 KV, head_dim 64 or 128, any group size and
// block size (the shapes the MFMA kernel does not take).  One workgroup per
// (partition, KV head, sequence) serves the whole GQA group (attn_vec.h), so
// each K/V row of the partition is read once per group, with 16-byte loads.
// ----------------------------------------------------------------------------
template <int D, bool BF16, int GC>
__global__ __launch_bounds__(64 * kVecWaves) void decode_vec_kernel(DecodeParams p) {
  constexpr int NW = kVecWaves;
  using G = VecGeom<D, BF16>;
  __shared__ float red[(NW + 1) * GC * (D + 2)];
  const int part = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int g = p.num_heads / p.num_kv_heads;
  const int bs = p.block_size;
  const int L = clamp_len(p.seq_lens[b], p.max_len_cap);
  const int nblk = (L + bs - 1) / bs;
  const int nparts = nblk == 0 ? 1 : (nblk + p.part_blocks - 1) / p.part_blocks;
  if (part >= nparts) return;  // the whole workgroup leaves together
  const int t0 = part * p.part_blocks * bs;
  const int t1 = min(L, t0 + p.part_blocks * bs);
  const int col = ((threadIdx.x & 63) % G::kLPR) * G::kVPL;
  const float sl2 = p.scale * kLog2e;
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
  const uint8_t *qb = reinterpret_cast<const uint8_t *>(p.q);
  for (int h0 = 0; h0 < g; h0 += GC) {
    float q[GC][G::kVPL];
#pragma unroll
    for (int hh = 0; hh < GC; ++hh) {
      const int h = kh * g + min(h0 + hh, g - 1);  // heads past the group repeat the last one, unused
      const uint8_t *qr = qb + (((int64_t)b * p.num_heads + h) * D + col) * G::kElem;
#pragma unroll
      for (int c = 0; c < G::kCPL; ++c) unpack16<BF16>(ld16(qr + 16 * c), &q[hh][c * (G::kVPL / G::kCPL)]);
    }
    const float *res = vec_attend<D, BF16, NW, GC>(red, q, p.k_cache, p.v_cache, table, t0, t1, kh,
                                                   p.num_kv_heads, bs, p.num_blocks, sl2);
    for (int idx = threadIdx.x; idx < GC * D; idx += 64 * NW) {
      const int hh = idx / D, d = idx - hh * D;
      if (h0 + hh >= g) continue;
      const float *e = res + hh * (D + 2);
      const int64_t row = (int64_t)b * p.num_heads + (int64_t)kh * g + h0 + hh;
      if (nparts == 1) {
        store_out(p.out, p.out_bf16, row * D + d, e[D + 1] > 0.f ? e[d] / e[D + 1] : 0.f);
      } else {
        p.ws_o[(row * p.nparts_max + part) * D + d] = e[d];
        if (d == 0) {
          p.ws_ml[(row * p.nparts_max + part) * 2 + 0] = e[D];
          p.ws_ml[(row * p.nparts_max + part) * 2 + 1] = e[D + 1];
        }
      }
    }
    __syncthreads();  // the next chunk of heads reuses `red`
  }
}

// ----------------------------------------------------------------------------
// Partition merge: one workgroup per (query head, sequence), one thread per
// output dim; partitions combined in ascending order.  The (max, sum) pairs
// are staged in LDS once and the partial outputs fetched in batches of eight
// independent loads, so the merge costs a few memory latencies, not one per
// partition.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
  constexpr int kChunk = 256;
  __shared__ float s_m[kChunk];
  __shared__ float s_w[kChunk];
  __shared__ float s_red[128];
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(p.seq_lens[b], p.max_len_cap);
  const int nblk = (L + p.tile_tokens - 1) / p.tile_tokens;
  const int nparts = nblk == 0 ? 1 : (nblk + p.part_blocks - 1) / p.part_blocks;
  if (nparts <= 1) return;
  const int64_t row = (int64_t)b * p.num_heads + h;
  const float *ml = p.ws_ml + row * p.nparts_max * 2;
  const float *wo = p.ws_o + row * p.nparts_max * p.head_dim;
  const int tid = threadIdx.x;
  // global max over partitions
  float M = kNegInf;
  for (int q = tid; q < nparts; q += blockDim.x) M = fmaxf(M, ml[2 * q]);
  s_red[tid] = M;
  __syncthreads();
  for (int off = 64; off > 0; off >>= 1) {
    if (tid < off) s_red[tid] = fmaxf(s_red[tid], s_red[tid + off]);
    __syncthreads();
  }
  const float M_use = s_red[0] == kNegInf ? 0.f : s_red[0];
  __syncthreads();
  float lsum = 0.f;
  float acc[2] = {0.f, 0.f};  // head_dim <= 2 * 128 threads... dims tid and tid + 128
  for (int q0 = 0; q0 < nparts; q0 += kChunk) {
    const int n = min(kChunk, nparts - q0);
    for (int q = tid; q < n; q += blockDim.x) {
      const float wgt = fast_exp2(ml[2 * (q0 + q)] - M_use);
      s_w[q] = wgt;
      s_m[q] = ml[2 * (q0 + q) + 1] * wgt;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int d = tid + u * 128;
      if (d < p.head_dim) {
        float o = 0.f;
        for (int k0 = 0; k0 < n; k0 += 8) {
          float v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = wo[(int64_t)(q0 + min(k0 + k, n - 1)) * p.head_dim + d];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k0 + k < n) o += v[k] * s_w[k0 + k];
        }
        acc[u] += o;
      }
    }
    for (int q = 0; q < n; ++q) lsum += s_m[q];
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int d = tid + u * 128;
    if (d < p.head_dim)
      store_out(p.out, p.out_bf16, row * p.head_dim + d, lsum > 0.f ? acc[u] * p.v_scale / lsum : 0.f);
  }
}

// The vector kernel with the head chunk GC that fits the group: the group
// size rounded up to a power of two, at most 8.
template <int D, bool BF16, class Params>
void launch_vec(dim3 grid, dim3 block, hipStream_t stream, const Params &p) {
  const int g = p.num_heads / p.num_kv_heads;
  if (g <= 1)
    hipLaunchKernelGGL((decode_vec_kernel<D, BF16, 1>), grid, block, 0, stream, p);
  else if (g <= 2)
    hipLaunchKernelGGL((decode_vec_kernel<D, BF16, 2>), grid, block, 0, stream, p);
  else if (g <= 4)
    hipLaunchKernelGGL((decode_vec_kernel<D, BF16, 4>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_vec_kernel<D, BF16, 8>), grid, block, 0, stream, p);
}

}  // namespace

#if PAGED_ATTN_DEBUG
PA_DEBUG_WORD_ACCESSOR(debug_word_decode)
#endif

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
  const int g = p.num_heads / p.num_kv_heads;
  const bool mfma = (p.kv_bf16 || p.kv_fp8) && p.head_dim == 128 && mfma_block_size(p.block_size) && g <= 16;
  if (p.num_seqs == 0) return hipSuccess;
  if (mfma) {
    const dim3 grid(p.nparts_max, p.num_kv_heads, p.num_seqs), block(64 * PA_DECODE_WAVES);
    constexpr int NW = PA_DECODE_WAVES;
    if (p.kv_fp8) {
      switch (p.block_size) {
        case 8: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 8, true>), grid, block, 0, stream, p); break;
        case 16: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 16, true>), grid, block, 0, stream, p); break;
        case 32: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 32, true>), grid, block, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 64, true>), grid, block, 0, stream, p); break;
        default: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 128, true>), grid, block, 0, stream, p); break;
      }
    } else {
      switch (p.block_size) {
        case 8: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 8, false>), grid, block, 0, stream, p); break;
        case 16: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 16, false>), grid, block, 0, stream, p); break;
        case 32: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 32, false>), grid, block, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 64, false>), grid, block, 0, stream, p); break;
        default: hipLaunchKernelGGL((decode_mfma_d128_kernel<NW, 128, false>), grid, block, 0, stream, p); break;
      }
    }
  } else {
    const dim3 grid(p.nparts_max, p.num_kv_heads, p.num_seqs), block(64 * kVecWaves);
    if (p.head_dim == 64) {
      if (p.kv_bf16)
        launch_vec<64, true>(grid, block, stream, p);
      else
        launch_vec<64, false>(grid, block, stream, p);
    } else {
      if (p.kv_bf16)
        launch_vec<128, true>(grid, block, stream, p);
      else
        launch_vec<128, false>(grid, block, stream, p);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nparts_max <= 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(p.num_heads, p.num_seqs), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
