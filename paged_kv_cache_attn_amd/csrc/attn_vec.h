// attn_vec.h -- attention on the vector ALUs for the shapes the MFMA kernels
// do not take (fp32 K/V, head_dim 64, other block sizes, large or odd GQA
// groups): one workgroup serves every query head of one KV head, so each K/V
// row is read from memory once per group, not once per query head.
//
// Per (sequence or query row, KV head): out[h] = sum_t softmax_t(scale *
// q[h] . K_t) V_t over the row's keys [t0, t1) (Month 2 "PagedAttention"
// §2.1 and §5.4: token t sits at offset t % bs of physical block
// block_tables[b][t / bs]).
//
// Lane layout.  A K or V row of D elements is read by LPR = D * elem / 32
// lanes, two 16-byte loads each (lane j of the row holds elements
// j*VPL .. j*VPL + VPL - 1), so a wave reads 64 / LPR rows per pair of load
// instructions, whole rows.  Those LPR lanes form a token slot:
// slot k of wave w takes the row's tokens t0 + (w * SLOTS + k) + i * NW *
// SLOTS, i = 0, 1, ...  The q . k dot product of every head is summed over
// the slot's lanes (DPP row operations); each slot keeps its own online
// softmax (running max, running sum, unnormalised output of its elements)
// per head, in the exp2 domain, updated once per batch of tokens.  At the end the slots of a wave are merged by a
// butterfly of xor shuffles (the merge rule of Lecture 16 "LLM Serving (1)"
// §3.3; both partners compute the same sums, since float addition is
// commutative) and the waves through LDS in ascending order.  Every order
// depends only on logical token positions, so results are bit-identical
// under any physical block permutation.
//
// Heads are processed GC at a time (GC: the group size rounded up to a power
// of two, at most 8; q and the output of GC heads live in registers); a
// group larger than 8 walks the keys again per chunk of 8 heads, reading
// them from the L2.
#pragma once

#include "pa_device.h"

namespace pa {

template <int D, bool BF16>
struct VecGeom {
  static constexpr int kElem = BF16 ? 2 : 4;
  static constexpr int kCPL = 2;                  // 16-byte chunks per lane per row
  static constexpr int kVPL = kCPL * 16 / kElem;  // elements per lane per row
  static constexpr int kLPR = D / kVPL;           // lanes per row
  static constexpr int kSlots = 64 / kLPR;        // rows a wave reads per load instruction
  static_assert(kLPR >= 2 && kLPR <= 32 && 64 % kLPR == 0, "row must span 2..32 lanes");
};

// The kVPL values of a 16-byte chunk as floats (bf16 widens exactly).
template <bool BF16>
__device__ __forceinline__ void unpack16(const u32x4 &w, float *x) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
}

// Sum over the N lanes of an aligned lane group (N = 2 .. 32), the same
// bits in every lane of the group: DPP within a row of 16 lanes (swap of
// neighbours, of neighbouring pairs, mirror within 8, mirror within 16),
// then the row swap of v_permlane16_swap for 32.  Each step adds the
// partner's value to the lane's own, which gives both partners the same sum
// (float addition is commutative).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  if constexpr (N >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  if constexpr (N >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  if constexpr (N >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  if constexpr (N >= 32) {
    float b;
    const float a = xor16_first(v, b);
    v = a + b;
  }
  return v;
}

// One workgroup's attention for GC heads over keys [t0, t1) of one
// (sequence, KV head).  Returns the LDS area res where, for head h < GC,
// res[h * (D + 2) + d] is the unnormalised output o[d] (d < D), res[.. + D]
// the max (log2 units, -inf for no keys) and res[.. + D + 1] the sum of
// weights, merged over the whole workgroup; readable on return.  `red`
// must hold (NW + 1) * GC * (D + 2) floats.  Every thread of the workgroup
// calls this (it holds barriers).
template <int D, bool BF16, int NW, int GC>
__device__ __forceinline__ float *vec_attend(float *red, const float (&q)[GC][VecGeom<D, BF16>::kVPL],
                                           const void *k_cache, const void *v_cache, const int32_t *table,
                                           int t0, int t1, int kh, int num_kv_heads, int bs, int num_blocks,
                                           float sl2) {
  using G = VecGeom<D, BF16>;
  constexpr int VPL = G::kVPL, LPR = G::kLPR, SLOTS = G::kSlots, CPL = G::kCPL;
  constexpr int STRIDE = NW * SLOTS;  // tokens the workgroup reads per step
  constexpr int U = 2;                // tokens of a slot per batch
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int slot = w * SLOTS + lane / LPR;
  const int col = (lane % LPR) * VPL;  // first element of this lane in a row
  const uint8_t *kc = reinterpret_cast<const uint8_t *>(k_cache);
  const uint8_t *vc = reinterpret_cast<const uint8_t *>(v_cache);
  const int64_t row_bytes = (int64_t)D * G::kElem;
  const int64_t col_bytes = (int64_t)col * G::kElem;

  float m[GC], l[GC], acc[GC][VPL];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) acc[h][j] = 0.f;
  }

  // The slot's tokens go in batches of U: batch k is tokens t0 + slot +
  // (k * U + u) * STRIDE, u < U.  The K/V chunks of batch k + 1 are in flight
  // while batch k is used, and the block-table entries of batch k + 2 while
  // those load, so no load waits on a table read of its own iteration.
  // Every load is issued whatever the token: a token past t1 reads the
  // table entry of the range's last token, and a masked token (past t1, or
  // with a block id out of range) reads row t % bs of block 0.  Its score is
  // masked and its V values are taken as zeros, so what it read never
  // counts.  (A load skipped on some paths would make the compiler's wait
  // counting, which merges the paths, wait for every load in flight before
  // each batch, the next batch's included.)
  struct KV {
    u32x4 k[U][CPL], v[U][CPL];
    bool ok[U];  // the token is in range and its block id valid
  };
  auto tok = [&](int k, int u) { return t0 + slot + (k * U + u) * STRIDE; };
  // raw table entries only: they are tested where the K/V loads use them, a
  // batch later, so nothing waits for them here
  auto load_table = [&](int k, int (&ent)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) ent[u] = table[min(tok(k, u), t1 - 1) / bs];  // t1 > t0 + slot here
  };
  auto load_kv = [&](int k, const int (&ent)[U], KV &kv) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tok(k, u);
      debug_report(t < t1 && (unsigned)ent[u] >= (unsigned)num_blocks, kDbgBlockRange);
      kv.ok[u] = t < t1 && (unsigned)ent[u] < (unsigned)num_blocks;
      const int e = kv.ok[u] ? ent[u] : 0;
      const int64_t off = (((int64_t)e * num_kv_heads + kh) * bs + (t % bs)) * row_bytes + col_bytes;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        kv.k[u][c] = ld16(kc + off + 16 * c);
        kv.v[u][c] = ld16(vc + off + 16 * c);
      }
    }
  };
  // One batch: the U scores of every head first, then one max update and
  // rescale per head for the whole batch (the online-softmax rule of Month
  // 2 "PagedAttention" §5.4, applied to U keys at a time).
  auto step = [&](const KV &kv) {
    float kx[U][VPL];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) unpack16<BF16>(kv.k[u][c], &kx[u][c * (VPL / CPL)]);
    float x[GC][U];
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float sdot = 0.f;
#pragma unroll
        for (int j = 0; j < VPL; ++j) sdot = __builtin_fmaf(q[h][j], kx[u][j], sdot);
        sdot = group_sum<LPR>(sdot);  // every lane of the slot: the whole dot product
        x[h][u] = kv.ok[u] ? sdot * sl2 : kNegInf;
      }
    float vx[U][VPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) unpack16<BF16>(kv.v[u][c], &vx[u][c * (VPL / CPL)]);
#pragma unroll
      for (int j = 0; j < VPL; ++j) vx[u][j] = kv.ok[u] ? vx[u][j] : 0.f;  // a masked token adds 0 * 0
    }
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      float mx = x[h][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, x[h][u]);
      const float m_new = fmaxf(m[h], mx);
      if (m_new == kNegInf) continue;  // nothing seen yet and nothing new
      const float corr = fast_exp2(m[h] - m_new);  // 0 while m is -inf
      float e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) e[u] = fast_exp2(x[h][u] - m_new);  // 0 for a masked token
      float es = e[0];
#pragma unroll
      for (int u = 1; u < U; ++u) es += e[u];
      l[h] = __builtin_fmaf(l[h], corr, es);
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        float a = acc[h][j] * corr;
#pragma unroll
        for (int u = 0; u < U; ++u) a = __builtin_fmaf(e[u], vx[u][j], a);
        acc[h][j] = a;
      }
      m[h] = m_new;
    }
  };

  // Two fixed K/V register sets used in turn (no register of a load in
  // flight is ever copied), table entries of batches k, k + 1, k + 2 in p0,
  // p1, p2.  The loop has one exit, at the bottom: each turn loads the next
  // two batches whether or not they exist, so every path issues the same
  // loads and each step waits for its own batch only.  A batch past the
  // slot's last one is fully masked: it reads rows of block 0 and its step
  // changes nothing (the max stays, the correction is exp2(0) = 1, every
  // weight is 0), so the result is that of stopping at the last batch.
  const int nbatch = t1 > t0 + slot ? (t1 - t0 - slot + U * STRIDE - 1) / (U * STRIDE) : 0;
  if (nbatch > 0) {
    KV kv0, kv1;
    int p0[U], p1[U], p2[U];
    load_table(0, p0);
    load_table(1, p1);
    load_kv(0, p0, kv0);
    for (int k = 0; k < nbatch; k += 2) {
      // (the scheduling barriers keep each step's arithmetic, which waits
      // for its batch, from moving above the next batch's loads)
      load_table(k + 2, p2);
      load_kv(k + 1, p1, kv1);
      __builtin_amdgcn_sched_barrier(0);
      step(kv0);
      load_table(k + 3, p0);
      load_kv(k + 2, p2, kv0);
      __builtin_amdgcn_sched_barrier(0);
      step(kv1);
#pragma unroll
      for (int u = 0; u < U; ++u) {  // batch k + 2's entries to p0, k + 3's to p1
        const int t = p0[u];
        p0[u] = p2[u];
        p1[u] = t;
      }
    }
  }

  // merge the slots of this wave: butterfly over the slot bits of the lane id
#pragma unroll
  for (int mask = LPR; mask < 64; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      const float mo = __shfl_xor(m[h], mask, 64), lo = __shfl_xor(l[h], mask, 64);
      const float M = fmaxf(m[h], mo);
      const float Mu = M == kNegInf ? 0.f : M;
      const float wa = fast_exp2(m[h] - Mu), wb = fast_exp2(mo - Mu);
      l[h] = l[h] * wa + lo * wb;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const float ao = __shfl_xor(acc[h][j], mask, 64);
        acc[h][j] = acc[h][j] * wa + ao * wb;
      }
      m[h] = M;
    }
  }
  // then the waves, through LDS, in ascending order, into the result area
  // after the NW wave entries (no entry is overwritten while it is read)
  float *mine = red + (size_t)w * GC * (D + 2);
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < GC; ++h) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) mine[h * (D + 2) + col + j] = acc[h][j];
      if (lane == 0) {
        mine[h * (D + 2) + D] = m[h];
        mine[h * (D + 2) + D + 1] = l[h];
      }
    }
  }
  __syncthreads();
  float *res = red + (size_t)NW * GC * (D + 2);
  for (int idx = threadIdx.x; idx < GC * (D + 2); idx += 64 * NW) {
    const int h = idx / (D + 2), d = idx - h * (D + 2);
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red[(ww * GC + h) * (D + 2) + D]);
    const float Mu = M == kNegInf ? 0.f : M;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float *e = red + (ww * GC + h) * (D + 2);
      v += e[d == D ? D + 1 : d] * fast_exp2(e[D] - Mu);  // (d == D: a placeholder, replaced by M)
    }
    res[idx] = d == D ? M : v;
  }
  __syncthreads();
  return res;
}

}  // namespace pa
