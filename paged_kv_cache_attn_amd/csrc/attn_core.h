// attn_core.h -- one wave's attention over 16-token KV blocks on MFMA (gfx950).
//
// A wave serves 16 query "columns" at once (the GQA group of one decode
// token, or several chunk tokens x the group in prefill).  Per 16-token
// block of one KV head (bf16, head_dim 128, 4 KB of K and 4 KB of V):
//   S^T[token][col] = K_blk . Q^T      4 x v_mfma_f32_16x16x32_bf16
//   online softmax per column (the pages' rescale rule, Month 2
//   "PagedAttention" §5.4), in the exp2 domain
//   O^T[dim][col] += V_blk^T . P^T     16 x v_mfma_f32_16x16x16_bf16 (P as
//                                      bf16 hi + lo parts)
// Operand placement (lane = 16r + c):
//   K: lane loads token c, dims 32i + 8r .. +7 (i = 0..3): A of the QK MFMA;
//   Q: lane holds column c, the same dims: B of the QK MFMA;
//   S: lane receives tokens 4r .. 4r+3 of column c, which is exactly the
//      P^T (B) operand layout of the 16x16x16 PV MFMA;
//   V: lane loads tokens 4r + v (v = 0..3), dims 8c .. 8c+7, i.e. whole
//      256-byte rows per instruction; v_perm regroups them into the V^T (A)
//      operand {V[4r+v][8c + jj]}_v for jj = 0..7;
//   O: acc[jj][i] = O[column c][dim 32r + 8i + jj].
// Every quantity a column needs (its max, its sum, its correction factor)
// lives in the lanes of that column, so only the block max crosses rows.
#pragma once

#include "pa_device.h"

namespace pa {

struct KVTile {
  u32x4 k[4];
  u32x4 v[4];
};

// kt, vt: start of one (block, head) tile, [16][128] bf16 each.
__device__ __forceinline__ void load_kv_tile_d128(KVTile &t, const uint16_t *kt, const uint16_t *vt,
                                                  int r, int c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) t.k[i] = ld16(kt + c * 128 + 32 * i + 8 * r);
#pragma unroll
  for (int v = 0; v < 4; ++v) t.v[v] = ld16(vt + (4 * r + v) * 128 + 8 * c);
}

// -- 16-token tiles over any block size ---------------------------------------
// The kernels walk a (sequence, KV head) row in tiles of 16 consecutive
// tokens whatever the cache's block size bs (M2 "PagedAttention" §5.3; the
// cache is [num_blocks][Hkv][bs][128]).  With bs a multiple of 16, tile j lies
// in block j / (bs / 16), starting at row (j mod (bs / 16)) * 16.  With bs = 8
// its first eight tokens are block 2j and the last eight block 2j + 1.  A tile
// is described by two table-derived entries e0, e1:
//   bs >= 16: e0 = physical block, e1 = sub-tile index inside it;
//   bs == 8:  e0, e1 = physical blocks of its two halves.
// An entry out of range is replaced by block 0 and reported to the caller,
// which masks the tile instead of dereferencing it (and, in the debug build,
// records it).  nblk_tab = ceil(L / bs) is the
// number of table entries the row uses; the second half of a bs = 8 tile past
// it is never read (its tokens are past L and masked).
struct TileRows {
  int64_t lo, hi;  // element offsets (from the cache base) of the tile's rows 0 and 8
};
struct TileMap {
  int sh;        // log2(bs / 16) for bs >= 16, -1 for bs == 8
  int num_blocks;
  int hstride;   // elements of one KV head inside a block (bs * 128)
  int blk;       // elements of one physical block (all KV heads; < 2^31 by the host checks)
  __device__ __forceinline__ TileMap(int bs, int num_kv_heads, int nb) {
    constexpr int D = 128;
    sh = bs >= 16 ? __builtin_ctz((unsigned)bs) - 4 : -1;
    num_blocks = nb;
    hstride = bs * D;
    blk = num_kv_heads * hstride;
  }
  // (TablePtr: a generic or a constant-address-space pointer to int32 entries.)
  // Branch-free: both table reads are issued for every block size (for
  // bs >= 16 the second one repeats the first address), so a loop that calls
  // this stays one basic block.
  // Table index of the (first) entry that tile j lives in.
  __device__ __forceinline__ int first_index(int j) const { return sh < 0 ? 2 * j : j >> (sh & 31); }
  // the table indices of tile j's entries
  __device__ __forceinline__ void indices(int j, int nblk_tab, int &i0, int &i1) const {
    const bool halves = sh < 0;
    i0 = halves ? 2 * j : j >> (sh & 31);
    i1 = halves && 2 * j + 1 < nblk_tab ? 2 * j + 1 : i0;
  }
  // tile j's entries from the table values t0, t1 read at those indices
  __device__ __forceinline__ bool entries_from(int t0, int t1, int j, int &e0, int &e1) const {
    const bool halves = sh < 0;
    const bool ok = (unsigned)t0 < (unsigned)num_blocks && (!halves || (unsigned)t1 < (unsigned)num_blocks);
    e0 = ok ? t0 : 0;
    e1 = halves ? (ok ? t1 : 0) : j & ((1 << (sh & 31)) - 1);
    return ok;
  }
  template <typename TablePtr>
  __device__ __forceinline__ bool entries(TablePtr table, int j, int nblk_tab, int &e0, int &e1) const {
    int i0, i1;
    indices(j, nblk_tab, i0, i1);
    return entries_from(table[i0], table[i1], j, e0, e1);
  }
  // the rows of the tile with entries e0, e1 in KV head kh (32-bit selects
  // only, then one multiply-add per row, so nothing here becomes a branch)
  __device__ __forceinline__ TileRows rows(int e0, int e1, int kh) const {
    constexpr int D = 128;
    const int head = kh * hstride;
    const bool halves = sh < 0;
    const int blk_hi = halves ? e1 : e0;
    const int off_lo = halves ? head : head + e1 * 16 * D;
    const int off_hi = halves ? head : off_lo + 8 * D;
    return {(int64_t)e0 * blk + off_lo, (int64_t)blk_hi * blk + off_hi};
  }
};

// The operands of one tile (see load_kv_tile_d128) from its two row bases.
// `stream` (wave-uniform) picks non-temporal loads, for a tile no other row
// of the call reads, over ordinary ones, which leave it in the L2 for the
// rows that share its block.
__device__ __forceinline__ void load_kv_tile_rows(KVTile &t, const uint16_t *kc, const uint16_t *vc,
                                                  const TileRows &tr, int r, int c, bool stream) {
  const int64_t kr = (c < 8 ? tr.lo : tr.hi) + (c & 7) * 128;
  const int64_t vr = r < 2 ? tr.lo : tr.hi;  // tokens 4r .. 4r+3 share a half
  if (stream) {
    // (the empty statements keep the compiler from merging the two load
    // sequences into one, which would drop the non-temporal hint)
    asm volatile("");
#pragma unroll
    for (int i = 0; i < 4; ++i) t.k[i] = ld16_stream(kc + kr + 32 * i + 8 * r);
#pragma unroll
    for (int v = 0; v < 4; ++v) t.v[v] = ld16_stream(vc + vr + ((4 * r + v) & 7) * 128 + 8 * c);
    asm volatile("");
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) t.k[i] = ld16(kc + kr + 32 * i + 8 * r);
#pragma unroll
    for (int v = 0; v < 4; ++v) t.v[v] = ld16(vc + vr + ((4 * r + v) & 7) * 128 + 8 * c);
  }
}

// The tile of load_kv_tile_rows with token `tpos` (0 .. 15; -1: none) read
// from the rows nk, nv (one K row and one V row of 128 bf16) instead of the
// cache: the lanes that hold that token take their addresses from those
// rows, so every register is still filled by exactly one load and every
// tile issues the same load sequence.  STREAM picks the load kind.
template <bool STREAM>
__device__ __forceinline__ void load_kv_tile_rows_subst_as(KVTile &t, const uint16_t *kc, const uint16_t *vc,
                                                           const TileRows &tr, int r, int c, int tpos,
                                                           const uint16_t *nk, const uint16_t *nv) {
  const uint16_t *krow = c == tpos ? nk : kc + (c < 8 ? tr.lo : tr.hi) + (c & 7) * 128;
  const int64_t vr = r < 2 ? tr.lo : tr.hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) t.k[i] = STREAM ? ld16_stream(krow + 32 * i + 8 * r) : ld16(krow + 32 * i + 8 * r);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint16_t *vrow = 4 * r + v == tpos ? nv : vc + vr + ((4 * r + v) & 7) * 128;
    t.v[v] = STREAM ? ld16_stream(vrow + 8 * c) : ld16(vrow + 8 * c);
  }
}

// -- FP8 (E4M3) tiles ------------------------------------------------------------
// A tile as loaded from an FP8 cache (rows of 128 bytes): lane (r, c) holds
// K[token c][bytes 16r .. 16r+15] and [64+16r .. 64+16r+15] (two 16-byte
// loads; each instruction reads 64 contiguous bytes of all 16 rows), and
// V[token 4r+v][dims 8c .. 8c+7] (8-byte loads, whole rows per instruction).
// expand() turns it into the bf16 tile the MFMA step takes, exactly.  The K
// dims a lane holds are a permutation of the bf16 tile's (chunk i covers
// dims 64(i/2) + 16r + 8(i%2) .. +7); the QK product sums over all dims, so
// the q operand is loaded with the same permutation (load_q_operand_fp8k).
struct KVTile8 {
  u32x4 k[2];
  u32x2 v[4];
};

__device__ __forceinline__ void load_kv_tile_rows_fp8(KVTile8 &t, const uint8_t *kc, const uint8_t *vc,
                                                      const TileRows &tr, int r, int c, bool stream) {
  const int64_t kr = (c < 8 ? tr.lo : tr.hi) + (c & 7) * 128 + 16 * r;
  const int64_t vr = r < 2 ? tr.lo : tr.hi;
  if (stream) {
    asm volatile("");  // see load_kv_tile_rows
    t.k[0] = ld16_stream(kc + kr);
    t.k[1] = ld16_stream(kc + kr + 64);
#pragma unroll
    for (int v = 0; v < 4; ++v) t.v[v] = ld8_stream(vc + vr + ((4 * r + v) & 7) * 128 + 8 * c);
    asm volatile("");
  } else {
    t.k[0] = ld16(kc + kr);
    t.k[1] = ld16(kc + kr + 64);
#pragma unroll
    for (int v = 0; v < 4; ++v) t.v[v] = ld8(vc + vr + ((4 * r + v) & 7) * 128 + 8 * c);
  }
}

// The same loads with the load kind a template argument, for a loop that
// fixes it for a whole share: one load sequence, no branch between two.
template <bool STREAM>
__device__ __forceinline__ void load_kv_tile_rows_fp8_as(KVTile8 &t, const uint8_t *kc, const uint8_t *vc,
                                                         const TileRows &tr, int r, int c) {
  const int64_t kr = (c < 8 ? tr.lo : tr.hi) + (c & 7) * 128 + 16 * r;
  const int64_t vr = r < 2 ? tr.lo : tr.hi;
  t.k[0] = STREAM ? ld16_stream(kc + kr) : ld16(kc + kr);
  t.k[1] = STREAM ? ld16_stream(kc + kr + 64) : ld16(kc + kr + 64);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint8_t *src = vc + vr + ((4 * r + v) & 7) * 128 + 8 * c;
    t.v[v] = STREAM ? ld8_stream(src) : ld8(src);
  }
}

__device__ __forceinline__ KVTile expand_fp8_tile(const KVTile8 &s) {
  KVTile t;
  t.k[0] = fp8x8_to_bf16x8(s.k[0][0], s.k[0][1]);
  t.k[1] = fp8x8_to_bf16x8(s.k[0][2], s.k[0][3]);
  t.k[2] = fp8x8_to_bf16x8(s.k[1][0], s.k[1][1]);
  t.k[3] = fp8x8_to_bf16x8(s.k[1][2], s.k[1][3]);
#pragma unroll
  for (int v = 0; v < 4; ++v) t.v[v] = fp8x8_to_bf16x8(s.v[v][0], s.v[v][1]);
  return t;
}

// The q operand in the FP8 tile's K-dim order (nullptr -> zeros).
__device__ __forceinline__ void load_q_operand_fp8k(bf16x8 qb[4], const uint16_t *qrow, int r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 v = qrow ? ld16(qrow + 64 * (i >> 1) + 16 * r + 8 * (i & 1)) : u32x4{0u, 0u, 0u, 0u};
    qb[i] = __builtin_bit_cast(bf16x8, v);
  }
}

// The two cache formats the decode kernels take, behind one interface:
// Raw is the tile as loaded (and carried through the prefetch ring), expand()
// the bf16 tile the step multiplies.
template <bool kFp8>
struct KVFormat;
template <>
struct KVFormat<false> {
  using Elem = uint16_t;
  using Raw = KVTile;
  static __device__ __forceinline__ void load(Raw &t, const Elem *kc, const Elem *vc, const TileRows &tr, int r,
                                              int c, bool stream) {
    load_kv_tile_rows(t, kc, vc, tr, r, c, stream);
  }
  template <bool STREAM>
  static __device__ __forceinline__ void load_as(Raw &t, const Elem *kc, const Elem *vc, const TileRows &tr, int r,
                                                 int c) {
    load_kv_tile_rows(t, kc, vc, tr, r, c, STREAM);
  }
  static __device__ __forceinline__ KVTile expand(const Raw &t) { return t; }
  static __device__ __forceinline__ void load_q(bf16x8 qb[4], const uint16_t *qrow, int r);
};
template <>
struct KVFormat<true> {
  using Elem = uint8_t;
  using Raw = KVTile8;
  static __device__ __forceinline__ void load(Raw &t, const Elem *kc, const Elem *vc, const TileRows &tr, int r,
                                              int c, bool stream) {
    load_kv_tile_rows_fp8(t, kc, vc, tr, r, c, stream);
  }
  template <bool STREAM>
  static __device__ __forceinline__ void load_as(Raw &t, const Elem *kc, const Elem *vc, const TileRows &tr, int r,
                                                 int c) {
    load_kv_tile_rows_fp8_as<STREAM>(t, kc, vc, tr, r, c);
  }
  static __device__ __forceinline__ KVTile expand(const Raw &t) { return expand_fp8_tile(t); }
  static __device__ __forceinline__ void load_q(bf16x8 qb[4], const uint16_t *qrow, int r) {
    load_q_operand_fp8k(qb, qrow, r);
  }
};

// Q^T operand for column c from a query row of 128 bf16 (nullptr -> zeros).
__device__ __forceinline__ void load_q_operand_d128(bf16x8 qb[4], const uint16_t *qrow, int r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 v = qrow ? ld16(qrow + 32 * i + 8 * r) : u32x4{0u, 0u, 0u, 0u};
    qb[i] = __builtin_bit_cast(bf16x8, v);
  }
}

__device__ __forceinline__ void KVFormat<false>::load_q(bf16x8 qb[4], const uint16_t *qrow, int r) {
  load_q_operand_d128(qb, qrow, r);
}

// Slack of the lazy output rescale (log2 units): weights may reach 2^8
// before the running max is moved up, which fp32 sums and the bf16 hi + lo
// split carry without loss.
constexpr float kLazyRescale = 8.f;

// The lazy max update shared by the decode and prefill steps.  `local` is this
// lane's max of the new scores (log2 units).  Only when some lane's max
// exceeds its column's running max m by more than kLazyRescale (a
// wave-uniform test) is the column max taken across the four lanes that hold
// a column, m raised to it and the output (acc, l) rescaled; otherwise m stays
// and the new weights may exceed 1 by up to 2^kLazyRescale.  Taking the
// column max only on that path changes nothing: the test fires exactly when
// the column max would pass it.  nm is -m, or 0 while m is -inf.
template <int N>
__device__ __forceinline__ void raise_lazy_max(float local, float &m, float &nm, float &l, floatx4 (&acc)[N]) {
  if (__builtin_amdgcn_ballot_w64(local > m + kLazyRescale) != 0) {
    const float m_new = fmaxf(m, row_max4(local));
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float corr = fast_exp2(m - m_use);
    l *= corr;
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] *= corr;
    m = m_new;
    nm = m_new == kNegInf ? 0.f : -m_new;
  }
}

// Splits two weights into bf16 hi parts (each rounded to nearest even) and
// bf16 lo parts (the exactly representable remainders, rounded), packed in
// pairs as the MFMA operands take them.  The hi parts are widened back with
// one permute / one mask instead of a second conversion.
__device__ __forceinline__ void split_bf16x2(float e0, float e1, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(e0, e1);
  const float h0 = __uint_as_float(__builtin_amdgcn_perm(0u, hi, 0x01000c0cu));  // hi << 16
  const float h1 = __uint_as_float(hi & 0xffff0000u);
  lo = pack_bf16x2(e0 - h0, e1 - h1);
}

struct MfmaAttnState {
  float m;          // running max of the column, log2 domain
  float nm;         // -m, or 0 while m is -inf (the exponent offset)
  float l;          // running sum of this lane's share of the weights
  floatx4 acc[8];   // unnormalised output, see the header comment

  __device__ __forceinline__ void init() {
    m = kNegInf;
    nm = 0.f;
    l = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // One 16-token block whose first token has logical index tok0; keys with
  // logical index >= lim are masked for this lane's column.  sl2 =
  // scale * log2(e) > 0.  As in the prefill step, the max is taken on the
  // raw scores and scaled once, and the output is rescaled only when some
  // column's max grows by more than 2^kLazyRescale (wave-uniform), so most
  // tiles of a long row skip the 32-register rescale.
  __device__ __forceinline__ void step(const bf16x8 qb[4], const KVTile &t, int tok0, int lim,
                                       float sl2, int r) {
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) s = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[i]), qb[i], s);
    const int tok = tok0 + 4 * r;
    float x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = (tok + v < lim) ? s[v] : kNegInf;
    raise_lazy_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])) * sl2, m, nm, l, acc);
    float e[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) e[v] = fast_exp2(__builtin_fmaf(x[v], sl2, nm));
    // The weights enter the bf16 PV product as hi + lo bf16 parts: hi is e
    // rounded to bf16, lo is the (exactly representable) remainder rounded to
    // bf16, so hi + lo carries e to about 2^-17 relative.
    uint32_t hi0, hi1, lo0, lo1;
    split_bf16x2(e[0], e[1], hi0, lo0);
    split_bf16x2(e[2], e[3], hi1, lo1);
    l += (e[0] + e[1]) + (e[2] + e[3]);
    const u32x2 pb_hi = {hi0, hi1};
    const u32x2 pb_lo = {lo0, lo1};
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const u32x2 a_lo = {pack_lo_halves(t.v[0][w2], t.v[1][w2]), pack_lo_halves(t.v[2][w2], t.v[3][w2])};
      const u32x2 a_hi = {pack_hi_halves(t.v[0][w2], t.v[1][w2]), pack_hi_halves(t.v[2][w2], t.v[3][w2])};
      acc[2 * w2] = mfma_16x16x16_bf16(a_lo, pb_hi, acc[2 * w2]);
      acc[2 * w2] = mfma_16x16x16_bf16(a_lo, pb_lo, acc[2 * w2]);
      acc[2 * w2 + 1] = mfma_16x16x16_bf16(a_hi, pb_hi, acc[2 * w2 + 1]);
      acc[2 * w2 + 1] = mfma_16x16x16_bf16(a_hi, pb_lo, acc[2 * w2 + 1]);
    }
  }
};

// Prefill variant: two 16-token blocks at a time, so the PV product can use
// the full-rate 16x16x32 MFMA (K = 32 keys).  For a lane the 8 contraction
// indices k = 8r .. 8r+7 stand for keys 4r..4r+3 of block A and 4r..4r+3 of
// block B; the P^T operand (from the two QK outputs) and the V^T operand use
// the same order.  The V^T operand of output dims 16t .. 16t+15 arrives
// ready-made (vt[t], from LDS transpose reads): lane (r, c) holds
// V_A[4r..4r+3][16t + c] then V_B[4r..4r+3][16t + c].  So
//   acc[t][i] = O[column c][dim 16t + 4r + i].
// The PV product runs in fp16 (v_mfma_f32_16x16x32_f16): V is held as fp16
// in LDS (widened from the cache on its way there) and each weight is
// rounded to fp16 once, a relative error of at most 2^-11 per weight; the
// sum l is taken from the unrounded fp32 weights.
// The output is rescaled only when a column's running max grows by more than
// 2^kLazyRescale, so most pairs skip the 32-register rescale; weights can
// then exceed 1 (by at most that factor), which fp32 sums and fp16 carry.
// Scores stay unscaled until the exponent: m is kept in log2 units and each
// weight is exp2(s * sl2 - m) with one fma (scaling by sl2 > 0 commutes with
// the max).

struct MfmaAttnPairState {
  float m;
  float nm;  // -m, or 0 while m is -inf
  float l;
  floatx4 acc[8];

  __device__ __forceinline__ void init() {
    m = kNegInf;
    nm = 0.f;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // The raw scores of blocks A (keys tok0 .. tok0+15) and B (keys tok0+16 ..)
  // for this lane's column: ka / kb are the K operands (token c, dims 32i + 8r ..).
  static __device__ __forceinline__ void scores(const bf16x8 qb[4], const u32x4 ka[4], const u32x4 kb[4],
                                                float x[8]) {
    floatx4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[i]), qb[i], sa);
      sb = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[i]), qb[i], sb);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x[v] = sa[v];
      x[4 + v] = sb[v];
    }
  }

  // Raises the running max to cover scores x (scaled by sl2 into log2 units),
  // rescaling the output only when some column's max grew past the slack.
  __device__ __forceinline__ void raise_max(const float x[8], float sl2) {
    const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    raise_lazy_max(mx * sl2, m, nm, l, acc);
  }

  // The weights exp2(x * sl2 - m) as the fp16 operand; adds them to l.
  __device__ __forceinline__ void weights(const float x[8], float sl2, f16x8 &pb) {
    float e[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) e[v] = fast_exp2(__builtin_fmaf(x[v], sl2, nm));
    l += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    pb = __builtin_bit_cast(f16x8, u32x4{pack_f16x2(e[0], e[1]), pack_f16x2(e[2], e[3]), pack_f16x2(e[4], e[5]),
                                         pack_f16x2(e[6], e[7])});
  }

  // O^T += V^T P^T for the eight 16-dim tiles.
  __device__ __forceinline__ void pv(const f16x8 vt[8], const f16x8 &pb) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = mfma_16x16x32_f16(vt[t], pb, acc[t]);
  }

  // One pair of blocks for this lane's column: vt are the V^T operands.  When
  // `mask` is set (wave-uniform; false when every key of both blocks is
  // visible to every column of the wave), keys of A at or past lim_a and keys
  // of B at or past lim_b are masked for this lane's column.
  __device__ __forceinline__ void step(const bf16x8 qb[4], const u32x4 ka[4], const u32x4 kb[4],
                                       const f16x8 vt[8], int tok0, int lim_a, int lim_b, bool mask,
                                       float sl2, int r) {
    float x[8];
    scores(qb, ka, kb, x);
    if (mask) {
      const int ta = tok0 + 4 * r, tb = tok0 + 16 + 4 * r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[v] = ta + v < lim_a ? x[v] : kNegInf;
        x[4 + v] = tb + v < lim_b ? x[4 + v] : kNegInf;
      }
    }
    raise_max(x, sl2);
    f16x8 pb;
    weights(x, sl2, pb);
    pv(vt, pb);
  }
};

// Two column groups over the same pair of blocks (load_v() fills the V^T
// operands vt): the same arithmetic per
// group as MfmaAttnPairState::step (`mask0` / `mask1` as its `mask`, with the
// groups' own key limits), ordered so that one group's matrix products can
// run while the other group's softmax is computed: both score products
// first, then the max updates, then group 0's weights and PV products, then
// group 1's.  A group whose keys are all masked leaves its state unchanged
// (its weights are exp2(-inf) = 0).
template <class LoadV>
__device__ __forceinline__ void pair_step_x2(MfmaAttnPairState &s0, MfmaAttnPairState &s1, const bf16x8 q0[4],
                                             const bf16x8 q1[4], const u32x4 ka[4], const u32x4 kb[4],
                                             LoadV &&load_v, const f16x8 vt[8], int tok0, int lim_a0, int lim_b0,
                                             bool mask0, int lim_a1, int lim_b1, bool mask1, float sl2, int r) {
  float x0[8], x1[8];
  MfmaAttnPairState::scores(q0, ka, kb, x0);
  MfmaAttnPairState::scores(q1, ka, kb, x1);
  load_v();  // fills vt; issued after the score products have read ka / kb
  const int ta = tok0 + 4 * r, tb = tok0 + 16 + 4 * r;
  if (mask0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x0[v] = ta + v < lim_a0 ? x0[v] : kNegInf;
      x0[4 + v] = tb + v < lim_b0 ? x0[4 + v] : kNegInf;
    }
  }
  if (mask1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x1[v] = ta + v < lim_a1 ? x1[v] : kNegInf;
      x1[4 + v] = tb + v < lim_b1 ? x1[4 + v] : kNegInf;
    }
  }
  s0.raise_max(x0, sl2);
  s1.raise_max(x1, sl2);
  f16x8 p0, p1;
  s0.weights(x0, sl2, p0);
  s0.pv(vt, p0);
  s1.weights(x1, sl2, p1);
  s1.pv(vt, p1);
}

}  // namespace pa
