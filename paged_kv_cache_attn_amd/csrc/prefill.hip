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
// MFMA kernel: a group of 16 columns = (16 / g) consecutive chunk tokens x the
// g query heads of one KV head, so every K/V tile read is shared by the whole
// GQA group; each wave owns two such groups, and the four waves of a
// workgroup cover consecutive tokens and walk the same key blocks, in
// ascending order with per-column causal bounds.
#include <type_traits>

#include "attn_core.h"
#include "attn_vec.h"
#include "pa_launch.h"

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
#ifndef PA_PREFILL_GROUPS
#define PA_PREFILL_GROUPS 2
#endif


namespace pa {

namespace {

__device__ __forceinline__ void store_out(void *out, int out_bf16, int64_t idx, float v) {
  if (out_bf16) {
    reinterpret_cast<__bf16 *>(out)[idx] = (__bf16)v;
  } else {
    reinterpret_cast<float *>(out)[idx] = v;
  }
}

// bf16 KV, head_dim 128, block size 8, 16, 32, 64 or 128 (walked in
// 16-token tiles), g in {1, 2, 4, 8, 16}.
//
// A workgroup of NW waves serves NW * CG * 16 / g consecutive chunk tokens of
// one KV head.  Wave w owns CG groups of 16 columns (16 / g tokens x the g
// query heads each).  Keys are taken two blocks (32 keys) at a time: the
// workgroup loads each pair of K/V tiles from global memory ONCE into LDS
// (bf16: straight into a four-stage ring; FP8: through registers into a
// three-stage ring), and every wave reads its MFMA operands from there, so
// global/L2 traffic falls by the workgroup's column count.
//
// An LDS stage holds four 4 KB tiles (K_a, V_a, K_b, V_b).  In a
// K tile the 16-byte chunk k of token t sits at chunk t*16 + (k ^ t), so the
// K operand reads (token c, chunk 4i + r) touch 16 distinct bank groups per
// 16 lanes.  A V tile is read with ds_read_b64_tr_b16, which hands lane
// 16r + c element (c mod 4) of the 8-byte word addressed by lane
// 16r + 4j + (c / 4) as its element j: when lane (r, j, q) addresses
// V[4r + j][16t + 4q .. +3], lane (r, c) receives V[4r .. 4r+3][16t + c], the
// V^T operand.  Those reads take 32 contiguous bytes from each of 16 tokens,
// so a V tile swizzles 32-byte segments: segment s of token t sits at
// segment t*8 + (s ^ (t & 7)).
//
// Block-table entries are read through the scalar cache (the table is not
// written during the call), so the K/V loads are the only vector-memory
// operations of the loop and a wait for one pair never waits on table reads.
//
// Dispatch order: each XCD takes a contiguous run of (sequence, KV head)
// groups; within the run, sets of kset groups go one after another, and a
// set's tiles go heaviest first (the last query tile of the chunk, which
// reads the most keys) across all of its groups, then the next heaviest.
// With kset * ntiles about one XCD's workgroup slots, a set fills the XCD,
// the long tiles start first and the short ones fill in behind them (longest
// processing time first), while the set's K/V still fits that XCD's L2.  A
// column group past its causal bound is fully masked (every wave joins every
// barrier).  grid = ntiles * Hkv * B workgroups, ntiles =
// ceil(max_query_len / (NW * CG * 16 / g)).  The block size BSZ is a template
// argument so the table walk folds to constants for each supported size.
//
// V is held in LDS as fp16 for the fp16 PV product: bf16 caches load a pair's
// V tiles as they are and each lane converts the slots it loaded in place,
// one pair ahead of their use; FP8 caches widen on the way in.
//
// FP8 (E4M3) caches: a pair is 512 16-byte chunks in HBM instead of 1024;
// each chunk is expanded on its way into LDS (K to bf16, V to fp16, both
// exactly), so the LDS layout and everything after it are those of the bf16
// cache.  k_scale is
// folded into the score scale and v_scale into the final normalisation.
template <int NW, int CG, int BSZ, bool FP8>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mfma_d128_kernel(
    PrefillParams p, int ntiles) {
  using Elem = typename KVFormat<FP8>::Elem;
  constexpr int D = 128;
  constexpr int BS = 16;
  constexpr int kTile = 4096;            // bytes of one K or V tile in LDS (bf16)
  constexpr int kStage = 4 * kTile;      // K_a, V_a, K_b, V_b
  constexpr int kTileShift = FP8 ? 7 : 8;
  constexpr int kTileChunks = 1 << kTileShift;      // 16-byte chunks of one tile in HBM
  constexpr int kChunkElems = FP8 ? 16 : 8;         // elements per chunk
  constexpr int kChunksPerThread = 4 * kTileChunks / (64 * NW);
  // bf16 pairs go from global memory straight into LDS (four stages); FP8
  // pairs are widened on the way, through registers (three stages).  Each
  // stage is an array of its own, so the compiler can tell a load into one
  // stage from reads of another and waits only for what a read needs.
  constexpr bool kDma = !FP8;
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds3[kDma ? kStage : 16];
  auto stage_mem = [&](auto st) __attribute__((always_inline)) -> uint8_t * {
    constexpr int k = decltype(st)::value;
    return k == 0 ? lds0 : k == 1 ? lds1 : k == 2 ? lds2 : lds3;
  };

  const unsigned item = xcd_contiguous(blockIdx.x, gridDim.x);
  const unsigned nt = (unsigned)ntiles, ngrp = gridDim.x / nt;
  constexpr unsigned kXcdSlots = 32 * 2;  // CUs per XCD x workgroups per CU
  const unsigned kset = nt >= kXcdSlots ? 1u : kXcdSlots / nt;
  const unsigned set = item / (kset * nt), off = item - set * kset * nt;
  const unsigned nset = min(kset, ngrp - set * kset);  // groups in this set
  // the quotients are uniform; readfirstlane keeps them (and the addresses
  // built from them) in scalar registers
  const unsigned grp = __builtin_amdgcn_readfirstlane(set * kset + off % nset);
  const int tile = __builtin_amdgcn_readfirstlane(ntiles - 1 - (int)(off / nset));
  // a group is (sequence, KV head, sub-group): the query heads of a KV head
  // are served hs at a time (hs = 1 unless the group size does not divide
  // 16), the sub-groups of one KV head next to each other
  const int hs = max(p.head_split, 1);
  const unsigned nkv = (unsigned)(p.num_kv_heads * hs);
  const int kv = (int)(grp % nkv);
  const int b = (int)(grp / nkv);
  const int kh = kv / hs;
  const int g = p.num_heads / p.num_kv_heads / hs;  // query heads per column group row
  const int64_t hbase = (int64_t)kh * (g * hs) + (int64_t)(kv - kh * hs) * g;  // the sub-group's first head
  const int tpgrp = 16 / g;              // chunk tokens per column group
  const int tpw = CG * tpgrp;            // per wave
  const int tpg = NW * tpw;              // per workgroup
  const int q0 = p.query_start_loc[b];
  const int n_b = p.query_start_loc[b + 1] - q0;
  const int S = clamp_len(p.seq_lens[b], p.max_len_cap);
  debug_report(threadIdx.x == 0 && (q0 < 0 || n_b < 0 || n_b > S || (int64_t)q0 + n_b > p.num_query_tokens),
               kDbgQueryLoc);
  if (tile * tpg >= n_b || q0 < 0) return;  // the whole workgroup leaves together
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4, c = lane & 15;

  // key bound of the whole workgroup (its last valid chunk row)
  const int last_qi_wg = min(tile * tpg + tpg, n_b) - 1;
  const int kend_wg = max(0, S - n_b + last_qi_wg + 1);
  const int nblk = (kend_wg + BS - 1) / BS;
  const int npair = (nblk + 1) / 2;

  // columns of each group of this wave
  const int ti = c / g, hh = c - (c / g) * g;
  int lim[CG], lim_min[CG], kend[CG];
  bool col_ok[CG];
  bf16x8 qb[CG][4];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const int first = tile * tpg + w * tpw + cg * tpgrp;  // first chunk row of the group
    const int qi = first + ti;
    col_ok[cg] = qi < n_b && (int64_t)q0 + qi < p.num_query_tokens;
    lim[cg] = col_ok[cg] ? S - n_b + qi + 1 : 0;
    lim_min[cg] = S - n_b + first + 1;
    const int last = min(first + tpgrp, n_b) - 1;
    kend[cg] = last >= first ? max(0, S - n_b + last + 1) : 0;
    // idle columns read a valid row (never stored) so every value stays finite
    // (clamped to the query rows, whatever query_start_loc holds)
    const int64_t row_ld = min((int64_t)q0 + (col_ok[cg] ? qi : last_qi_wg), (int64_t)p.num_query_tokens - 1);
    load_q_operand_d128(qb[cg],
                        reinterpret_cast<const uint16_t *>(p.q) + (row_ld * p.num_heads + hbase + hh) * D,
                        r);
  }

  const float sl2 = p.scale * p.k_scale * kLog2e;
  const __attribute__((address_space(4))) int32_t *table =
      (const __attribute__((address_space(4))) int32_t *)(p.block_tables + (int64_t)b * p.max_blocks_per_seq);
  const Elem *kc = reinterpret_cast<const Elem *>(p.k_cache);
  const Elem *vc = reinterpret_cast<const Elem *>(p.v_cache);
  const TileMap map(BSZ, p.num_kv_heads, p.num_blocks);
  const int nblk_tab = (S + BSZ - 1) / BSZ;  // table entries the sequence uses

  // Cooperative pair load: the 4 * kTileChunks 16-byte chunks of a pair of
  // 16-token tiles, consecutive threads on consecutive chunks of a tile.  Returns
  // which of the two tiles hold real data (bit 0: A, bit 1: B); tile
  // j >= nblk (the odd tail) and a tile with an out-of-range table entry are
  // read from block 0 and masked later.  Which tile, K or V, and which half
  // of the tile (rows 0-7 or 8-15) a thread loads is the same for its whole
  // wave, so the two row bases are selected in scalar registers.
  // The table values a pair's tiles live in (read through the scalar cache),
  // apart from the loads they address, so a loop can read them one pair early.
  auto pair_table = [&](int pr) __attribute__((always_inline)) -> int4 {
    pr = min(pr, max(npair - 1, 0));
    int ia0, ia1, ib0, ib1;
    map.indices(2 * pr, nblk_tab, ia0, ia1);
    map.indices(max(0, min(2 * pr + 1, nblk - 1)), nblk_tab, ib0, ib1);
    return int4{table[ia0], table[ia1], table[ib0], table[ib1]};
  };
  auto gload_from = [&](int pr, u32x4 *regs, int4 tv) __attribute__((always_inline)) -> int {
    pr = min(pr, max(npair - 1, 0));
    const int ja = 2 * pr, jb = 2 * pr + 1;
    int a0, a1, b0, b1;
    const bool oka = map.entries_from(tv.x, tv.y, ja, a0, a1);
    const bool entb = map.entries_from(tv.z, tv.w, max(0, min(jb, nblk - 1)), b0, b1);
    const bool okb = entb && jb < nblk;
    const int bad = !oka || (jb < nblk && !entb);  // an entry out of range (bit 2 of the result)
    const TileRows ra = map.rows(a0, a1, kh);
    const TileRows rb = map.rows(b0, b1, kh);  // the odd tail repeats tile nblk - 1, masked
#pragma unroll
    for (int k = 0; k < kChunksPerThread; ++k) {
      const int uw = w * 64 + k * 64 * NW;  // first chunk of the wave (a multiple of 64)
      const int kind = uw >> kTileShift;    // 0 K_a, 1 V_a, 2 K_b, 3 V_b
      const TileRows &tr = kind < 2 ? ra : rb;
      // rows 8-15 start 8 rows after their own base: rebase so chunk q sits at q * kChunkElems
      const int64_t base = (uw & (kTileChunks / 2)) == 0 ? tr.lo : tr.hi - 8 * D;
      regs[k] = ld16(((kind & 1) ? vc : kc) + base + ((uw & (kTileChunks - 1)) + lane) * kChunkElems);
    }
    return (int)oka | ((int)okb << 1) | (bad << 2);
  };
  auto gload = [&](int pr, u32x4 *regs) -> int { return gload_from(pr, regs, pair_table(pr)); };
  // Direct pair load (bf16): the k-th load of wave w fills the 64 consecutive
  // 16-byte slots of the stage from slot (k * NW + w) * 64 on, one per lane
  // (64 slots = 4 rows of one tile), so each lane fetches the global chunk
  // that the swizzled layout below puts in its slot: in a K tile slot col of
  // row t holds chunk col ^ t, in a V tile chunk 2 ((col / 2) ^ (t & 7)) +
  // (col & 1).  Same tiles, masking bits and clamping as gload.
  // With four waves, load k of wave w is tile k, rows 4w .. 4w + 3 (one row
  // per 16 lanes), all in one half of the tile (rows 0-7 or 8-15, contiguous
  // at every block size): each load is a wave-uniform tile base in scalar
  // registers plus a per-lane byte offset that never changes.
  constexpr bool kRowsContig = NW == 4;
  const int trow = 4 * w + (lane >> 4), tcol = lane & 15;
  const uint32_t off_k = (uint32_t)(trow * D + (tcol ^ trow) * 8) * 2u;
  const uint32_t off_v = (uint32_t)(trow * D + ((((tcol >> 1) ^ (trow & 7)) << 1) | (tcol & 1)) * 8) * 2u;
  auto dma_from = [&](int pr, auto st, int4 tv) __attribute__((always_inline)) -> int {
    pr = min(pr, max(npair - 1, 0));
    const int ja = 2 * pr, jb = 2 * pr + 1;
    int a0, a1, b0, b1;
    const bool oka = map.entries_from(tv.x, tv.y, ja, a0, a1);
    const bool entb = map.entries_from(tv.z, tv.w, max(0, min(jb, nblk - 1)), b0, b1);
    const bool okb = entb && jb < nblk;
    const int bad = !oka || (jb < nblk && !entb);  // an entry out of range (bit 2 of the result)
    const TileRows ra = map.rows(a0, a1, kh);
    const TileRows rb = map.rows(b0, b1, kh);
    if constexpr (kRowsContig) {
      uint8_t *sm = stage_mem(st) + w * 1024;
      const uint8_t *kb8 = reinterpret_cast<const uint8_t *>(kc), *vb8 = reinterpret_cast<const uint8_t *>(vc);
      // rows 8-15 start 8 rows after their own base (the same address as
      // tr.lo when the block holds the whole tile)
      const int64_t ba = w < 2 ? ra.lo : ra.hi - 8 * D, bb = w < 2 ? rb.lo : rb.hi - 8 * D;
      load_lds16_sv(kb8 + ba * 2, off_k, sm + 0 * 4096);
      load_lds16_sv(vb8 + ba * 2, off_v, sm + 1 * 4096);
      load_lds16_sv(kb8 + bb * 2, off_k, sm + 2 * 4096);
      load_lds16_sv(vb8 + bb * 2, off_v, sm + 3 * 4096);
    } else {
      const int col = lane & 15;
#pragma unroll
      for (int k = 0; k < kChunksPerThread; ++k) {
        const int slot0 = (k * NW + w) * 64;  // wave-uniform
        const int kind = slot0 >> 8;          // 0 K_a, 1 V_a, 2 K_b, 3 V_b
        const int t = ((slot0 & 255) >> 4) + (lane >> 4);
        const int ch = (kind & 1) ? ((((col >> 1) ^ (t & 7)) << 1) | (col & 1)) : (col ^ t);
        const TileRows &tr = kind < 2 ? ra : rb;
        const int64_t base = (slot0 & 128) == 0 ? tr.lo : tr.hi - 8 * D;  // rows 0-7 or 8-15 of the tile
        const Elem *src = ((kind & 1) ? vc : kc) + base + t * D + ch * 8;
        load_lds16(src, stage_mem(st) + slot0 * 16);
      }
    }
    return (int)oka | ((int)okb << 1) | (bad << 2);
  };
  auto dma = [&](int pr, auto st) __attribute__((always_inline)) -> int { return dma_from(pr, st, pair_table(pr)); };
  // LDS byte offset of bf16 chunk kc (0..15) of row t in a K or a V tile
  auto lds_off = [](bool is_v, int t, int kc) -> int {
    return is_v ? t * 256 + ((((kc >> 1) ^ (t & 7)) << 5) | ((kc & 1) << 4)) : (t * 16 + (kc ^ t)) << 4;
  };
  auto lstore = [&](auto stage, const u32x4 *regs) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kChunksPerThread; ++k) {
      const int u = tid + k * 64 * NW;
      // (a tile spans at least one wave's chunks, so the tile kind is the
      // wave's: computed from w, it stays in scalar registers)
      static_assert(kTileShift >= 6, "a tile holds whole waves' chunks");
      const int kind = (w * 64 + k * 64 * NW) >> kTileShift, q = u & (kTileChunks - 1);
      uint8_t *tb = stage_mem(stage) + kind * kTile;
      if (FP8) {
        // 16 codes = 16-bit chunks 2 kc8 and 2 kc8 + 1 of row t (K as bf16,
        // V as fp16: both exact)
        const int t = q >> 3, kc8 = q & 7;
        if (kind & 1) {
          *reinterpret_cast<u32x4 *>(tb + lds_off(true, t, 2 * kc8)) = fp8x8_to_f16x8(regs[k][0], regs[k][1]);
          *reinterpret_cast<u32x4 *>(tb + lds_off(true, t, 2 * kc8 + 1)) = fp8x8_to_f16x8(regs[k][2], regs[k][3]);
        } else {
          *reinterpret_cast<u32x4 *>(tb + lds_off(false, t, 2 * kc8)) = fp8x8_to_bf16x8(regs[k][0], regs[k][1]);
          *reinterpret_cast<u32x4 *>(tb + lds_off(false, t, 2 * kc8 + 1)) =
              fp8x8_to_bf16x8(regs[k][2], regs[k][3]);
        }
      } else {
        *reinterpret_cast<u32x4 *>(tb + lds_off(kind & 1, q >> 4, q & 15)) = regs[k];
      }
    }
  };
  // bf16 caches: the V tiles of a pair arrive in LDS as bf16 and are turned
  // into fp16 in place before any wave reads them; each lane converts the
  // two 16-byte slots its own loads filled (loads 1 and 3: V_a and V_b), so
  // it needs only its own loads done, and the barrier before the pair's V
  // reads publishes the result.
  auto convert_v = [&](auto st) __attribute__((always_inline)) {
    static_assert(kRowsContig, "slots of a lane's V loads");
    uint8_t *own = stage_mem(st) + w * 1024 + lane * 16;
    u32x4 *pa = reinterpret_cast<u32x4 *>(own + 1 * kTile), *pb = reinterpret_cast<u32x4 *>(own + 3 * kTile);
    const u32x4 a = *pa, b = *pb;
    *pa = u32x4{bf16x2_to_f16x2(a[0]), bf16x2_to_f16x2(a[1]), bf16x2_to_f16x2(a[2]), bf16x2_to_f16x2(a[3])};
    *pb = u32x4{bf16x2_to_f16x2(b[0]), bf16x2_to_f16x2(b[1]), bf16x2_to_f16x2(b[2]), bf16x2_to_f16x2(b[3])};
  };
  // V^T operand address of this lane inside a V tile for dim tile dt: lane
  // (r, j, q) = (r, c >> 2, c & 3) points at V[4r + j][16 dt + 4q].
  const int vtok = 4 * r + (c >> 2);
  const int vq8 = (c & 3) * 8;
  auto vt_addr = [&](int dt) -> int { return vtok * 256 + (((dt ^ (vtok & 7)) << 5) | vq8); };
  // The operands of one pair for this wave, from LDS stage `stage`: K first,
  // the V^T operands on their own so that they can be read after the score
  // products have taken the K registers.
  auto lread_k = [&](auto stage, u32x4 *ka, u32x4 *kb) __attribute__((always_inline)) {
    const uint8_t *base = stage_mem(stage);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ck = (c * 16 + ((4 * i + r) ^ c)) << 4;
      ka[i] = *reinterpret_cast<const u32x4 *>(base + 0 * kTile + ck);
      kb[i] = *reinterpret_cast<const u32x4 *>(base + 2 * kTile + ck);
    }
  };
  auto lread_v = [&](auto stage, f16x8 *vt) __attribute__((always_inline)) {
    const uint8_t *base = stage_mem(stage);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const int off = vt_addr(dt);
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 1 * kTile + off));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 3 * kTile + off));
      const u32x2 a2 = __builtin_bit_cast(u32x2, va), b2 = __builtin_bit_cast(u32x2, vb);
      vt[dt] = __builtin_bit_cast(f16x8, u32x4{a2[0], a2[1], b2[0], b2[1]});
    }
  };
  auto compute = [&](auto stage, int pr, int okbits, MfmaAttnPairState *st) __attribute__((always_inline)) {
    u32x4 ka[4], kb[4];
    f16x8 vt[8];
    lread_k(stage, ka, kb);
    const int tok0 = 32 * pr;
    const bool oka = okbits & 1, okb = okbits & 2;
    if constexpr (CG == 2) {
      // both groups in one step (a group past its causal bound is fully masked)
      const bool full0 = tok0 + 32 <= lim_min[0] && oka && okb;
      const bool full1 = tok0 + 32 <= lim_min[1] && oka && okb;
      pair_step_x2(st[0], st[1], qb[0], qb[1], ka, kb, [&]() __attribute__((always_inline)) { lread_v(stage, vt); },
                   vt, tok0, oka ? lim[0] : 0, okb ? lim[0] : 0, !full0, oka ? lim[1] : 0, okb ? lim[1] : 0, !full1,
                   sl2, r);
    } else {
      lread_v(stage, vt);
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (tok0 < kend[cg]) {
          const bool full = tok0 + 32 <= lim_min[cg] && oka && okb;
          st[cg].step(qb[cg], ka, kb, vt, tok0, oka ? lim[cg] : 0, okb ? lim[cg] : 0, !full, sl2, r);
        }
      }
    }
  };

  MfmaAttnPairState st[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) st[cg].init();
  int seen = 0;  // OR of the pairs' load results: bit 2 = a block-table entry out of range

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  static_assert(!kDma || CG == 2, "bf16 caches take the pipelined two-group loop");
  if (kDma && npair > 0) {
    // Software-pipelined: iteration X takes the softmax and PV products of
    // pair X while the score products of pair X + 1 run, so the two column
    // groups' softmax chains overlap matrix work.  Pair X lands in stage
    // X % 4.  At the top of iteration X each thread waits for its own loads
    // of pair X + 1 (those of X + 2 may stay in flight: kChunksPerThread
    // loads) and the barrier covers every thread's; the loads of pair X + 3
    // then go into stage (X + 3) % 4, whose last reads (V of X - 1, K of
    // X - 1) came before that barrier.  Pairs past the end are not loaded
    // (a load there would hold the workgroup's end back by a memory round
    // trip); the last iteration then reads stale K tiles for a next pair
    // whose scores are never used, and near the end every load in flight is
    // waited for, since fewer follow the pair needed.
    int ok[4] = {0, 0, 0, 0};
    ok[0] = dma(0, S0());
    if (npair > 1) ok[1] = dma(1, S1());
    if (npair > 2) ok[2] = dma(2, S2());
    // the table values of the pair the next iteration loads, read one
    // iteration early so that no scalar-cache round trip sits between the
    // barrier and the loads
    int4 tv_next = pair_table(3);
    float x0[8], x1[8];  // scores of the pair the next iteration finishes
    if (npair > 2)
      vm_wait<2 * kChunksPerThread>();
    else
      vm_wait<0>();
    workgroup_barrier();
    convert_v(S0());
    {
      u32x4 ka[4], kb[4];
      lread_k(S0(), ka, kb);
      MfmaAttnPairState::scores(qb[0], ka, kb, x0);
      MfmaAttnPairState::scores(qb[CG - 1], ka, kb, x1);
    }
    auto piter = [&](int X, auto cur, auto nxt, auto ld) __attribute__((always_inline)) -> bool {
      // (the LDS stores of pair X's fp16 V, made in the previous iteration,
      // are waited for too)
      if (X + 2 < npair)
        vm_lgkm_wait<kChunksPerThread>();
      else
        vm_lgkm_wait<0>();
      workgroup_barrier();
      if (X + 3 < npair) ok[decltype(ld)::value] = dma_from(X + 3, ld, tv_next);
      tv_next = pair_table(X + 4);
      f16x8 vt[8];
      u32x4 ka[4], kb[4];
      lread_v(cur, vt);
      lread_k(nxt, ka, kb);
      const int okbits = ok[decltype(cur)::value];
      seen |= okbits;
      const int tok0 = 32 * X;
      const bool oka = okbits & 1, okb = okbits & 2;
      const bool full0 = tok0 + 32 <= lim_min[0] && oka && okb;
      const bool full1 = tok0 + 32 <= lim_min[CG - 1] && oka && okb;
      const int ta = tok0 + 4 * r, tb = tok0 + 16 + 4 * r;
      if (!full0) {
        const int la = oka ? lim[0] : 0, lb = okb ? lim[0] : 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x0[v] = ta + v < la ? x0[v] : kNegInf;
          x0[4 + v] = tb + v < lb ? x0[4 + v] : kNegInf;
        }
      }
      if (!full1) {
        const int la = oka ? lim[CG - 1] : 0, lb = okb ? lim[CG - 1] : 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x1[v] = ta + v < la ? x1[v] : kNegInf;
          x1[4 + v] = tb + v < lb ? x1[4 + v] : kNegInf;
        }
      }
      st[0].raise_max(x0, sl2);
      st[CG - 1].raise_max(x1, sl2);
      float y0[8], y1[8];
      // The block of matrix products (the next pair's scores, this pair's
      // PV products and the softmax work placed between them) runs at a
      // raised wave priority, so that a wave with matrix work ready issues
      // ahead of the SIMD's other wave when both are ready.
      __builtin_amdgcn_s_setprio(1);
      MfmaAttnPairState::scores(qb[0], ka, kb, y0);
      MfmaAttnPairState::scores(qb[CG - 1], ka, kb, y1);
      f16x8 p0, p1;
      st[0].weights(x0, sl2, p0);
      st[0].pv(vt, p0);
      st[CG - 1].weights(x1, sl2, p1);
      st[CG - 1].pv(vt, p1);
      __builtin_amdgcn_s_setprio(0);
      // pair X + 1's V, read by every wave in the next iteration (here, where
      // the matrix unit still has this pair's products queued)
      if (X + 1 < npair) convert_v(nxt);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        x0[v] = y0[v];
        x1[v] = y1[v];
      }
      // Scheduling of the block above (from the last rescale test on): its 32
      // MFMAs (16 score products of pair X + 1, 16 PV products of pair X) each
      // followed by up to three VALU instructions (weights, exponentials,
      // fp16 packing), so the vector work issues while the matrix unit is busy
      // instead of in runs between MFMA runs.  Only placement changes.
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);  // three VALU (incl. transcendental)
      }
      return X + 1 < npair;
    };
    for (int X = 0;; X += 4) {
      if (!piter(X, S0(), S1(), S3())) break;
      if (!piter(X + 1, S1(), S2(), S0())) break;
      if (!piter(X + 2, S2(), S3(), S1())) break;
      if (!piter(X + 3, S3(), S0(), S2())) break;
    }
  } else if (npair > 0) {
    // Pair X sits in register set X % 3 and LDS stage X % 3.  Its loads are
    // issued while pair X - 3 is computed and reach LDS while pair X - 1 is,
    // so each load has two pairs of work to arrive.
    u32x4 rs[3][kChunksPerThread];
    int ok_r[3], ok_s[3];
    ok_r[0] = gload(0, rs[0]);
    lstore(S0(), rs[0]);
    ok_s[0] = ok_r[0];
    ok_r[1] = gload(1, rs[1]);
    ok_r[2] = gload(2, rs[2]);
    int4 tv_next = pair_table(3);  // read one pair early, as in the loop above
    auto iter = [&](int X, auto phase) -> bool {
      constexpr int j = decltype(phase)::value, j1 = (j + 1) % 3;
      __syncthreads();
      if (X + 1 < npair) lstore(std::integral_constant<int, j1>(), rs[j1]);
      ok_s[j1] = ok_r[j1];
      ok_r[j] = gload_from(X + 3, rs[j], tv_next);
      tv_next = pair_table(X + 4);
      seen |= ok_s[j];
      compute(phase, X, ok_s[j], st);
      return X + 1 < npair;
    };
    for (int X = 0;; X += 3) {
      if (!iter(X, std::integral_constant<int, 0>())) break;
      if (!iter(X + 1, std::integral_constant<int, 1>())) break;
      if (!iter(X + 2, std::integral_constant<int, 2>())) break;
    }
  }

  // (reported after the loop: a report inside it would keep the table out of
  // the scalar cache in the debug build)
  debug_report((seen >> 2) & 1, kDbgBlockRange);
  (void)seen;
  // acc[t][i] = O[column c][dim 16t + 4r + i]
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const float l = row_sum4(st[cg].l);
    const float inv = l > 0.f ? p.v_scale / l : 0.f;
    const int qi = tile * tpg + w * tpw + cg * tpgrp + ti;
    const int64_t row = ((int64_t)q0 + qi) * p.num_heads + hbase + hh;
    if (!col_ok[cg]) continue;
    if (p.out_bf16) {
      uint16_t *o = reinterpret_cast<uint16_t *>(p.out) + row * D + 4 * r;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const floatx4 v = st[cg].acc[t] * inv;
        *reinterpret_cast<u32x2 *>(o + 16 * t) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    } else {
      float *o = reinterpret_cast<float *>(p.out) + row * D + 4 * r;
#pragma unroll
      for (int t = 0; t < 8; ++t) *reinterpret_cast<floatx4 *>(o + 16 * t) = st[cg].acc[t] * inv;
    }
  }
}

// Vector kernel: fp32 or bf16 KV, head_dim 64 or 128, any group size and
// block size (the shapes the MFMA kernel does not take).  One workgroup per
// (chunk row, KV head, sequence) serves the row's whole GQA group over its
// causal keys (attn_vec.h): each K/V row is read once per group.
constexpr int kVecWaves = 4;

template <int D, bool BF16, int GC>
__global__ __launch_bounds__(64 * kVecWaves) void prefill_vec_kernel(PrefillParams p) {
  constexpr int NW = kVecWaves;
  using G = VecGeom<D, BF16>;
  __shared__ float red[(NW + 1) * GC * (D + 2)];
  const int qi = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int q0 = p.query_start_loc[b];
  const int n_b = p.query_start_loc[b + 1] - q0;
  const int S = clamp_len(p.seq_lens[b], p.max_len_cap);
  debug_report(qi == 0 && threadIdx.x == 0 &&
                   (q0 < 0 || n_b < 0 || n_b > S || (int64_t)q0 + n_b > p.num_query_tokens),
               kDbgQueryLoc);
  // (uniform over the workgroup: it leaves together)
  if (qi >= n_b || q0 < 0 || (int64_t)q0 + qi >= p.num_query_tokens) return;
  const int g = p.num_heads / p.num_kv_heads;
  const int nkeys = max(0, min(S, S - n_b + qi + 1));
  const int col = ((threadIdx.x & 63) % G::kLPR) * G::kVPL;
  const float sl2 = p.scale * kLog2e;
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
  const uint8_t *qb = reinterpret_cast<const uint8_t *>(p.q);
  const int64_t qrow = (int64_t)(q0 + qi) * p.num_heads + (int64_t)kh * g;
  for (int h0 = 0; h0 < g; h0 += GC) {
    float q[GC][G::kVPL];
#pragma unroll
    for (int hh = 0; hh < GC; ++hh) {  // heads past the group repeat the last one, unused
      const uint8_t *qr = qb + ((qrow + min(h0 + hh, g - 1)) * D + col) * G::kElem;
#pragma unroll
      for (int c = 0; c < G::kCPL; ++c) unpack16<BF16>(ld16(qr + 16 * c), &q[hh][c * (G::kVPL / G::kCPL)]);
    }
    const float *res = vec_attend<D, BF16, NW, GC>(red, q, p.k_cache, p.v_cache, table, 0, nkeys, kh,
                                                   p.num_kv_heads, p.block_size, p.num_blocks, sl2);
    for (int idx = threadIdx.x; idx < GC * D; idx += 64 * NW) {
      const int hh = idx / D, d = idx - hh * D;
      if (h0 + hh >= g) continue;
      const float *e = res + hh * (D + 2);
      store_out(p.out, p.out_bf16, (qrow + h0 + hh) * D + d, e[D + 1] > 0.f ? e[d] / e[D + 1] : 0.f);
    }
    __syncthreads();  // the next chunk of heads reuses `red`
  }
}

// The vector kernel with the head chunk GC that fits the group: the group
// size rounded up to a power of two, at most 8.
template <int D, bool BF16, class Params>
void launch_vec(dim3 grid, dim3 block, hipStream_t stream, const Params &p) {
  const int g = p.num_heads / p.num_kv_heads;
  if (g <= 1)
    hipLaunchKernelGGL((prefill_vec_kernel<D, BF16, 1>), grid, block, 0, stream, p);
  else if (g <= 2)
    hipLaunchKernelGGL((prefill_vec_kernel<D, BF16, 2>), grid, block, 0, stream, p);
  else if (g <= 4)
    hipLaunchKernelGGL((prefill_vec_kernel<D, BF16, 4>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_vec_kernel<D, BF16, 8>), grid, block, 0, stream, p);
}

}  // namespace

#if PAGED_ATTN_DEBUG
PA_DEBUG_WORD_ACCESSOR(debug_word_prefill)
#endif

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_query_len == 0) return hipSuccess;
  const int hs = max(p.head_split, 1);
  const int g = p.num_heads / p.num_kv_heads / hs;  // heads per sub-group
  const bool mfma = (p.kv_bf16 || p.kv_fp8) && p.head_dim == 128 && mfma_block_size(p.block_size);
  if (mfma) {
    if (g * hs * p.num_kv_heads != p.num_heads || g > 16 || 16 % g != 0) return hipErrorInvalidValue;
    constexpr int NW = PA_PREFILL_WAVES, CG = PA_PREFILL_GROUPS;
    const int tpg = NW * CG * (16 / g);
    const int64_t ntiles = (p.max_query_len + tpg - 1) / tpg;
    const int64_t items = ntiles * p.num_kv_heads * hs * p.num_seqs;
    if (items * 64 * NW > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)items), block(64 * NW);
#define PA_PREFILL_LAUNCH(BSZ, FP8)                                                                   \
  hipLaunchKernelGGL((prefill_mfma_d128_kernel<NW, CG, BSZ, FP8>), grid, block, 0, stream, p, (int)ntiles)
    if (p.kv_fp8) {
      switch (p.block_size) {
        case 8: PA_PREFILL_LAUNCH(8, true); break;
        case 16: PA_PREFILL_LAUNCH(16, true); break;
        case 32: PA_PREFILL_LAUNCH(32, true); break;
        case 64: PA_PREFILL_LAUNCH(64, true); break;
        default: PA_PREFILL_LAUNCH(128, true); break;
      }
    } else {
      switch (p.block_size) {
        case 8: PA_PREFILL_LAUNCH(8, false); break;
        case 16: PA_PREFILL_LAUNCH(16, false); break;
        case 32: PA_PREFILL_LAUNCH(32, false); break;
        case 64: PA_PREFILL_LAUNCH(64, false); break;
        default: PA_PREFILL_LAUNCH(128, false); break;
      }
    }
#undef PA_PREFILL_LAUNCH
  } else {
    const dim3 grid(p.max_query_len, p.num_kv_heads, p.num_seqs), block(64 * kVecWaves);
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
  return hipGetLastError();
}

}  // namespace pa
