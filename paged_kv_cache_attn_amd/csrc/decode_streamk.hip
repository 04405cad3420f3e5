// decode_streamk.hip -- balanced ("stream-K") paged decode on gfx950.
//
// Same arithmetic as the MFMA decode tile step (attn_core.h), different work
// split.  The blocks of all (sequence, KV head) rows are laid end to end in
// one flat index space (KV head major, then sequence, then logical block) and
// cut into equal contiguous ranges, one per workgroup, so every workgroup
// streams the same number of 8 KB K+V tiles whatever the length mix.  A
// range covers whole rows, whose output it writes directly, and at most two
// partial rows at its ends, for which it leaves (max, sum, unnormalised
// output) in the workspace with plain stores; a descriptor per range names
// the split row whose last piece the range holds (written by the range
// itself, or, for a planned call, taken from the plan).  A second, small
// kernel (one workgroup per range) merges the pieces of those rows, in
// ascending range order, with the online-softmax merge rule (Lecture 16 "LLM
// Serving (1)" §3.3), and writes the zeros of rows with no tokens; the
// kernel boundary makes the pieces visible across XCDs.  The split depends
// only on logical block positions, so results are bit-identical under any
// physical block permutation.
#include "attn_core.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kD = 128;
// Prefetch ring depth of the balanced decode kernel (2 to 4 tiles per wave).
#ifndef PA_DECODE_SLOTS
#define PA_DECODE_SLOTS 2
#endif
constexpr int kSlots = PA_DECODE_SLOTS;
static_assert(kSlots >= 2 && kSlots <= 4, "decode ring depth out of range");
constexpr int kBS = 16;  // tokens per tile: the unit of the flat space, whatever the block size


// Range of workgroup gi: [range_begin(gi), range_begin(gi + 1)).
__device__ __forceinline__ int range_begin(int gi, int T, int G, int R) {
  if (R > 0) return (int)min((int64_t)gi * R, (int64_t)T);
  return (int)((int64_t)gi * T / G);
}

// Workgroup whose range holds flat block x.
__device__ __forceinline__ int range_of(int x, int T, int G, int R) {
  if (R > 0) return x / R;
  return (int)(((int64_t)(x + 1) * G + T - 1) / T) - 1;
}

// Number of ranges actually used: balanced ranges are never more than the
// blocks, so every range is non-empty and a row's pieces are exactly the
// ranges between its first and last block.
__device__ __forceinline__ int ranges_used(int grid, int T, int R) {
  return R > 0 ? grid : max(1, min(grid, T));
}

// Rows are (sequence, KV head) pairs, or, for a GQA group of more than 16
// query heads, (sub-group, KV head) pairs: each sequence then appears
// head_split times in a row (same length, same table) and its copy sub
// serves query heads sub * g .. sub * g + g - 1 of every group, g being the
// sub-group size (heads per row).  seq_of maps a row's sequence index vb to
// the caller's sequence, head0 gives the row's first query head.
__device__ __forceinline__ int seq_of(const DecodeParams &p, int vb) {
  return p.head_split > 1 ? vb / p.head_split : vb;
}
__device__ __forceinline__ int64_t head0(const DecodeParams &p, int vb, int kh, int g) {
  if (p.head_split <= 1) return (int64_t)vb * p.num_heads + (int64_t)kh * g;
  const int b = vb / p.head_split, sub = vb - b * p.head_split;
  return (int64_t)b * p.num_heads + ((int64_t)kh * p.head_split + sub) * g;
}

__device__ __forceinline__ void store_value(void *out, int out_bf16, int64_t i, float v) {
  if (out_bf16)
    reinterpret_cast<__bf16 *>(out)[i] = (__bf16)v;
  else
    reinterpret_cast<float *>(out)[i] = v;
}

// Two waves per SIMD: with the two-slot ring that is 16 tiles (128 KB of bf16
// K/V) in flight per CU.
//
// Inside a workgroup every wave owns a contiguous quarter of the range and
// streams it alone.  A row that lies wholly inside a wave's share is
// finalised in registers and written out; the (at most two) rows at the ends
// of a wave's share are parked in LDS and combined, in wave order, once all
// waves are done.  So no barrier interrupts the stream, and runs of short
// rows are spread evenly over the waves.
//
// FP8 (E4M3) caches: the ring carries the tiles as loaded (16 instead of 32
// registers each), expanded to bf16 just before their step; k_scale is
// folded into the score scale, v_scale into the final normalisation.
//
// MODE kFused computes its range's staging (the prologue below) itself;
// kPlanOnly runs only that prologue and writes the staging to a plan buffer;
// kPlanned loads the staging from such a plan in one memory round trip.  A
// plan depends only on seq_lens and the block tables, so one plan serves every
// layer of a decode step.
enum : int { kFused = 0, kPlanOnly = 1, kPlanned = 2 };

// Timestamp build (PAGED_ATTN_TIMELINE=1): the planned main kernel and the
// merge kernel record the s_memrealtime clock at fixed points of every
// workgroup, by hardware workgroup id, for pa_timeline (points listed in
// include/paged_attn.h).  The release build compiles none of it.
#if PAGED_ATTN_TIMELINE
#include "paged_attn.h"  // PA_TIMELINE_ROWS
static __device__ unsigned long long tl_main[PA_TIMELINE_ROWS][8];
static __device__ unsigned long long tl_merge[PA_TIMELINE_ROWS][2];
#define TL_MAIN(col, who)                                                          \
  do {                                                                             \
    if ((who) && blockIdx.x < PA_TIMELINE_ROWS)                                    \
      tl_main[blockIdx.x][(col)] = __builtin_amdgcn_s_memrealtime();               \
  } while (0)
#define TL_MERGE(col)                                                              \
  do {                                                                             \
    if (threadIdx.x == 0 && blockIdx.x < PA_TIMELINE_ROWS)                         \
      tl_merge[blockIdx.x][(col)] = __builtin_amdgcn_s_memrealtime();              \
  } while (0)
#else
#define TL_MAIN(col, who) \
  do {                    \
  } while (0)
#define TL_MERGE(col) \
  do {                \
  } while (0)
#endif

template <int NW, bool FP8, int MODE, bool APPEND = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_streamk_kernel(
    DecodeParams p) {
  static_assert(!APPEND || (MODE == kPlanned && !FP8), "the folded write serves planned bf16 calls");
  using F = KVFormat<FP8>;
  __shared__ int s_pref[MODE == kPlanned ? 1 : kStreamKMaxSeqs + 1];  // first flat block of each sequence
  __shared__ int s_len[MODE == kPlanned ? 1 : kStreamKMaxSeqs];       // clamped sequence lengths
  __shared__ int s_scan[64 * NW];
  __shared__ int2 s_rows[kStreamKTabCache];    // each position's tile rows 0 and 8, in 8-row
                                               //   units (x = -1: a table entry out of range)
  __shared__ int s_prow[kStreamKTabCache + 1]; // row (b * Hkv + kh) of each position, -1 past the end
  __shared__ int s_pj[kStreamKTabCache];       // block index inside the row
  __shared__ int2 s_ln[kStreamKTabCache];      // {sequence length, blocks of the row} of each position
  __shared__ int s_keep[kStreamKTabCache];     // 1: a neighbouring row uses the position's block
  __shared__ int64_t s_slot[APPEND ? kStreamKMaxSeqs : 1];  // APPEND: each sequence's new-token slot
  __shared__ int s_brow[NW][2];                // row start of each parked boundary state (-1: none)
  __shared__ int s_brid[NW][2];                // its row, b * Hkv + kh
  __shared__ int s_bnb[NW][2];                 // its blocks
  extern __shared__ float s_park[];            // [NW][2][g][kD + 2]: acc, then max and sum

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4, c = lane & 15;
  const int Hkv = p.num_kv_heads;
  const int B = p.num_seqs * max(p.head_split, 1);       // sequences of rows (seq_of)
  const int g = p.num_heads / Hkv / max(p.head_split, 1);  // query heads per row
  const int gi = (int)xcd_contiguous(blockIdx.x, gridDim.x);  // this workgroup's range
  const int R = p.sk_range_blocks;
  if constexpr (MODE == kPlanned) TL_MAIN(0, tid == 0);

  int T, G, s, e;
  if constexpr (MODE != kPlanned) {
    // -- flat index space: KV head major, then sequence, then tile ------------
    // (s_pref: exclusive prefix over sequences of tiles; a KV head's rows span
    // s_pref[B] positions).  Each XCD takes a contiguous run of ranges, so with
    // the heads outermost an XCD serves one or two KV heads of every
    // sequence: blocks that sequences share (a common prompt) are then read
    // from HBM about once, not once per XCD, and the rows that share a block
    // sit next to each other.
    if (B <= 64) {
      // one wave scans with cross-lane adds; a single barrier publishes it
      if (w == 0) {
        int L = lane < B ? p.seq_lens[seq_of(p, lane)] : 0;
        L = clamp_len(L, p.max_len_cap);
        const int v = (L + kBS - 1) / kBS;
        int incl = v;
  #pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int t = __shfl_up(incl, off, 64);
          incl += lane >= off ? t : 0;
        }
        if (lane < B) {
          s_len[lane] = L;
          s_pref[lane] = incl - v;
        }
        if (lane == (B > 0 ? B - 1 : 0)) s_pref[B] = B > 0 ? incl : 0;
      }
      if (tid < 2 * NW) s_brow[tid >> 1][tid & 1] = -1;
      __syncthreads();
    } else {
      const int nt = 64 * NW;
      const int per = (B + nt - 1) / nt;
      const int b0 = min(tid * per, B), b1 = min(b0 + per, B);
      int local = 0;
      for (int b = b0; b < b1; ++b) {
        int L = p.seq_lens[seq_of(p, b)];
        L = clamp_len(L, p.max_len_cap);
        s_len[b] = L;
        local += (L + kBS - 1) / kBS;
      }
      s_scan[tid] = local;
      if (tid < 2 * NW) s_brow[tid >> 1][tid & 1] = -1;
      __syncthreads();
      for (int off = 1; off < nt; off <<= 1) {
        const int v = tid >= off ? s_scan[tid - off] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
      }
      int run = s_scan[tid] - local;
      for (int b = b0; b < b1; ++b) {
        s_pref[b] = run;
        run += (s_len[b] + kBS - 1) / kBS;
      }
      if (tid == nt - 1) s_pref[B] = s_scan[tid];
      __syncthreads();
    }
    const int Th = s_pref[B];  // positions of one KV head (the host keeps Th * Hkv within int)
    T = Th * Hkv;
    G = ranges_used((int)gridDim.x, T, R);

    // no split row under this range's first position unless the staging
    // loop below says so
    if (tid == 0) p.sk_desc[gi] = int4{-1, 0, 0, 0};

    s = range_begin(gi, T, G, R);
    e = range_begin(gi + 1, T, G, R);
    if constexpr (MODE == kPlanOnly) {
      if (tid == 0) p.plan_hdr[gi] = int4{gi < G ? s : 0, gi < G ? e : 0, T, G};
    }
    if (gi >= G) return;
    if (s >= e || e - s > kStreamKTabCache) return;  // the planner keeps ranges within the cache

    const TileMap map(p.block_size, Hkv, p.num_blocks);
    // Stage, for every position of this range, where its tile's rows 0 and 8
    // start (element offsets / 1024, exact: both are multiples of 8 rows of
    // 128), its (sequence, KV head) row and its tile index inside the row (the
    // table loads of all positions issued together), so the streaming loop does
    // no searching and no tile load waits on a dependent table read.  The
    // planner keeps ranges within kStreamKTabCache positions; the host keeps a
    // cache below 2^41 elements, so the offsets / 1024 fit in 31 bits.
    for (int pos = s + tid; pos < e; pos += 64 * NW) {
      const int kh = pos / Th, rem = pos - kh * Th;  // pos < T, so Th > 0
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= rem) lo = mid; else hi = mid;
      }
      const int nb = s_pref[lo + 1] - s_pref[lo];
      const int j = rem - s_pref[lo];
      int e0, e1;
      const bool ok = map.entries(p.block_tables + (int64_t)seq_of(p, lo) * p.max_blocks_per_seq, j,
                                  (s_len[lo] + p.block_size - 1) / p.block_size, e0, e1);
      debug_report(!ok, kDbgBlockRange);
      const TileRows tr = map.rows(e0, e1, kh);
      // Mark a tile whose block the previous or the next sequence also uses at
      // the same place (forked or prefix-sharing sequences, which sit next to
      // each other in a batch): a wave share holding one loads with ordinary
      // loads, which keep it in the L2 for those rows; every other share
      // streams through the caches (non-temporal loads).
      int keep = 0;
      if (ok) {
        const int i0 = map.first_index(j), bsz = p.block_size;
        const int64_t mb = p.max_blocks_per_seq;
        if (lo > 0 && i0 < (s_len[lo - 1] + bsz - 1) / bsz)
          keep |= p.block_tables[seq_of(p, lo - 1) * mb + i0] == e0;
        if (lo + 1 < B && i0 < (s_len[lo + 1] + bsz - 1) / bsz)
          keep |= p.block_tables[seq_of(p, lo + 1) * mb + i0] == e0;
      }
      s_rows[pos - s] = ok ? int2{(int)(tr.lo >> 10), (int)(tr.hi >> 10)} : int2{-1, 0};
      s_prow[pos - s] = lo * Hkv + kh;
      s_pj[pos - s] = j;
      s_ln[pos - s] = int2{s_len[lo], nb};
      s_keep[pos - s] = keep;
      // the merge descriptor: the row under the range's first position, if
      // it began in an earlier range or goes on past this one, with its span
      // of ranges (same thread as the -1 written above: pos == s only for
      // tid 0).  A plan keeps it, so planned calls do no range arithmetic.
      if (pos == s && (j > 0 || s - j + nb > e)) {
        const int rs = s - j;
        const int g_first = min(max(range_of(rs, T, G, R), 0), gi);
        const int g_last = max(range_of(rs + nb - 1, T, G, R), gi);
        p.sk_desc[gi] = int4{lo * Hkv + kh, g_first, rs <= range_begin(g_first, T, G, R) ? 0 : 1, g_last};
      }
      if constexpr (MODE == kPlanOnly) {
        const int64_t at = (int64_t)gi * p.plan_stride + (pos - s);
        p.plan_rec[at] = int4{s_rows[pos - s].x, s_rows[pos - s].y, lo * Hkv + kh, j};
        p.plan_rec2[at] = int2{s_len[lo], nb | (keep ? kKeepTile : 0)};
      }
    }
    if constexpr (MODE == kPlanOnly) return;
    if (tid == 0) s_prow[e - s] = -1;
    __syncthreads();
  } else {
    // -- the staging from the plan: header and records in one round trip ----
    // (the merge descriptors are the plan's own: nothing to reset here)
    if (tid < 2 * NW) s_brow[tid >> 1][tid & 1] = -1;
    constexpr int kMaxPer = (kStreamKTabCache + 64 * NW - 1) / (64 * NW);
    const int4 h = p.plan_hdr[gi];
    int4 ra[kMaxPer];
    int2 rb[kMaxPer];
    // every load issued unconditionally (positions past the plan's stride
    // re-read its last record, unused), so none waits on another
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      const int li = min(tid + k * 64 * NW, p.plan_stride - 1);
      ra[k] = p.plan_rec[(int64_t)gi * p.plan_stride + li];
      rb[k] = p.plan_rec2[(int64_t)gi * p.plan_stride + li];
    }
    // APPEND: the slots of the step's new tokens, in the same round trip
    constexpr int kSlotPer = APPEND ? kStreamKMaxSeqs / (64 * NW) : 1;
    int64_t sv[kSlotPer];
    if constexpr (APPEND) {
#pragma unroll
      for (int k = 0; k < kSlotPer; ++k) {
        const int bi = tid + k * 64 * NW;
        sv[k] = bi < p.num_seqs ? p.slot_mapping[bi] : -1;  // (the folded write has one row per sequence)
      }
    }
    asm volatile("" ::: "memory");  // issue those loads before the header is tested
    if constexpr (APPEND) {
#pragma unroll
      for (int k = 0; k < kSlotPer; ++k)
        if (tid + k * 64 * NW < p.num_seqs) s_slot[tid + k * 64 * NW] = sv[k];
    }
    s = h.x;
    e = h.y;
    T = h.z;
    G = h.w;
    // (rows with no tokens get their zeros from the merge kernel, so this
    // prologue has one memory round trip: header and records)
    if (gi >= G || G > (int)gridDim.x || s < 0 || s >= e || e > T || e - s > p.plan_stride) return;
    // The plan is trusted for its values but not for its bounds: a record
    // whose tile lies outside the cache or whose row is not a (sequence, KV
    // head) row of this call is masked and charged to row 0, so a stale or
    // foreign plan gives wrong results, never an access out of bounds.
    const int64_t units = ((int64_t)p.num_blocks * Hkv * p.block_size * kD) >> 10;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      const int li = tid + k * 64 * NW;
      if (li < e - s) {
        const bool ok = ra[k].x >= -1 && ra[k].x < units && ra[k].y >= 0 && ra[k].y < units && ra[k].z >= 0 &&
                        ra[k].z < B * Hkv && ra[k].w >= 0;
        debug_report(!ok, kDbgPlan);
        s_rows[li] = ok ? int2{ra[k].x, ra[k].y} : int2{-1, 0};
        s_prow[li] = ok ? ra[k].z : 0;
        s_pj[li] = ok ? ra[k].w : 0;
        s_ln[li] = int2{rb[k].x, rb[k].y & ~kKeepTile};
        s_keep[li] = (rb[k].y & kKeepTile) != 0;
      }
    }
    if (tid == 0) s_prow[e - s] = -1;
    __syncthreads();
    TL_MAIN(1, tid == 0);
  }

  // this wave's share of the range, in local positions [ls, le)
  const int ls = (int)((int64_t)(e - s) * w / NW);
  const int le = (int)((int64_t)(e - s) * (w + 1) / NW);

  const float sl2 = p.scale * p.k_scale * kLog2e;
  const typename F::Elem *kc = reinterpret_cast<const typename F::Elem *>(p.k_cache);
  const typename F::Elem *vc = reinterpret_cast<const typename F::Elem *>(p.v_cache);
  const uint16_t *qbase = reinterpret_cast<const uint16_t *>(p.q);
  const bool col_ok = c < g;
  const int c_ld = c < g ? c : g - 1;  // idle columns read a valid row, never stored

  // A slot holds one tile and the q operand of its row, loaded together at
  // the same prefetch distance.  The q operand is loaded only when the slot's
  // previous occupant (position li - dist, dist = ring depth) belonged to
  // another row; otherwise the registers still hold this row's q.  An
  // out-of-range table entry is never dereferenced: the tile is read from
  // block 0 and fully masked.
  struct Slot {
    typename F::Raw t;
    bf16x8 q[4];
    int lim;
  };
  // Position li (< le) into slot sl.  The load kind is fixed for the share
  // (KIND 1 non-temporal, 2 ordinary), and q, when loaded, goes out before
  // the tile, so a slot's last loads are always its tile's and every path
  // issues the same ones (see the loop below).
  auto load_slot = [&](int li, Slot &sl, int dist, auto kind) __attribute__((always_inline)) {
    constexpr bool STREAM = decltype(kind)::value == 1;
    const int lp = li - dist;
    const int2 u = s_rows[li];
    const int row = s_prow[li];
    const int b = row / Hkv, kh = row - b * Hkv;
    const bool ok = u.x >= 0;
    const bool need_q = lp < ls || s_prow[lp < le ? lp : le - 1] != row;  // uniform
    if (__builtin_amdgcn_readfirstlane((int)need_q))
      F::load_q(sl.q, qbase + (head0(p, b, kh, g) + c_ld) * kD, r);
    sl.lim = ok ? s_ln[li].x : 0;
    // a masked tile reads the first rows of the cache
    const TileRows tr{(int64_t)max(u.x, 0) << 10, (int64_t)u.y << 10};
    if constexpr (APPEND) {
      // A row's last tile holds position L - 1; when the caller's slot for
      // the sequence's new token names that place, the lanes that hold that
      // token read the new K/V row in its stead (the same load instructions
      // for every tile).  (Block sizes of this path are powers of two.)
      int tpos = -1;
      const int2 ln = s_ln[li];
      if (ok && s_pj[li] == ln.y - 1) {  // uniform: the position's record
        const int at_pos = (ln.x - 1) & 15;
        const int64_t at = (at_pos < 8 ? tr.lo : tr.hi) + (at_pos & 7) * kD;
        const int64_t sm = s_slot[b];
        const int lb = __builtin_ctz((unsigned)p.block_size);
        if (sm >= 0 && sm < ((int64_t)p.num_blocks << lb) &&
            ((((sm >> lb) * Hkv + kh) << lb) + (sm & (p.block_size - 1))) * kD == at)
          tpos = at_pos;
      }
      load_kv_tile_rows_subst_as<STREAM>(
          sl.t, kc, vc, tr, r, c, tpos,
          reinterpret_cast<const uint16_t *>(p.new_k) + ((int64_t)b * Hkv + kh) * kD,
          reinterpret_cast<const uint16_t *>(p.new_v) + ((int64_t)b * Hkv + kh) * kD);
    } else {
      F::template load_as<STREAM>(sl.t, kc, vc, tr, r, c);
    }
  };

  if (ls < le) {
    MfmaAttnState st;
    st.init();
    int slot_used = 0;
    int seg_j0 = s_pj[ls];  // first block of the current row inside this share
    // close the current row if position li was its last one in the share
    auto after_step = [&](int li) {
      const int row = s_prow[li];
      const bool row_end = li + 1 == le || s_prow[li + 1] != row;
      if (!row_end) return;
      const int b = row / Hkv, kh = row - b * Hkv;
      const int nb = s_ln[li].y;
      const float lw = row_sum4(st.l);
      const bool whole = seg_j0 == 0 && s_pj[li] == nb - 1;
      if (whole) {
        if (col_ok) {
          const float inv = lw > 0.f ? p.v_scale / lw : 0.f;
          const int64_t orow = (head0(p, b, kh, g) + c) * kD;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
              store_value(p.out, p.out_bf16, orow + 32 * r + 8 * i + jj, st.acc[jj][i] * inv);
        }
      } else {
        // a wave has at most two boundary rows: its first and its last
        // (the bound only matters for a plan that is not this call's)
        const int k = slot_used < 2 ? slot_used++ : 1;
        float *pc = s_park + (((size_t)w * 2 + k) * g + (col_ok ? c : 0)) * (kD + 2);
        if (col_ok) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) pc[32 * r + 8 * i + jj] = st.acc[jj][i];
          if (r == 0) {
            pc[kD] = st.m;
            pc[kD + 1] = lw;
          }
        }
        if (lane == 0) {
          s_brow[w][k] = s + li - s_pj[li];  // flat index of the row's first block
          s_brid[w][k] = row;
          s_bnb[w][k] = nb;
        }
      }
      if (li + 1 == le) return;
      seg_j0 = s_pj[li + 1];
      st.init();
    };
    // kSlots fixed register slots: position li lives in slot (li - ls) mod
    // kSlots, so no tile register is copied while its load is in flight.  Two
    // slots (one tile computed while the next one loads) keep about 128 KB in
    // flight per CU.  The share's last NS - 1 positions, which load nothing,
    // run apart, so every other step follows the same loads: each slot's
    // tile loads are the last it issues, on every path, and the compiler's
    // wait before a step covers that step's own tile only, leaving the later
    // NS - 1 tiles in flight.  (A branch between two load sequences, or a
    // path that loads nothing, makes its counting merge paths with different
    // numbers of loads in flight, and it then waits for all of them, the next
    // tile's prefetch included.)  So the load kind is one for the share:
    // ordinary loads throughout when any of its tiles is marked as shared
    // with a neighbouring row, else non-temporal ones.
    bool keep_any = false;
    for (int k = ls + lane; k < le; k += 64) keep_any |= s_keep[k] != 0;
    auto run = [&](auto kind) __attribute__((always_inline)) {
      constexpr int NS = kSlots;
      Slot s[NS];
#pragma unroll
      for (int i = 0; i < NS - 1; ++i)
        if (ls + i < le) load_slot(ls + i, s[i], NS, kind);
      auto one = [&](int li, auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        load_slot(li + NS - 1, s[(k + NS - 1) % NS], NS, kind);
        st.step(s[k].q, F::expand(s[k].t), s_pj[li] * kBS, s[k].lim, sl2, r);
        after_step(li);
      };
      // positions li .. le - 1 (fewer than NS of them), from slot k on
      auto last = [&](int li, auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
#pragma unroll
        for (int j = 0; j < NS - 1; ++j) {
          if (li + j < le) {
            Slot &sj = s[(k + j) % NS];
            st.step(sj.q, F::expand(sj.t), s_pj[li + j] * kBS, sj.lim, sl2, r);
            after_step(li + j);
          }
        }
      };
      using E0 = std::integral_constant<int, 0>;
      using E1 = std::integral_constant<int, 1 % NS>;
      using E2 = std::integral_constant<int, 2 % NS>;
      using E3 = std::integral_constant<int, 3 % NS>;
      for (int li = ls;; li += NS) {
        if (li + NS - 1 >= le) {
          last(li, E0());
          break;
        }
        one(li, E0());
        if (li + NS >= le) {
          last(li + 1, E1());
          break;
        }
        one(li + 1, E1());
        if constexpr (NS > 2) {
          if (li + NS + 1 >= le) {
            last(li + 2, E2());
            break;
          }
          one(li + 2, E2());
        }
        if constexpr (NS > 3) {
          if (li + NS + 2 >= le) {
            last(li + 3, E3());
            break;
          }
          one(li + 3, E3());
        }
      }
    };
    if (__builtin_amdgcn_ballot_w64(keep_any) == 0)
      run(std::integral_constant<int, 1>());
    else
      run(std::integral_constant<int, 2>());
  }
  if constexpr (MODE == kPlanned) TL_MAIN(2 + (w & 3), lane == 0);
  __syncthreads();
  if constexpr (MODE == kPlanned) TL_MAIN(6, tid == 0);

  // -- combine the parked boundary rows, in wave order -----------------------
  // The 2 * NW entries (w, k), in order, form runs of equal row start, one
  // run per row.  Every thread reads all entries at once and walks the runs
  // in the same order; for each of its output elements it loads the members'
  // max, sum and partial value together and combines them in entry order.
  constexpr int NE = 2 * NW;
  int ers[NE], erow[NE], enb[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    ers[i] = s_brow[i >> 1][i & 1];
    erow[i] = s_brid[i >> 1][i & 1];
    enb[i] = s_bnb[i >> 1][i & 1];
  }
  int prev_rs = -1;
#pragma unroll
  for (int h = 0; h < NE; ++h) {
    const int rs = ers[h];
    if (rs < 0 || rs == prev_rs) continue;  // empty, or inside the current run
    prev_rs = rs;
    const int row = erow[h];
    const int b = row / Hkv, kh = row - b * Hkv;
    const int nb = enb[h];
    const bool whole = rs >= s && rs + nb <= e;
    const int slot = rs <= s ? 0 : 1;
    const int64_t out_row0 = head0(p, b, kh, g);
    // the run's members: the entries from h on with this row start (a bit
    // mask, uniform; empty entries may sit between members).  Most runs have
    // one member: a row that only touches one wave's share.
    unsigned mem = 0;
#pragma unroll
    for (int i = h; i < NE; ++i) mem |= (ers[i] == rs ? 1u : 0u) << i;
    const bool single = (mem & (mem - 1)) == 0;
    // Two output elements per thread and pass (all of them at g <= 4), so
    // that the members' LDS reads of both go out together.
    constexpr int kPer = 2;
    for (int idx0 = tid; idx0 < g * kD; idx0 += kPer * 64 * NW) {
      float M[kPer], lsum[kPer], o[kPer];
      int cc[kPer], d[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int idx = min(idx0 + u * 64 * NW, g * kD - 1);  // a past-the-end element repeats the last one
        cc[u] = idx / kD;
        d[u] = idx - cc[u] * kD;
      }
      if (single) {
        // weight exp2(0) = 1 (an all-masked entry carries zero sum and output)
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const float *pc = s_park + ((size_t)h * g + cc[u]) * (kD + 2);
          M[u] = pc[kD];
          lsum[u] = pc[kD + 1];
          o[u] = pc[d[u]];
        }
      } else {
        float mv[NE][kPer], lv[NE][kPer], ov[NE][kPer];
#pragma unroll
        for (int i = h; i < NE; ++i) {
          if ((mem >> i) & 1u) {
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
              const float *pc = s_park + ((size_t)i * g + cc[u]) * (kD + 2);
              mv[i][u] = pc[kD];
              lv[i][u] = pc[kD + 1];
              ov[i][u] = pc[d[u]];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          float Mx = kNegInf;
#pragma unroll
          for (int i = h; i < NE; ++i)
            if ((mem >> i) & 1u) Mx = fmaxf(Mx, mv[i][u]);
          const float M_use = Mx == kNegInf ? 0.f : Mx;
          float ls = 0.f, ov_ = 0.f;
#pragma unroll
          for (int i = h; i < NE; ++i) {
            if ((mem >> i) & 1u) {
              const float wgt = fast_exp2(mv[i][u] - M_use);
              ls += lv[i][u] * wgt;
              ov_ += ov[i][u] * wgt;
            }
          }
          M[u] = Mx;
          lsum[u] = ls;
          o[u] = ov_;
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (idx0 + u * 64 * NW >= g * kD) continue;
        if (whole) {
          store_value(p.out, p.out_bf16, (out_row0 + cc[u]) * kD + d[u],
                      lsum[u] > 0.f ? o[u] * p.v_scale / lsum[u] : 0.f);
        } else {
          const int64_t base = ((int64_t)gi * 2 + slot) * g + cc[u];
          p.sk_part[base * kD + d[u]] = o[u];
          if (d[u] == 0) {
            p.sk_ml[base * 2 + 0] = M[u];
            p.sk_ml[base * 2 + 1] = lsum[u];
          }
        }
      }
    }
  }
  if constexpr (MODE == kPlanned) TL_MAIN(7, tid == 0);
}

// One workgroup per range gi; its descriptor names the split row under the
// range's first position, if any, and that row's span of ranges.  A row of
// at most kShortRow pieces is merged, in ascending range order, by the
// workgroup of its last range, a thread owning output elements (column,
// dim).  Most split rows have exactly two pieces -- the end of range gi - 1
// and the start of range gi -- so those are loaded together with the
// descriptor, in one memory round trip; rows with more pieces take a second
// one.  A longer row (few rows cut over many ranges) is shared out: its
// output elements are cut into chunks of cw consecutive elements, dealt to
// the ranges whose first piece is the row's, and inside a workgroup the
// pieces are dealt to the threads (kBatch per memory round trip) and the
// per-thread results combined through LDS, so no workgroup walks all the
// pieces alone.  The merge rule is associative, so the grouping changes only
// the rounding.
//
// APPEND: the workgroups also write the step's new K/V rows to their slots
// (row gi, gi + grid, ...), after every read of the main kernel, as
// kv_cache_write does: slot < 0 or past the cache skips the row.
template <bool APPEND>
__global__ __launch_bounds__(1024) void decode_streamk_merge_kernel(DecodeParams p) {
  TL_MERGE(0);
  constexpr int kBatch = 8;
  constexpr int kShortRow = 8;
  constexpr int kPer = 2;  // the launch uses max(g * kD / 2, 256) threads: two elements each
  __shared__ float s_m[1024], s_l[1024], s_o[1024];
  // the same range numbering as the main kernel, so this workgroup runs on
  // the XCD that wrote range gi's pieces (and, but at XCD edges, gi - 1's)
  const int gi = (int)xcd_contiguous(blockIdx.x, gridDim.x);
  const int hs = max(p.head_split, 1);
  const int g = p.num_heads / p.num_kv_heads / hs;  // query heads per row
  const int gp = gi > 0 ? gi - 1 : 0;
  const int4 dsc = p.sk_desc[gi];
  const int nrows = p.num_seqs * hs * p.num_kv_heads;
  const int nreal = p.num_seqs * p.num_kv_heads;  // (sequence, KV head) rows: the folded write's
  const int len0 = gi < nrows ? p.seq_lens[seq_of(p, gi / p.num_kv_heads)] : 1;  // with the descriptor: one round trip
  // speculative: (gp, slot 0), (gp, slot 1), (gi, slot 0) for both elements
  const int E = g * kD;  // output elements of a row
  float sm[3][kPer], sl[3][kPer], so[3][kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int idx = min((int)threadIdx.x + u * (int)blockDim.x, E - 1);
    const int cc = idx / kD, d = idx - cc * kD;
    const int64_t pc[3] = {((int64_t)gp * 2 + 0) * g + cc, ((int64_t)gp * 2 + 1) * g + cc, ((int64_t)gi * 2) * g + cc};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      sm[k][u] = p.sk_ml[pc[k] * 2];
      sl[k][u] = p.sk_ml[pc[k] * 2 + 1];
      so[k][u] = p.sk_part[pc[k] * kD + d];
    }
  }
  // APPEND: row gi's new K (threads 0 .. 15) or V (16 .. 31) chunk and its
  // slot, loaded with the rest
  int64_t wsm = -1;
  u32x4 wdat = {0u, 0u, 0u, 0u};
  const int wpart = threadIdx.x / (kD / 8), wch = threadIdx.x % (kD / 8);
  if constexpr (APPEND) {
    if (gi < nreal && threadIdx.x < 2 * (kD / 8)) {
      wsm = p.slot_mapping[gi / p.num_kv_heads];
      wdat = ld16(reinterpret_cast<const uint16_t *>(wpart ? p.new_v : p.new_k) + (int64_t)gi * kD + 8 * wch);
    }
  }
  asm volatile("" ::: "memory");  // keep those loads ahead of the branch below
  // rows with no tokens (no piece, no range) get zeros, spread over the
  // workgroups: row gi, gi + grid, ...
  for (int zr = gi; zr < nrows; zr += (int)gridDim.x) {
    if (clamp_len(zr == gi ? len0 : p.seq_lens[seq_of(p, zr / p.num_kv_heads)], p.max_len_cap) != 0) continue;
    const int b = zr / p.num_kv_heads, kh = zr - b * p.num_kv_heads;
    for (int idx = threadIdx.x; idx < g * kD; idx += blockDim.x)
      store_value(p.out, p.out_bf16, head0(p, b, kh, g) * kD + idx, 0.f);
  }
  if constexpr (APPEND) {
    // rows gi, gi + grid, ...: 16-byte chunks, threads 0 .. 15 the K row,
    // 16 .. 31 the V row (block sizes of this path are powers of two)
    const int lb = __builtin_ctz((unsigned)p.block_size);
    const int64_t nslots = (int64_t)p.num_blocks << lb;
    for (int wr = gi; wr < nreal; wr += (int)gridDim.x) {
      if (threadIdx.x >= 2 * (kD / 8)) break;
      const int kh = wr % p.num_kv_heads;
      int64_t sm = wsm;
      u32x4 dat = wdat;
      if (wr != gi) {  // beyond the first row: loaded here
        sm = p.slot_mapping[wr / p.num_kv_heads];
        dat = ld16(reinterpret_cast<const uint16_t *>(wpart ? p.new_v : p.new_k) + (int64_t)wr * kD + 8 * wch);
      }
      if (sm < 0 || sm >= nslots) continue;
      const int64_t dst = ((((sm >> lb) * p.num_kv_heads + kh) << lb) + (sm & (p.block_size - 1))) * kD;
      uint16_t *cache = reinterpret_cast<uint16_t *>(const_cast<void *>(wpart ? p.v_cache : p.k_cache));
      st16(cache + dst + 8 * wch, dat);
    }
  }
  // a planned call's descriptors come from the plan: trusted for their
  // values, not for their bounds (a stale or foreign plan gives wrong
  // results, never an access out of bounds)
  const int row = dsc.x;
  if (row < 0 || row >= nrows) {
    TL_MERGE(1);
    return;
  }
  const int g_first = min(max(dsc.y, 0), gi), s_first = dsc.z & 1;
  const int g_last = min(max(dsc.w, gi), (int)gridDim.x - 1), nc = g_last - g_first + 1;
  const int b = row / p.num_kv_heads, kh = row - b * p.num_kv_heads;
  const int64_t out_row0 = head0(p, b, kh, g);
  auto piece = [&](int k, int cc) -> int64_t {  // (range, slot, column) index of piece k
    return ((int64_t)(g_first + k) * 2 + (k == 0 ? s_first : 0)) * g + cc;
  };
  if (nc > kShortRow) {
    // chunk width: 64 elements, halved (down to 16) while every chunk still
    // finds a workgroup; the workgroups are the ranges g_first + s_first ..
    // g_last (a stale descriptor can give qi < 0: that workgroup idles)
    const int q0 = g_first + s_first, nw = g_last - q0 + 1, qi = gi - q0;
    int cw = 64;
    while (cw > 16 && E / (cw / 2) <= nw) cw >>= 1;
    const int nchunk = E / cw, lanes = (int)blockDim.x / cw;
    const int el = (int)threadIdx.x % cw, ln = (int)threadIdx.x / cw;
    for (int c = qi < 0 ? nchunk : qi; c < nchunk; c += nw) {
      const int idx = c * cw + el, cc = idx / kD, d = idx - cc * kD;
      float M = kNegInf, lsum = 0.f, o = 0.f;
      for (int k0 = ln; k0 < nc; k0 += lanes * kBatch) {
        float pm[kBatch], pl[kBatch], po[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int kk = k0 + k * lanes;
          const int64_t pc = piece(min(kk, nc - 1), cc);
          pm[k] = kk < nc ? p.sk_ml[pc * 2] : kNegInf;
          pl[k] = p.sk_ml[pc * 2 + 1];
          po[k] = p.sk_part[pc * kD + d];
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) Mb = fmaxf(Mb, pm[k]);
        const float Mu = Mb == kNegInf ? 0.f : Mb;
        const float cf = fast_exp2(M - Mu);
        lsum *= cf;
        o *= cf;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const float wgt = fast_exp2(pm[k] - Mu);
          lsum += pl[k] * wgt;
          o += po[k] * wgt;
        }
        M = Mb;
      }
      s_m[threadIdx.x] = M;
      s_l[threadIdx.x] = lsum;
      s_o[threadIdx.x] = o;
      __syncthreads();
      if (ln == 0) {
        float Mt = kNegInf;
        for (int t = 0; t < lanes; ++t) Mt = fmaxf(Mt, s_m[t * cw + el]);
        const float Mu = Mt == kNegInf ? 0.f : Mt;
        float lt = 0.f, ot = 0.f;
        for (int t = 0; t < lanes; ++t) {
          const float wgt = fast_exp2(s_m[t * cw + el] - Mu);
          lt += s_l[t * cw + el] * wgt;
          ot += s_o[t * cw + el] * wgt;
        }
        store_value(p.out, p.out_bf16, (out_row0 + cc) * kD + d, lt > 0.f ? ot * p.v_scale / lt : 0.f);
      }
      __syncthreads();
    }
    TL_MERGE(1);
    return;
  }
  if (gi != g_last) {  // a short row is merged by its last range
    TL_MERGE(1);
    return;
  }
  if (nc == 2) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = threadIdx.x + u * blockDim.x;
      if (idx >= E) continue;
      const int cc = idx / kD, d = idx - cc * kD;
      const int f = s_first;  // first piece: (gi - 1, s_first); second: (gi, 0)
      const float m0 = sm[f][u], m1 = sm[2][u];
      const float M = fmaxf(m0, m1);
      const float Mu = M == kNegInf ? 0.f : M;
      const float w0 = fast_exp2(m0 - Mu), w1 = fast_exp2(m1 - Mu);
      const float ls = sl[f][u] * w0 + sl[2][u] * w1;
      const float o = so[f][u] * w0 + so[2][u] * w1;
      store_value(p.out, p.out_bf16, (out_row0 + cc) * kD + d, ls > 0.f ? o * p.v_scale / ls : 0.f);
    }
    TL_MERGE(1);
    return;
  }
  for (int idx = threadIdx.x; idx < E; idx += blockDim.x) {
    const int cc = idx / kD, d = idx - cc * kD;
    float M = kNegInf, lsum = 0.f, o = 0.f;
    for (int k0 = 0; k0 < nc; k0 += kBatch) {
      float pm[kBatch], pl[kBatch], po[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int kk = min(k0 + k, nc - 1);
        const int64_t pc = piece(kk, cc);
        pm[k] = k0 + k < nc ? p.sk_ml[pc * 2] : kNegInf;
        pl[k] = p.sk_ml[pc * 2 + 1];
        po[k] = p.sk_part[pc * kD + d];
      }
      float Mb = M;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) Mb = fmaxf(Mb, pm[k]);
      const float Mu = Mb == kNegInf ? 0.f : Mb;
      const float cf = fast_exp2(M - Mu);  // rescale what came before (0 at the start)
      lsum *= cf;
      o *= cf;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float wgt = fast_exp2(pm[k] - Mu);  // 0 for the padding entries
        lsum += pl[k] * wgt;
        o += po[k] * wgt;
      }
      M = Mb;
    }
    store_value(p.out, p.out_bf16, (out_row0 + cc) * kD + d, lsum > 0.f ? o * p.v_scale / lsum : 0.f);
  }
  TL_MERGE(1);
}

}  // namespace

#if PAGED_ATTN_DEBUG
PA_DEBUG_WORD_ACCESSOR(debug_word_streamk)
#endif

#if PAGED_ATTN_TIMELINE
hipError_t timeline_symbols(void **main_stamps, void **merge_stamps) {
  const hipError_t e = hipGetSymbolAddress(main_stamps, HIP_SYMBOL(tl_main));
  if (e != hipSuccess) return e;
  return hipGetSymbolAddress(merge_stamps, HIP_SYMBOL(tl_merge));
}
#endif

hipError_t launch_decode_streamk_plan(const DecodeParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_streamk_kernel<PA_DECODE_WAVES, false, kPlanOnly>), dim3(p.sk_ranges),
                     dim3(64 * PA_DECODE_WAVES), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_streamk(const DecodeParams &p, hipStream_t stream) {
  const int g = p.num_heads / p.num_kv_heads / std::max(p.head_split, 1);  // query heads per row
  const size_t park = (size_t)PA_DECODE_WAVES * 2 * g * (kD + 2) * sizeof(float);
  const dim3 grid(p.sk_ranges), block(64 * PA_DECODE_WAVES);
  const bool planned = p.plan_hdr != nullptr;
  if (p.new_k) {
    // the step's write folded in (planned bf16 calls only; the caller checks)
    hipLaunchKernelGGL((decode_streamk_kernel<PA_DECODE_WAVES, false, kPlanned, true>), grid, block, park, stream,
                       p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_streamk_merge_kernel<true>, dim3(p.sk_ranges), dim3(std::max(g * kD / 2, 256)), 0, stream, p);
    return hipGetLastError();
  }
  if (p.kv_fp8 && planned)
    hipLaunchKernelGGL((decode_streamk_kernel<PA_DECODE_WAVES, true, kPlanned>), grid, block, park, stream, p);
  else if (p.kv_fp8)
    hipLaunchKernelGGL((decode_streamk_kernel<PA_DECODE_WAVES, true, kFused>), grid, block, park, stream, p);
  else if (planned)
    hipLaunchKernelGGL((decode_streamk_kernel<PA_DECODE_WAVES, false, kPlanned>), grid, block, park, stream, p);
  else
    hipLaunchKernelGGL((decode_streamk_kernel<PA_DECODE_WAVES, false, kFused>), grid, block, park, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_streamk_merge_kernel<false>, dim3(p.sk_ranges), dim3(std::max(g * kD / 2, 256)), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
