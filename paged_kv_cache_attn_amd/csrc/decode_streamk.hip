// decode_streamk.hip -- balanced ("stream-K") paged decode on gfx950.
//
// Same arithmetic as the MFMA decode tile step (attn_core.h), different work
// split.  The blocks of all (sequence, KV head) rows are laid end to end in
// one flat index space (sequence-major, then KV head, then logical block) and
// cut into equal contiguous ranges, one per workgroup, so every workgroup
// streams the same number of 8 KB K+V tiles whatever the length mix.  A
// range covers whole rows (whose output it writes directly) and at most two
// partial rows at its ends.  Each partial row leaves (max, sum, unnormalised
// output) in the workspace; the contributor that arrives last -- decided by
// a per-row atomic ticket -- merges the partials in ascending range order
// with the online-softmax merge rule (Lecture 16 "LLM Serving (1)" §3.3) and
// writes the row.  The split depends only on logical block positions, so
// results are bit-identical under any physical block permutation, and there
// is no second kernel launch.
//
// Tickets are 64-bit words (call generation << 32 | arrivals); a word whose
// generation differs from the current call's counts as zero arrivals, so the
// workspace needs no clearing between calls.
//
// Cross-workgroup hand-off without cache maintenance.  MI355X's eight XCDs
// each have their own L2, which are not coherent with one another for plain
// accesses; an agent-scope fence therefore writes back and invalidates the
// whole L2 and costs microseconds.  Instead every partial is written with an
// agent-scope atomic store (global_store ... sc1, written through to the
// level all XCDs share), the stores are drained (s_waitcnt vmcnt(0)) before
// the workgroup takes its ticket, and the merging workgroup reads the
// partials with agent-scope atomic loads (global_load ... sc1), which do not
// hit stale L2 lines.  No plain access ever touches the partials.
#include "attn_core.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kD = 128;
constexpr int kBS = 16;
constexpr int kStreamKTabCache = 1024;  // block-table entries staged per range

struct SegInfo {
  int b, kh;
  int nb;          // blocks of the row
  int row_start;   // flat index of the row's block 0
  int j0, j1;      // blocks [j0, j1) of the row inside this range
  int flat_end;    // flat index just past the segment
};

// Agent-scope relaxed atomics: coherent across XCDs without L2 maintenance.
__device__ __forceinline__ void coherent_store(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Two waves per SIMD: with the three-slot ring that is 16 tiles (128 KB) in
// flight per CU, enough to cover HBM latency at full bandwidth.
template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_streamk_kernel(
    DecodeParams p) {
  __shared__ int s_pref[kStreamKMaxSeqs + 1];  // first flat block of each sequence
  __shared__ int s_len[kStreamKMaxSeqs];       // clamped sequence lengths
  __shared__ int s_scan[64 * NW];
  __shared__ int s_tab[kStreamKTabCache];      // physical block of flat positions s..
  __shared__ float sm_o[NW][16][kD];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4, c = lane & 15;
  const int B = p.num_seqs, Hkv = p.num_kv_heads;
  const int g = p.num_heads / Hkv;
  const int gi = blockIdx.x;
  const int R = p.sk_range_blocks;

  // -- flat index space: exclusive prefix over sequences of blocks * Hkv ----
  {
    const int nt = 64 * NW;
    const int per = (B + nt - 1) / nt;
    const int b0 = min(tid * per, B), b1 = min(b0 + per, B);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
      int L = p.seq_lens[b];
      L = L < 0 ? 0 : (L > p.max_len_cap ? p.max_len_cap : L);
      s_len[b] = L;
      local += ((L + kBS - 1) / kBS) * Hkv;
    }
    s_scan[tid] = local;
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
      run += ((s_len[b] + kBS - 1) / kBS) * Hkv;
    }
    if (tid == nt - 1) s_pref[B] = s_scan[tid];
    __syncthreads();
  }
  const int T = s_pref[B];
  // Balanced ranges: no more ranges than blocks, so every range is non-empty
  // and the contributors of a row are exactly the ranges between its first and
  // last block.  Workgroups past the last range only write zero rows.
  const int G = R > 0 ? (int)gridDim.x : max(1, min((int)gridDim.x, T));

  // -- rows with no tokens get zeros (spread over the workgroups) -----------
  for (int row = gi; row < B * Hkv; row += (int)gridDim.x) {
    const int b = row / Hkv, kh = row - b * Hkv;
    if (s_len[b] != 0) continue;
    for (int idx = tid; idx < g * kD; idx += 64 * NW) {
      const int64_t o = ((int64_t)b * p.num_heads + (int64_t)kh * g) * kD + idx;
      if (p.out_bf16)
        reinterpret_cast<__bf16 *>(p.out)[o] = (__bf16)0.f;
      else
        reinterpret_cast<float *>(p.out)[o] = 0.f;
    }
  }

  if (gi >= G) return;
  const int s = range_begin(gi, T, G, R);
  const int e = range_begin(gi + 1, T, G, R);
  if (s >= e) return;

  auto seg_at = [&](int pos) -> SegInfo {
    // largest b with s_pref[b] <= pos (s_pref[B] = T > pos); wave-uniform
    int lo = 0, hi = B;  // invariant: s_pref[lo] <= pos < s_pref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= pos) lo = mid; else hi = mid;
    }
    SegInfo S;
    S.b = __builtin_amdgcn_readfirstlane(lo);
    const int p0 = __builtin_amdgcn_readfirstlane(s_pref[S.b]);
    S.nb = (__builtin_amdgcn_readfirstlane(s_pref[S.b + 1]) - p0) / Hkv;
    S.kh = (pos - p0) / S.nb;
    S.row_start = p0 + S.kh * S.nb;
    S.j0 = pos - S.row_start;
    S.j1 = min(e, S.row_start + S.nb) - S.row_start;
    S.flat_end = S.row_start + S.j1;
    return S;
  };

  // Stage the physical block ids of this range in LDS (one load per block,
  // issued together), so no tile load waits on a dependent table read.
  const bool tab_cached = e - s <= kStreamKTabCache;
  if (tab_cached) {
    for (int pos = s + tid; pos < e; pos += 64 * NW) {
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= pos) lo = mid; else hi = mid;
      }
      const int nb = (s_pref[lo + 1] - s_pref[lo]) / Hkv;
      const int j = (pos - s_pref[lo]) % nb;
      s_tab[pos - s] = p.block_tables[(int64_t)lo * p.max_blocks_per_seq + j];
    }
  }
  __syncthreads();

  // This wave's blocks: in every segment, j0 + w, j0 + w + NW, ... < j1.
  // A cursor is (segment, j); `valid` false past the range.
  struct Cursor {
    SegInfo S;
    int j;
    bool valid;
  };
  auto first_in = [&](SegInfo S) -> Cursor {
    Cursor cu;
    while (true) {
      if (S.j0 + w < S.j1) {
        cu.S = S;
        cu.j = S.j0 + w;
        cu.valid = true;
        return cu;
      }
      if (S.flat_end >= e) {
        cu.valid = false;
        return cu;
      }
      S = seg_at(S.flat_end);
    }
  };
  auto advance = [&](const Cursor &cu) -> Cursor {
    if (cu.j + NW < cu.S.j1) {
      Cursor n = cu;
      n.j += NW;
      return n;
    }
    if (cu.S.flat_end >= e) {
      Cursor n;
      n.valid = false;
      return n;
    }
    return first_in(seg_at(cu.S.flat_end));
  };

  const float sl2 = p.scale * kLog2e;
  const uint16_t *kc = reinterpret_cast<const uint16_t *>(p.k_cache);
  const uint16_t *vc = reinterpret_cast<const uint16_t *>(p.v_cache);
  const uint16_t *qbase = reinterpret_cast<const uint16_t *>(p.q);
  const int64_t blk_stride = (int64_t)Hkv * kBS * kD;
  const bool col_ok = c < g;

  struct Slot {
    KVTile t;
    int lim;
  };
  auto load_slot = [&](const Cursor &cu, Slot &sl) {
    const int pos = cu.S.row_start + cu.j;
    int phys = tab_cached ? s_tab[pos - s] : p.block_tables[(int64_t)cu.S.b * p.max_blocks_per_seq + cu.j];
    const bool ok = (unsigned)phys < (unsigned)p.num_blocks;
    sl.lim = ok ? s_len[cu.S.b] : 0;
    phys = ok ? phys : 0;
    const int64_t base = phys * blk_stride + (int64_t)cu.S.kh * kBS * kD;
    load_kv_tile_d128(sl.t, kc + base, vc + base, r, c);
  };
  auto load_q = [&](const SegInfo &Sg, bf16x8 *qo) {
    load_q_operand_d128(
        qo, col_ok ? qbase + ((int64_t)Sg.b * p.num_heads + (int64_t)Sg.kh * g + c) * kD : nullptr, r);
  };
  Cursor none;
  none.valid = false;

  // q of the current and of the next segment (double-buffered); K/V tiles in
  // a ring of three slots, so two tiles are in flight while one is used.
  MfmaAttnState st;
  SegInfo S = seg_at(s);
  bf16x8 qc[4], qn[4];
  load_q(S, qc);
  bool has_next = S.flat_end < e;
  SegInfo Sn = S;
  if (has_next) {
    Sn = seg_at(S.flat_end);
    load_q(Sn, qn);
  }
  Cursor c0 = first_in(S);
  Cursor c1 = c0.valid ? advance(c0) : none;
  Slot s0, s1, s2;
  if (c0.valid) load_slot(c0, s0);
  if (c1.valid) load_slot(c1, s1);

  while (true) {
    st.init();
    while (c0.valid && c0.S.row_start == S.row_start) {
      const Cursor c2 = c1.valid ? advance(c1) : none;
      if (c2.valid) load_slot(c2, s2);
      st.step(qc, s0.t, c0.j * kBS, s0.lim, sl2, r);
      c0 = c1;
      c1 = c2;
      s0 = s1;
      s1 = s2;
    }

    // -- merge the waves' states for segment S ------------------------------
    const float lw = row_sum4(st.l);
    if (col_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sm_o[w][c][32 * r + 8 * i + jj] = st.acc[jj][i];
      if (r == 0) {
        sm_m[w][c] = st.m;
        sm_l[w][c] = lw;
      }
    }
    __syncthreads();
    const bool whole = S.j0 == 0 && S.j1 == S.nb;
    const int row = S.b * Hkv + S.kh;
    const int64_t out_row0 = (int64_t)S.b * p.num_heads + (int64_t)S.kh * g;
    const int slot = S.row_start <= s ? 0 : 1;
    for (int idx = tid; idx < g * kD; idx += 64 * NW) {
      const int cc = idx / kD, d = idx - cc * kD;
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
      if (whole) {
        const float v = lsum > 0.f ? o / lsum : 0.f;
        const int64_t oi = (out_row0 + cc) * kD + d;
        if (p.out_bf16)
          reinterpret_cast<__bf16 *>(p.out)[oi] = (__bf16)v;
        else
          reinterpret_cast<float *>(p.out)[oi] = v;
      } else {
        const int64_t base = ((int64_t)gi * 2 + slot) * g + cc;
        coherent_store(p.sk_part + base * kD + d, o);
        if (d == 0) {
          coherent_store(p.sk_ml + base * 2 + 0, M);
          coherent_store(p.sk_ml + base * 2 + 1, lsum);
        }
      }
    }

    if (!whole) {
      // publish this partial (stores drained), then take a ticket; the last
      // arrival merges
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int g_first = range_of(S.row_start, T, G, R);
      const int g_last = range_of(S.row_start + S.nb - 1, T, G, R);
      if (tid == 0) {
        const unsigned long long gen = (unsigned long long)p.sk_gen << 32;
        unsigned long long *tk = p.sk_tickets + row;
        unsigned long long old = __hip_atomic_load(tk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned long long arrived;
        while (true) {
          arrived = ((old >> 32) == (unsigned long long)p.sk_gen) ? (old & 0xffffffffull) : 0ull;
          const unsigned long long want = gen | (arrived + 1);
          const unsigned long long seen = atomicCAS(tk, old, want);
          if (seen == old) break;
          old = seen;
        }
        s_last = (int)(arrived + 1) == (g_last - g_first + 1);
      }
      __syncthreads();
      if (s_last) {
        // All loads of the merge are issued together: (max, sum) of every
        // (contributor, column) is staged in LDS by one coherent load per
        // thread, the weights are formed once per (contributor, column), and
        // each output element fetches its contributors' partials in batches of
        // eight independent loads.  sm_o is free to reuse here.
        const int nc = g_last - g_first + 1;
        float *s_cm = &sm_o[0][0][0];
        float *s_cl = s_cm + nc * g;
        float *s_cw = s_cl + nc * g;
        if (3 * nc * g <= NW * 16 * kD) {
          for (int idx = tid; idx < nc * g; idx += 64 * NW) {
            const int k = idx / g, cc = idx - k * g;
            const int gg = g_first + k;
            const int sl = S.row_start <= range_begin(gg, T, G, R) ? 0 : 1;
            const int64_t base = ((int64_t)gg * 2 + sl) * g + cc;
            s_cm[idx] = coherent_load(p.sk_ml + base * 2 + 0);
            s_cl[idx] = coherent_load(p.sk_ml + base * 2 + 1);
          }
          __syncthreads();
          for (int cc = tid; cc < g; cc += 64 * NW) {
            float M = kNegInf;
            for (int k = 0; k < nc; ++k) M = fmaxf(M, s_cm[k * g + cc]);
            const float M_use = M == kNegInf ? 0.f : M;
            float lsum = 0.f;
            for (int k = 0; k < nc; ++k) {
              const float wgt = fast_exp2(s_cm[k * g + cc] - M_use);
              s_cw[k * g + cc] = wgt;
              lsum += s_cl[k * g + cc] * wgt;
            }
            s_cm[cc] = lsum;  // row sum per column (slot 0 of s_cm is no longer needed)
          }
          __syncthreads();
          for (int idx = tid; idx < g * kD; idx += 64 * NW) {
            const int cc = idx / kD, d = idx - cc * kD;
            float o = 0.f;
            for (int k0 = 0; k0 < nc; k0 += 8) {
              float v[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const int k = min(k0 + u, nc - 1);
                const int gg = g_first + k;
                const int sl = S.row_start <= range_begin(gg, T, G, R) ? 0 : 1;
                v[u] = coherent_load(p.sk_part + (((int64_t)gg * 2 + sl) * g + cc) * kD + d);
              }
#pragma unroll
              for (int u = 0; u < 8; ++u)
                if (k0 + u < nc) o += v[u] * s_cw[(k0 + u) * g + cc];
            }
            const float lsum = s_cm[cc];
            const float val = lsum > 0.f ? o / lsum : 0.f;
            const int64_t oi = (out_row0 + cc) * kD + d;
            if (p.out_bf16)
              reinterpret_cast<__bf16 *>(p.out)[oi] = (__bf16)val;
            else
              reinterpret_cast<float *>(p.out)[oi] = val;
          }
        } else {
          // more contributors than the staging space: plain loop
          for (int idx = tid; idx < g * kD; idx += 64 * NW) {
            const int cc = idx / kD, d = idx - cc * kD;
            float M = kNegInf;
            for (int gg = g_first; gg <= g_last; ++gg) {
              const int sl = S.row_start <= range_begin(gg, T, G, R) ? 0 : 1;
              M = fmaxf(M, coherent_load(p.sk_ml + (((int64_t)gg * 2 + sl) * g + cc) * 2 + 0));
            }
            const float M_use = M == kNegInf ? 0.f : M;
            float lsum = 0.f, o = 0.f;
            for (int gg = g_first; gg <= g_last; ++gg) {
              const int sl = S.row_start <= range_begin(gg, T, G, R) ? 0 : 1;
              const int64_t base = ((int64_t)gg * 2 + sl) * g + cc;
              const float wgt = fast_exp2(coherent_load(p.sk_ml + base * 2 + 0) - M_use);
              lsum += coherent_load(p.sk_ml + base * 2 + 1) * wgt;
              o += coherent_load(p.sk_part + base * kD + d) * wgt;
            }
            const float val = lsum > 0.f ? o / lsum : 0.f;
            const int64_t oi = (out_row0 + cc) * kD + d;
            if (p.out_bf16)
              reinterpret_cast<__bf16 *>(p.out)[oi] = (__bf16)val;
            else
              reinterpret_cast<float *>(p.out)[oi] = val;
          }
        }
      }
    }
    __syncthreads();  // sm_* and s_last are reused by the next segment
    if (!has_next) break;
    S = Sn;
#pragma unroll
    for (int i = 0; i < 4; ++i) qc[i] = qn[i];
    has_next = S.flat_end < e;
    if (has_next) {
      Sn = seg_at(S.flat_end);
      load_q(Sn, qn);
    }
  }
}

}  // namespace

hipError_t launch_decode_streamk(const DecodeParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_streamk_kernel<PA_DECODE_WAVES>, dim3(p.sk_ranges), dim3(64 * PA_DECODE_WAVES),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
