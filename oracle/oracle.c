/*
 * oracle.c -- plain CPU reference for paged KV-cache attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the GPU
 * library and includes nothing from it.
 *
 * Every floating-point result is computed in fp64 from the exactly decoded
 * input values (a bf16 value widens to double without rounding).  Nothing is
 * blocked, fused or reordered beyond the plain definition.
 *
 * Sources (web pages on KV-cache management):
 *  - Month 2 "PagedAttention" (infra learning path, memory chapter):
 *      §2.1  attention with a KV cache, softmax(Q_i K_{:i}^T / sqrt(d)) V_{:i};
 *      §5.2  one physical KV pool per layer, separate K and V tensors;
 *      §5.4  the kernel visits logical blocks through the block table.
 *  - Lecture 7 "KV Cache Management: PagedAttention and Mooncake" (CS349E):
 *      §4.1  fixed-size blocks, block table, only the last block is partial;
 *      §4.2  blockwise attention equals attention over the contiguous KV;
 *      §4.3  the fused kernels: KV write, attention through the table,
 *            batched copy of the blocks copy-on-write needs.
 *  - Lecture 16 "LLM Serving (1): Batching, PagedAttention, RadixAttention"
 *    (CMU 15-779): §3.3 block table and blockwise attention with the
 *    online-softmax merge rule.
 *  - Lecture 27 "Better KV Caches: CacheGen, CacheBlend and LMCache"
 *    (CMU 11-868): §1.1 new tokens' queries attend to cached K,V directly
 *    (the chunked-prefill case).
 *
 * Readings taken where the pages are silent or garbled (each is listed in the
 * design notes with its reason):
 *  - a sequence of length L uses ceil(L/bs) blocks; offsets >= L in the last
 *    block are never read (the pages' loop bound floors the division, which
 *    would drop the partial last block that §4.1 says exists);
 *  - query head h reads KV head h / (Hq/Hkv) (contiguous GQA groups);
 *  - the kernel attends to exactly seq_lens[b] tokens, the current one
 *    included (its K,V are written before attention);
 *  - L == 0 gives an all-zero output row;
 *  - cache layout [num_blocks][Hkv][block_size][D], K and V separate;
 *  - slot = block * block_size + offset, slot < 0 means "skip this row".
 *
 * dtype codes: 0 = fp32, 1 = bf16 (stored as raw 16-bit patterns), 2 = fp8
 * E4M3 (raw 8-bit codes; the KV cache only).
 *
 * FP8 KV cache (Lecture 7 §10: KV quantised to FP8 / INT8 / INT4 shrinks
 * memory and bandwidth by the bit count; the pages fix no format or scale,
 * so the reading taken is): E4M3 as in the OCP 8-bit floating-point
 * definition -- sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals at exponent 0, no infinities, S.1111.111 is NaN, largest finite
 * magnitude 448 -- and one fp32 scale per tensor for K and one for V.  A row
 * is stored as code(x / scale), the quotient in fp32, rounded to the nearest
 * code (ties to the even code), magnitudes above 448 saturated to 448, NaN
 * to the NaN code; it is read back as value(code) * scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_RANGE (-2)
#define ORC_ERR_NOMEM (-3)

/* The value of an E4M3 code, by the definition above. */
static double fp8_value(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* The code of an fp32 value: nearest of the 127 finite magnitudes (a plain
 * search), ties to the even code, saturating at 448; the sign is kept (a
 * negative value that rounds to zero gives negative zero). */
static uint8_t fp8_code(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0;
  if (isnan(x)) return sign | 0x7F;
  double a = fabs((double)x);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 127; ++c) {
    double dd = fabs(a - fp8_value((uint8_t)c));
    if (dd < best_d || (dd == best_d && (c & 1) == 0)) {
      best_d = dd;
      best = c;
    }
  }
  return sign | (uint8_t)best;
}

static double elem(const void *base, int64_t i, int dtype) {
  if (dtype == 0) return (double)((const float *)base)[i];
  if (dtype == 2) return fp8_value(((const uint8_t *)base)[i]);
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int elem_bytes(int dtype) { return dtype == 0 ? 4 : dtype == 1 ? 2 : 1; }

/* Exposed for the pins: decode n codes / encode n fp32 values. */
void oracle_fp8_decode(const uint8_t *codes, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = fp8_value(codes[i]);
}
void oracle_fp8_encode(const float *x, uint8_t *codes, int64_t n) {
  for (int64_t i = 0; i < n; ++i) codes[i] = fp8_code(x[i]);
}

/* Index of element (blk, h, off, d) in a [NB][Hkv][bs][D] cache. */
static int64_t cache_index(int64_t blk, int h, int off, int d, int Hkv, int bs,
                           int D) {
  return (((blk * Hkv + h) * (int64_t)bs + off) * D) + d;
}

/*
 * KV write (Lecture 7 §4.3, first fused kernel; Lecture 16 §3.3 fill rule):
 * for every token t with slot s = slot_mapping[t] >= 0, copy key[t][h][:] to
 * K[s / bs][h][s % bs][:] and value[t][h][:] likewise, for every KV head h.
 * A pure byte copy.  Returns ORC_ERR_RANGE (after writing nothing for that
 * row) if a slot points past the pool.
 */
int oracle_kv_cache_write(const void *key, const void *value, void *k_cache,
                          void *v_cache, const int64_t *slot_mapping, int T,
                          int num_blocks, int Hkv, int bs, int D, int dtype) {
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return ORC_ERR_ARG;
  int eb = elem_bytes(dtype);
  int rc = ORC_OK;
  for (int t = 0; t < T; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t blk = s / bs;
    int off = (int)(s % bs);
    if (blk >= num_blocks) {
      rc = ORC_ERR_RANGE;
      continue;
    }
    for (int h = 0; h < Hkv; ++h) {
      int64_t src = ((int64_t)t * Hkv + h) * D;
      int64_t dst = cache_index(blk, h, off, 0, Hkv, bs, D);
      memcpy((char *)k_cache + dst * eb, (const char *)key + src * eb, (size_t)D * eb);
      memcpy((char *)v_cache + dst * eb, (const char *)value + src * eb, (size_t)D * eb);
    }
  }
  return rc;
}

/*
 * KV write into an FP8 cache (the write above, with the quantisation of the
 * header): key and value rows are fp32 (src_dtype 0) or bf16 (1); every
 * element x of a key row is stored as fp8_code((float)x / k_scale), of a
 * value row as fp8_code((float)x / v_scale), the quotient an fp32 division.
 */
int oracle_kv_cache_write_fp8(const void *key, const void *value, int src_dtype, uint8_t *k_cache,
                              uint8_t *v_cache, const int64_t *slot_mapping, int T, int num_blocks,
                              int Hkv, int bs, int D, float k_scale, float v_scale) {
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return ORC_ERR_ARG;
  if (src_dtype != 0 && src_dtype != 1) return ORC_ERR_ARG;
  int rc = ORC_OK;
  for (int t = 0; t < T; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t blk = s / bs;
    int off = (int)(s % bs);
    if (blk >= num_blocks) {
      rc = ORC_ERR_RANGE;
      continue;
    }
    for (int h = 0; h < Hkv; ++h) {
      int64_t src = ((int64_t)t * Hkv + h) * D;
      int64_t dst = cache_index(blk, h, off, 0, Hkv, bs, D);
      for (int d = 0; d < D; ++d) {
        float kx = (float)elem(key, src + d, src_dtype), vx = (float)elem(value, src + d, src_dtype);
        k_cache[dst + d] = fp8_code(kx / k_scale);
        v_cache[dst + d] = fp8_code(vx / v_scale);
      }
    }
  }
  return rc;
}

/*
 * Block copy for copy-on-write (Lecture 7 §4.3 third fused kernel and §5.1;
 * Lecture 16 §3.5): for each pair (src, dst), K[dst] = K[src] and
 * V[dst] = V[src] over all KV heads of one layer.  Pairs are applied in
 * order; src == dst is a no-op.
 */
int oracle_block_copy(void *k_cache, void *v_cache, const int64_t *pairs, int N,
                      int num_blocks, int Hkv, int bs, int D, int dtype) {
  if (!k_cache || !v_cache || (!pairs && N > 0)) return ORC_ERR_ARG;
  size_t blk_bytes = (size_t)Hkv * bs * D * elem_bytes(dtype);
  for (int i = 0; i < N; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return ORC_ERR_RANGE;
    if (src == dst) continue;
    memmove((char *)k_cache + dst * blk_bytes, (const char *)k_cache + src * blk_bytes, blk_bytes);
    memmove((char *)v_cache + dst * blk_bytes, (const char *)v_cache + src * blk_bytes, blk_bytes);
  }
  return ORC_OK;
}

/*
 * Swapping (Lecture 7 §6.2: a preempted sequence group's blocks are copied to
 * CPU memory and later copied back, into whatever physical blocks are free;
 * Month 2 §8.1: the blocks of a sequence move together).  The host image is
 * a sequence of pieces, piece i = K block ids[i] followed by V block ids[i]
 * (blk_bytes each).  Out: an id outside [0, num_blocks) gives a zero piece.
 * In: such an id is skipped.  Byte copies, in order.
 */
int oracle_swap_out(const void *k_cache, const void *v_cache, const int64_t *ids, int n, void *host,
                    int num_blocks, int Hkv, int bs, int D, int dtype) {
  if (!k_cache || !v_cache || ((!ids || !host) && n > 0)) return ORC_ERR_ARG;
  size_t blk_bytes = (size_t)Hkv * bs * D * elem_bytes(dtype);
  for (int i = 0; i < n; ++i) {
    char *piece = (char *)host + (size_t)i * 2 * blk_bytes;
    if (ids[i] < 0 || ids[i] >= num_blocks) {
      memset(piece, 0, 2 * blk_bytes);
      continue;
    }
    memcpy(piece, (const char *)k_cache + ids[i] * blk_bytes, blk_bytes);
    memcpy(piece + blk_bytes, (const char *)v_cache + ids[i] * blk_bytes, blk_bytes);
  }
  return ORC_OK;
}

int oracle_swap_in(void *k_cache, void *v_cache, const int64_t *ids, int n, const void *host,
                   int num_blocks, int Hkv, int bs, int D, int dtype) {
  if (!k_cache || !v_cache || ((!ids || !host) && n > 0)) return ORC_ERR_ARG;
  size_t blk_bytes = (size_t)Hkv * bs * D * elem_bytes(dtype);
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= num_blocks) continue;
    const char *piece = (const char *)host + (size_t)i * 2 * blk_bytes;
    memcpy((char *)k_cache + ids[i] * blk_bytes, piece, blk_bytes);
    memcpy((char *)v_cache + ids[i] * blk_bytes, piece + blk_bytes, blk_bytes);
  }
  return ORC_OK;
}

/*
 * One attention row by the definition (Month 2 §2.1): the query q (length D)
 * against the first n_keys tokens of sequence b, reached through the block
 * table (Month 2 §5.4: logical block j lives in physical block
 * block_table[j]; token t sits at offset t % bs of logical block t / bs).
 *   s_t = scale * sum_d q[d] K_t[d]
 *   out = sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s)
 * Two passes over the scores, fp64 throughout.  n_keys == 0 gives zeros.
 */
static int attend_row(double *out, const void *q, int64_t q_off, int q_dtype, const void *k_cache,
                      const void *v_cache, int dtype, double k_scale, double v_scale,
                      const int32_t *table, int max_blocks, int n_keys, int kh, int Hkv, int D,
                      int bs, int num_blocks, double scale, double *scores) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n_keys <= 0) return ORC_OK;
  if ((n_keys + bs - 1) / bs > max_blocks) return ORC_ERR_RANGE;
  double m = -INFINITY;
  for (int t = 0; t < n_keys; ++t) {
    int32_t phys = table[t / bs];
    if (phys < 0 || phys >= num_blocks) return ORC_ERR_RANGE;
    int64_t base = cache_index(phys, kh, t % bs, 0, Hkv, bs, D);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += elem(q, q_off + d, q_dtype) * (elem(k_cache, base + d, dtype) * k_scale);
    scores[t] = scale * dot;
    if (scores[t] > m) m = scores[t];
  }
  double l = 0.0;
  for (int t = 0; t < n_keys; ++t) {
    double e = exp(scores[t] - m);
    l += e;
    int64_t base = cache_index(table[t / bs], kh, t % bs, 0, Hkv, bs, D);
    for (int d = 0; d < D; ++d) out[d] += e * (elem(v_cache, base + d, dtype) * v_scale);
  }
  for (int d = 0; d < D; ++d) out[d] /= l;
  return ORC_OK;
}

/*
 * Paged decode (Month 2 §5.4; Lecture 7 §4.2): for every sequence b and query
 * head h, one query row q[b][h][:] attends to all seq_lens[b] cached tokens
 * of KV head h / (Hq / Hkv).  out is fp64 [B][Hq][D]; q has the KV dtype and
 * layout [B][Hq][D]; block_tables is [B][max_blocks].
 */
int oracle_paged_decode_ex(double *out, const void *q, int q_dtype, const void *k_cache,
                           const void *v_cache, int dtype, double k_scale, double v_scale,
                           const int32_t *block_tables, int max_blocks, const int32_t *seq_lens,
                           int B, int Hq, int Hkv, int D, int bs, int num_blocks, double scale) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens) return ORC_ERR_ARG;
  if (Hkv <= 0 || Hq % Hkv != 0 || bs <= 0 || D <= 0) return ORC_ERR_ARG;
  int g = Hq / Hkv;
  int max_len = 0;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] > max_len) max_len = seq_lens[b];
  double *scores = (double *)malloc(sizeof(double) * (max_len > 0 ? max_len : 1));
  if (!scores) return ORC_ERR_NOMEM;
  int rc = ORC_OK;
  for (int b = 0; b < B && rc == ORC_OK; ++b) {
    for (int h = 0; h < Hq && rc == ORC_OK; ++h) {
      int64_t row = (int64_t)b * Hq + h;
      rc = attend_row(out + row * D, q, row * D, q_dtype, k_cache, v_cache, dtype, k_scale, v_scale,
                      block_tables + (int64_t)b * max_blocks, max_blocks, seq_lens[b],
                      h / g, Hkv, D, bs, num_blocks, scale, scores);
    }
  }
  free(scores);
  return rc;
}

/* q and the caches in one dtype (fp32 or bf16), no scales. */
int oracle_paged_decode(double *out, const void *q, const void *k_cache,
                        const void *v_cache, int dtype, const int32_t *block_tables,
                        int max_blocks, const int32_t *seq_lens, int B, int Hq,
                        int Hkv, int D, int bs, int num_blocks, double scale) {
  return oracle_paged_decode_ex(out, q, dtype, k_cache, v_cache, dtype, 1.0, 1.0, block_tables,
                                max_blocks, seq_lens, B, Hq, Hkv, D, bs, num_blocks, scale);
}

/*
 * Chunked prefill over cached blocks (Lecture 27 §1.1; Lecture 7 §8.3: only
 * the uncached suffix is computed, its queries attend to the cached prefix
 * and to themselves).  Sequence b owns query rows query_start_loc[b] ..
 * query_start_loc[b+1]-1 (n_b rows) and has seq_lens[b] tokens in the cache
 * after the chunk was written.  Row i of the chunk sits at position
 * pos = seq_lens[b] - n_b + i and attends to tokens 0..pos (causal).
 * q and out are [Tq][Hq][D].
 */
int oracle_paged_prefill_ex(double *out, const void *q, int q_dtype, const void *k_cache,
                            const void *v_cache, int dtype, double k_scale, double v_scale,
                            const int32_t *block_tables, int max_blocks,
                            const int32_t *query_start_loc, const int32_t *seq_lens, int B,
                            int Hq, int Hkv, int D, int bs, int num_blocks, double scale) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !seq_lens)
    return ORC_ERR_ARG;
  if (Hkv <= 0 || Hq % Hkv != 0 || bs <= 0 || D <= 0) return ORC_ERR_ARG;
  int g = Hq / Hkv;
  int max_len = 0;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] > max_len) max_len = seq_lens[b];
  double *scores = (double *)malloc(sizeof(double) * (max_len > 0 ? max_len : 1));
  if (!scores) return ORC_ERR_NOMEM;
  int rc = ORC_OK;
  for (int b = 0; b < B && rc == ORC_OK; ++b) {
    int q0 = query_start_loc[b], n_b = query_start_loc[b + 1] - q0;
    if (n_b < 0 || n_b > seq_lens[b]) {
      rc = ORC_ERR_ARG;
      break;
    }
    for (int i = 0; i < n_b && rc == ORC_OK; ++i) {
      int pos = seq_lens[b] - n_b + i;
      for (int h = 0; h < Hq && rc == ORC_OK; ++h) {
        int64_t row = (int64_t)(q0 + i) * Hq + h;
        rc = attend_row(out + row * D, q, row * D, q_dtype, k_cache, v_cache, dtype, k_scale,
                        v_scale, block_tables + (int64_t)b * max_blocks, max_blocks, pos + 1,
                        h / g, Hkv, D, bs, num_blocks, scale, scores);
      }
    }
  }
  free(scores);
  return rc;
}

int oracle_paged_prefill(double *out, const void *q, const void *k_cache,
                         const void *v_cache, int dtype, const int32_t *block_tables,
                         int max_blocks, const int32_t *query_start_loc,
                         const int32_t *seq_lens, int B, int Hq, int Hkv, int D,
                         int bs, int num_blocks, double scale) {
  return oracle_paged_prefill_ex(out, q, dtype, k_cache, v_cache, dtype, 1.0, 1.0, block_tables,
                                 max_blocks, query_start_loc, seq_lens, B, Hq, Hkv, D, bs,
                                 num_blocks, scale);
}

/*
 * Contiguous attention, no block table: the layout earlier systems used
 * (Lecture 7 §3.1) and the right-hand side of the equivalence in Lecture 7
 * §4.2 / Lecture 16 §3.3.  q is fp64 [Tq][Hq][D]; K and V are fp64
 * [Lk][Hkv][D] for one sequence.  Query row i attends to keys
 * 0..n_keys[i]-1.  out is fp64 [Tq][Hq][D].
 */
int oracle_contiguous_attention(double *out, const double *q, const double *K,
                                const double *V, const int32_t *n_keys, int Tq,
                                int Lk, int Hq, int Hkv, int D, double scale) {
  if (!out || !q || !K || !V || !n_keys) return ORC_ERR_ARG;
  if (Hkv <= 0 || Hq % Hkv != 0) return ORC_ERR_ARG;
  int g = Hq / Hkv;
  double *s = (double *)malloc(sizeof(double) * (Lk > 0 ? Lk : 1));
  if (!s) return ORC_ERR_NOMEM;
  for (int i = 0; i < Tq; ++i) {
    int n = n_keys[i];
    if (n > Lk) {
      free(s);
      return ORC_ERR_RANGE;
    }
    for (int h = 0; h < Hq; ++h) {
      int kh = h / g;
      const double *qr = q + ((int64_t)i * Hq + h) * D;
      double *o = out + ((int64_t)i * Hq + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (n <= 0) continue;
      double m = -INFINITY;
      for (int t = 0; t < n; ++t) {
        const double *k = K + ((int64_t)t * Hkv + kh) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qr[d] * k[d];
        s[t] = scale * dot;
        if (s[t] > m) m = s[t];
      }
      double l = 0.0;
      for (int t = 0; t < n; ++t) {
        double e = exp(s[t] - m);
        l += e;
        const double *v = V + ((int64_t)t * Hkv + kh) * D;
        for (int d = 0; d < D; ++d) o[d] += e * v[d];
      }
      for (int d = 0; d < D; ++d) o[d] /= l;
    }
  }
  free(s);
  return ORC_OK;
}

/*
 * A softmax summary of a set of keys for one query row (Lecture 16 §3.3:
 * attention over blocks is combined by the online-softmax rule, which is
 * associative and commutative): top = the largest score in the set, mass =
 * sum of exp(score - top), vec[d] = sum of exp(score - top) * value[d].  An
 * empty set has top = -inf, mass = 0, vec = 0.  The attention output over the
 * set is vec / mass.
 */
typedef struct {
  double top, mass;
  double *vec; /* D entries, owned by the caller */
} summary;

static void summary_clear(summary *s, int D) {
  s->top = -INFINITY;
  s->mass = 0.0;
  for (int d = 0; d < D; ++d) s->vec[d] = 0.0;
}

/* dst := summary of (dst's keys together with src's keys).  Each side is
 * re-expressed relative to the larger top, exp(top_side - top_both), and
 * the two are added. */
static void summary_absorb(summary *dst, const summary *src, int D) {
  if (src->top == -INFINITY) return; /* nothing to add */
  if (dst->top == -INFINITY) {
    dst->top = src->top;
    dst->mass = src->mass;
    for (int d = 0; d < D; ++d) dst->vec[d] = src->vec[d];
    return;
  }
  double both = dst->top > src->top ? dst->top : src->top;
  double wd = exp(dst->top - both), ws = exp(src->top - both);
  dst->mass = dst->mass * wd + src->mass * ws;
  for (int d = 0; d < D; ++d) dst->vec[d] = dst->vec[d] * wd + src->vec[d] * ws;
  dst->top = both;
}

/* The summary of the `valid` keys of one physical block for query q. */
static void summary_of_block(summary *s, double *scores, const void *q, int64_t q_off,
                             const void *k_cache, const void *v_cache, int dtype, int32_t phys,
                             int valid, int kh, int Hkv, int D, int bs, double scale) {
  summary_clear(s, D);
  for (int o = 0; o < valid; ++o) {
    int64_t at = cache_index(phys, kh, o, 0, Hkv, bs, D);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += elem(q, q_off + d, dtype) * elem(k_cache, at + d, dtype);
    scores[o] = scale * dot;
    if (scores[o] > s->top) s->top = scores[o];
  }
  for (int o = 0; o < valid; ++o) {
    double w = exp(scores[o] - s->top);
    int64_t at = cache_index(phys, kh, o, 0, Hkv, bs, D);
    s->mass += w;
    for (int d = 0; d < D; ++d) s->vec[d] += w * elem(v_cache, at + d, dtype);
  }
}

/*
 * The blockwise form of one decode row, kept to pin the plain definition
 * above against the pages' claim that blockwise attention reaches the same
 * result (Lecture 7 §4.2; Month 2 §5.4 walks the logical blocks through the
 * block table; Lecture 16 §3.3 gives the merge rule).  The row's logical
 * blocks are grouped into partitions of `partition_blocks` consecutive
 * blocks.  Every block is reduced to its own summary, the summaries of a
 * partition are absorbed into the partition's summary in the order
 * `visit_order` lists them (NULL: ascending; any order reaches the same real
 * number), and the partitions' summaries are then absorbed in ascending
 * order.  Only the valid offsets of the last block are scored (the ceil
 * reading of the loop bound).
 */
int oracle_blockwise_decode_row(double *out, const void *q, int64_t q_off,
                                const void *k_cache, const void *v_cache, int dtype,
                                const int32_t *table, int n_keys, int kh, int Hkv,
                                int D, int bs, int num_blocks, double scale,
                                int partition_blocks, const int32_t *visit_order) {
  if (!out || !q || !k_cache || !v_cache || !table || partition_blocks <= 0 || D <= 0) return ORC_ERR_ARG;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n_keys <= 0) return ORC_OK;
  int n_blocks = (n_keys + bs - 1) / bs;
  double *mem = (double *)calloc((size_t)3 * D + (size_t)bs, sizeof(double));
  if (!mem) return ORC_ERR_NOMEM;
  summary whole = {0, 0, mem}, part = {0, 0, mem + D}, blk = {0, 0, mem + 2 * D};
  double *scores = mem + 3 * D;
  summary_clear(&whole, D);
  int rc = ORC_OK;
  for (int first = 0; first < n_blocks && rc == ORC_OK; first += partition_blocks) {
    int count = n_blocks - first < partition_blocks ? n_blocks - first : partition_blocks;
    summary_clear(&part, D);
    for (int k = 0; k < count; ++k) {
      int j = visit_order ? visit_order[first + k] : first + k;
      if (j < first || j >= first + count) { rc = ORC_ERR_ARG; break; }
      int32_t phys = table[j];
      if (phys < 0 || phys >= num_blocks) { rc = ORC_ERR_RANGE; break; }
      int valid = n_keys - j * bs < bs ? n_keys - j * bs : bs;
      summary_of_block(&blk, scores, q, q_off, k_cache, v_cache, dtype, phys, valid, kh, Hkv, D, bs, scale);
      summary_absorb(&part, &blk, D);
    }
    summary_absorb(&whole, &part, D);
  }
  if (rc == ORC_OK)
    for (int d = 0; d < D; ++d) out[d] = whole.vec[d] / whole.mass;
  free(mem);
  return rc;
}
