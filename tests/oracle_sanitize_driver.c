/*
 * oracle_sanitize_driver.c -- runs every entry point of oracle/oracle.c on
 * small seeded problems, edge cases and bad arguments, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (test_oracle_sanitize.py)
 * sees each of its memory accesses and arithmetic paths.  It also checks a
 * few results that hold by construction (paged == contiguous, blockwise ==
 * plain, swap round trip, codec round trip), so a path that runs clean but
 * computes garbage is noticed too.  Test infrastructure only.
 *
 * Exit status 0: every check passed and no sanitizer report (the build makes
 * a report fatal).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (oracle/oracle.c is compiled alongside) */
void oracle_fp8_decode(const uint8_t *codes, double *out, int64_t n);
void oracle_fp8_encode(const float *x, uint8_t *codes, int64_t n);
int oracle_kv_cache_write(const void *key, const void *value, void *k_cache, void *v_cache,
                          const int64_t *slot_mapping, int T, int num_blocks, int Hkv, int bs, int D, int dtype);
int oracle_kv_cache_write_fp8(const void *key, const void *value, int src_dtype, uint8_t *k_cache,
                              uint8_t *v_cache, const int64_t *slot_mapping, int T, int num_blocks, int Hkv,
                              int bs, int D, float k_scale, float v_scale);
int oracle_block_copy(void *k_cache, void *v_cache, const int64_t *pairs, int N, int num_blocks, int Hkv, int bs,
                      int D, int dtype);
int oracle_swap_out(const void *k_cache, const void *v_cache, const int64_t *ids, int n, void *host,
                    int num_blocks, int Hkv, int bs, int D, int dtype);
int oracle_swap_in(void *k_cache, void *v_cache, const int64_t *ids, int n, const void *host, int num_blocks,
                   int Hkv, int bs, int D, int dtype);
int oracle_paged_decode_ex(double *out, const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                           int dtype, double k_scale, double v_scale, const int32_t *block_tables, int max_blocks,
                           const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int bs, int num_blocks,
                           double scale);
int oracle_paged_decode(double *out, const void *q, const void *k_cache, const void *v_cache, int dtype,
                        const int32_t *block_tables, int max_blocks, const int32_t *seq_lens, int B, int Hq,
                        int Hkv, int D, int bs, int num_blocks, double scale);
int oracle_paged_prefill_ex(double *out, const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                            int dtype, double k_scale, double v_scale, const int32_t *block_tables, int max_blocks,
                            const int32_t *query_start_loc, const int32_t *seq_lens, int B, int Hq, int Hkv, int D,
                            int bs, int num_blocks, double scale);
int oracle_contiguous_attention(double *out, const double *q, const double *K, const double *V,
                                const int32_t *n_keys, int Tq, int Lk, int Hq, int Hkv, int D, double scale);
int oracle_blockwise_decode_row(double *out, const void *q, int64_t q_off, const void *k_cache, const void *v_cache,
                                int dtype, const int32_t *table, int n_keys, int kh, int Hkv, int D, int bs,
                                int num_blocks, double scale, int partition_blocks, const int32_t *visit_order);

static int failures = 0;
#define CHECK(cond, ...)                       \
  do {                                         \
    if (!(cond)) {                             \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);            \
      fprintf(stderr, "\n");                   \
      ++failures;                              \
    }                                          \
  } while (0)

/* splitmix64 and a Box-Muller normal */
static uint64_t rng_state = 12345;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double uniform01(void) { return ((next_u64() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
static float normal(void) { return (float)(sqrt(-2.0 * log(uniform01())) * cos(6.283185307179586 * uniform01())); }

static uint16_t to_bf16(float f) {  /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}
static double bf16_val(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static double max_abs_diff(const double *a, const double *b, size_t n) {
  double m = 0;
  for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
  return m;
}

enum { Hkv = 2, Hq = 6, D = 16 };

/* a paged problem: block size bs, lengths lens[B], a shuffled pool */
typedef struct {
  int B, bs, nb, maxblk;
  int32_t *table, *lens;
} layout;

static layout make_layout(const int *lens, int B, int bs) {
  layout L = {B, bs, 0, 1, NULL, NULL};
  int need = 0;
  for (int b = 0; b < B; ++b) {
    int n = (lens[b] + bs - 1) / bs;
    need += n;
    if (n > L.maxblk) L.maxblk = n;
  }
  L.nb = need + 3;
  int *perm = malloc(sizeof(int) * L.nb);
  for (int i = 0; i < L.nb; ++i) perm[i] = i;
  for (int i = L.nb - 1; i > 0; --i) {
    int j = (int)(next_u64() % (uint64_t)(i + 1)), t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  L.table = malloc(sizeof(int32_t) * B * L.maxblk);
  L.lens = malloc(sizeof(int32_t) * B);
  int used = 0;
  for (int b = 0; b < B; ++b) {
    L.lens[b] = lens[b];
    for (int j = 0; j < L.maxblk; ++j)
      L.table[b * L.maxblk + j] = j < (lens[b] + bs - 1) / bs ? perm[used++] : -1;
  }
  free(perm);
  return L;
}

static void check_decode_and_prefill(int bs) {
  const int lens[] = {1, 17, 0, 40, bs, 2 * bs + 3};
  const int B = 6;
  layout L = make_layout(lens, B, bs);
  size_t ce = (size_t)L.nb * Hkv * bs * D;
  uint16_t *k = malloc(2 * ce), *v = malloc(2 * ce), *q = malloc(2 * B * Hq * D);
  for (size_t i = 0; i < ce; ++i) {
    k[i] = to_bf16(normal());
    v[i] = to_bf16(normal());
  }
  for (int i = 0; i < B * Hq * D; ++i) q[i] = to_bf16(normal());
  double *out = malloc(sizeof(double) * B * Hq * D);
  int rc = oracle_paged_decode(out, q, k, v, 1, L.table, L.maxblk, L.lens, B, Hq, Hkv, D, bs, L.nb, 0.3);
  CHECK(rc == 0, "decode rc %d", rc);
  for (int d = 0; d < Hq * D; ++d) CHECK(out[2 * Hq * D + d] == 0.0, "empty row not zero");
  /* paged == contiguous, and == the blockwise form with partitions of 2 blocks */
  for (int b = 0; b < B; ++b) {
    int n = lens[b];
    if (n == 0) continue;
    double *K = malloc(sizeof(double) * n * Hkv * D), *V = malloc(sizeof(double) * n * Hkv * D);
    double *qd = malloc(sizeof(double) * Hq * D), *co = malloc(sizeof(double) * Hq * D);
    for (int t = 0; t < n; ++t)
      for (int h = 0; h < Hkv; ++h)
        for (int d = 0; d < D; ++d) {
          size_t at = (((size_t)L.table[b * L.maxblk + t / bs] * Hkv + h) * bs + t % bs) * D + d;
          K[((size_t)t * Hkv + h) * D + d] = bf16_val(k[at]);
          V[((size_t)t * Hkv + h) * D + d] = bf16_val(v[at]);
        }
    for (int i = 0; i < Hq * D; ++i) qd[i] = bf16_val(q[b * Hq * D + i]);
    int32_t nk = n;
    rc = oracle_contiguous_attention(co, qd, K, V, &nk, 1, n, Hq, Hkv, D, 0.3);
    CHECK(rc == 0, "contiguous rc %d", rc);
    CHECK(max_abs_diff(co, out + (size_t)b * Hq * D, Hq * D) < 1e-12, "paged != contiguous (b=%d bs=%d)", b, bs);
    double row[D];
    for (int h = 0; h < Hq; ++h) {
      rc = oracle_blockwise_decode_row(row, q, (int64_t)(b * Hq + h) * D, k, v, 1, L.table + b * L.maxblk, n,
                                       h / (Hq / Hkv), Hkv, D, bs, L.nb, 0.3, 2, NULL);
      CHECK(rc == 0, "blockwise rc %d", rc);
      CHECK(max_abs_diff(row, out + ((size_t)b * Hq + h) * D, D) < 1e-12, "blockwise != plain");
    }
    free(K);
    free(V);
    free(qd);
    free(co);
  }
  /* a prefill chunk of 3 rows for each non-empty sequence (1 row for length 1) */
  int32_t qsl[7] = {0};
  for (int b = 0; b < B; ++b) qsl[b + 1] = qsl[b] + (lens[b] >= 3 ? 3 : lens[b]);
  uint16_t *qp = malloc(2 * (size_t)qsl[B] * Hq * D + 2);
  for (int i = 0; i < qsl[B] * Hq * D; ++i) qp[i] = to_bf16(normal());
  double *outp = malloc(sizeof(double) * (qsl[B] * Hq * D + 1));
  rc = oracle_paged_prefill_ex(outp, qp, 1, k, v, 1, 1.0, 1.0, L.table, L.maxblk, qsl, L.lens, B, Hq, Hkv, D, bs,
                               L.nb, 0.3);
  CHECK(rc == 0, "prefill rc %d", rc);
  /* a bad table entry is an error, not an access */
  int32_t saved = L.table[3 * L.maxblk + 1];
  L.table[3 * L.maxblk + 1] = L.nb + 7;
  rc = oracle_paged_decode(out, q, k, v, 1, L.table, L.maxblk, L.lens, B, Hq, Hkv, D, bs, L.nb, 0.3);
  CHECK(rc != 0, "bad table entry accepted");
  L.table[3 * L.maxblk + 1] = saved;
  /* NULL arguments */
  CHECK(oracle_paged_decode(NULL, q, k, v, 1, L.table, L.maxblk, L.lens, B, Hq, Hkv, D, bs, L.nb, 0.3) != 0,
        "NULL out accepted");
  free(k);
  free(v);
  free(q);
  free(out);
  free(qp);
  free(outp);
  free(L.table);
  free(L.lens);
}

static void check_memory_ops(void) {
  const int nb = 9, bs = 4, T = 5;
  size_t ce = (size_t)nb * Hkv * bs * D;
  float *k = malloc(4 * ce), *v = malloc(4 * ce), *k0 = malloc(4 * ce);
  for (size_t i = 0; i < ce; ++i) {
    k[i] = normal();
    v[i] = normal();
  }
  memcpy(k0, k, 4 * ce);
  float *key = malloc(4 * T * Hkv * D), *val = malloc(4 * T * Hkv * D);
  for (int i = 0; i < T * Hkv * D; ++i) {
    key[i] = normal();
    val[i] = normal();
  }
  int64_t slots[5] = {3, -1, nb * bs - 1, 12, 0};
  CHECK(oracle_kv_cache_write(key, val, k, v, slots, T, nb, Hkv, bs, D, 0) == 0, "write");
  /* token 4 went to slot 0: block 0, offset 0 of each KV head */
  for (int h = 0; h < Hkv; ++h)
    CHECK(memcmp(k + (size_t)h * bs * D, key + ((size_t)4 * Hkv + h) * D, 4 * D) == 0, "write layout (head %d)", h);
  int64_t pairs[6] = {1, 5, 2, 2, 7, 8};
  CHECK(oracle_block_copy(k, v, pairs, 3, nb, Hkv, bs, D, 0) == 0, "copy");
  size_t blk = (size_t)Hkv * bs * D;
  CHECK(memcmp(k + 5 * blk, k + 1 * blk, 4 * blk) == 0, "copy result");
  int64_t ids[3] = {4, 0, 8};
  uint8_t *host = malloc(3 * 2 * 4 * blk);
  CHECK(oracle_swap_out(k, v, ids, 3, host, nb, Hkv, bs, D, 0) == 0, "swap out");
  int64_t to[3] = {6, 3, 1};
  CHECK(oracle_swap_in(k, v, to, 3, host, nb, Hkv, bs, D, 0) == 0, "swap in");
  CHECK(memcmp(host, k + 6 * blk, 4 * blk) == 0, "swap round trip");
  /* FP8: the quantising write, then the codec over every code */
  uint8_t *kc = calloc(ce, 1), *vc = calloc(ce, 1);
  CHECK(oracle_kv_cache_write_fp8(key, val, 0, kc, vc, slots, T, nb, Hkv, bs, D, 0.01f, 0.02f) == 0, "fp8 write");
  uint8_t codes[256], back[256];
  double vals[256];
  float fv[256];
  for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
  oracle_fp8_decode(codes, vals, 256);
  for (int i = 0; i < 256; ++i) fv[i] = (float)vals[i];
  oracle_fp8_encode(fv, back, 256);
  for (int i = 0; i < 256; ++i)
    if ((i & 0x7F) != 0x7F) CHECK(back[i] == codes[i], "fp8 round trip code %d -> %d", i, back[i]);
  /* FP8 attention over the written codes */
  int32_t table[2] = {3, 0}, lens[1] = {6};
  uint16_t q[Hq * D];
  for (int i = 0; i < Hq * D; ++i) q[i] = to_bf16(normal());
  double out[Hq * D];
  CHECK(oracle_paged_decode_ex(out, q, 1, kc, vc, 2, 0.01, 0.02, table, 2, lens, 1, Hq, Hkv, D, bs, nb, 0.25) == 0,
        "fp8 decode");
  free(k);
  free(v);
  free(k0);
  free(key);
  free(val);
  free(host);
  free(kc);
  free(vc);
}

int main(void) {
  for (int bs = 1; bs <= 16; bs *= 4) check_decode_and_prefill(bs);
  check_memory_ops();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitize driver: all checks passed\n");
  return 0;
}
