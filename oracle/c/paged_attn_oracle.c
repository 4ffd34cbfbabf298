/*
 * Float64 paged-attention oracle in plain C -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library. It shares no code with the GPU library.
 *
 * What it computes (the method of the PagedAttention / vLLM abstract on the
 * papers page "external vector cache", with the causal visibility rule and
 * the reference attention of the course page "Module 10. KV Caches and
 * Efficient Inference": notebook section 2's FLOP model, where query j of a
 * causal suffix sees cached_prefix + j + 1 keys, and the project demo's
 * Demo 2 attention with the row maximum subtracted):
 *
 *   for every sequence b, query index i < nq, query head h:
 *     n   = L_b - nq + i + 1                      keys visible to the query
 *     g   = h / (Hq / Hkv)                        its KV head
 *     for t in 0..n-1 (token by token, through the block table):
 *       blk = table[b][t / bs], off = t % bs
 *       s_t = sigma * sum_d q[b,i,h,d] * K[blk,g,off,d]
 *     m = max_t s_t, p_t = exp(s_t - m), l = sum_t p_t
 *     out[b,i,h,:] = sum_t p_t V[blk,g,off,:] / l,  lse = m + log(l)
 *
 * sigma is the float32 scale widened to double; every stored element is
 * widened exactly to double (bf16: the float32 with those upper 16 bits).
 * A pool of per-row integer codes (the course page's teaching quantizer,
 * project demo Demo 2: symmetric codes, one scale per row) holds int8 codes
 * [num_blocks, Hkv, bs, D] and float32 scales [num_blocks, Hkv, bs]; its
 * element is code * scale, in double (pkv_oracle_attention_q8).
 *
 * Return codes: 0 ok; 1 bad argument; 2 a visible token maps to a table
 * entry outside [0, num_blocks); 3 a row sees no key (n <= 0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_Q8 = 2 };

/* Element idx of a pool; `scales` (one per row of D elements) only for
 * ORACLE_Q8. */
static double load_elem(const void *base, int dtype, size_t idx, const float *scales,
                        int D) {
  if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
  if (dtype == ORACLE_Q8)
    return (double)((const int8_t *)base)[idx] * (double)scales[idx / (size_t)D];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int attention_walk(const void *q, int q_dtype, const void *k_pool,
                          const void *v_pool, int kv_dtype, const float *k_scales,
                          const float *v_scales, const int32_t *tables, int max_blocks,
                          const int32_t *lens, int B, int nq, int Hq, int Hkv, int D, int bs,
                          int num_blocks, float scale, const int64_t *rows, int64_t n_rows,
                          double *out, double *lse, int threads);

int pkv_oracle_attention(const void *q, int q_dtype, const void *k_pool,
                         const void *v_pool, int kv_dtype,
                         const int32_t *tables, int max_blocks,
                         const int32_t *lens, int B, int nq, int Hq, int Hkv,
                         int D, int bs, int num_blocks, float scale,
                         const int64_t *rows, int64_t n_rows, double *out,
                         double *lse, int threads) {
  if (kv_dtype != ORACLE_F32 && kv_dtype != ORACLE_BF16) return 1;
  return attention_walk(q, q_dtype, k_pool, v_pool, kv_dtype, NULL, NULL, tables,
                        max_blocks, lens, B, nq, Hq, Hkv, D, bs, num_blocks, scale, rows,
                        n_rows, out, lse, threads);
}

int pkv_oracle_attention_q8(const void *q, int q_dtype, const int8_t *k_codes,
                            const int8_t *v_codes, const float *k_scales,
                            const float *v_scales, const int32_t *tables, int max_blocks,
                            const int32_t *lens, int B, int nq, int Hq, int Hkv, int D,
                            int bs, int num_blocks, float scale, const int64_t *rows,
                            int64_t n_rows, double *out, double *lse, int threads) {
  if (!k_scales || !v_scales) return 1;
  return attention_walk(q, q_dtype, k_codes, v_codes, ORACLE_Q8, k_scales, v_scales, tables,
                        max_blocks, lens, B, nq, Hq, Hkv, D, bs, num_blocks, scale, rows,
                        n_rows, out, lse, threads);
}

static int attention_walk(const void *q, int q_dtype, const void *k_pool,
                          const void *v_pool, int kv_dtype, const float *k_scales,
                          const float *v_scales, const int32_t *tables, int max_blocks,
                          const int32_t *lens, int B, int nq, int Hq, int Hkv, int D, int bs,
                          int num_blocks, float scale, const int64_t *rows, int64_t n_rows,
                          double *out, double *lse, int threads) {
  if (!q || !k_pool || !v_pool || !tables || !lens || !out) return 1;
  if (B <= 0 || nq <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 ||
      num_blocks <= 0 || max_blocks <= 0 || Hq % Hkv != 0)
    return 1;
  if (q_dtype != ORACLE_F32 && q_dtype != ORACLE_BF16) return 1;
  const int group = Hq / Hkv;
  const double sigma = (double)scale;
  const int64_t total_rows = (int64_t)B * nq * Hq;
  const int64_t count = rows ? n_rows : total_rows;
  int status = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif

#pragma omp parallel
  {
    int64_t cap = 0;
    double *scores = NULL;
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < count; ++r) {
      const int64_t row = rows ? rows[r] : r; /* (b * nq + i) * Hq + h */
      if (row < 0 || row >= total_rows) {
#pragma omp atomic write
        status = 1;
        continue;
      }
      const int h = (int)(row % Hq);
      const int i = (int)((row / Hq) % nq);
      const int b = (int)(row / ((int64_t)Hq * nq));
      const int g = h / group;
      const int64_t n = (int64_t)lens[b] - nq + i + 1;
      if (n <= 0 || n > (int64_t)max_blocks * bs) {
#pragma omp atomic write
        status = 3;
        continue;
      }
      if (n > cap) {
        free(scores);
        cap = n;
        scores = (double *)malloc(sizeof(double) * (size_t)cap);
      }
      const size_t qbase = (size_t)row * D;
      /* pass 1: scores, walking the block table token by token */
      double m = -INFINITY;
      int bad = 0;
      for (int64_t t = 0; t < n; ++t) {
        const int32_t blk = tables[(size_t)b * max_blocks + t / bs];
        if (blk < 0 || blk >= num_blocks) {
          bad = 1;
          break;
        }
        const size_t kbase =
            (((size_t)blk * Hkv + g) * bs + (size_t)(t % bs)) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += load_elem(q, q_dtype, qbase + d, NULL, D) *
                 load_elem(k_pool, kv_dtype, kbase + d, k_scales, D);
        scores[t] = sigma * dot;
        if (scores[t] > m) m = scores[t];
      }
      if (bad) {
#pragma omp atomic write
        status = 2;
        continue;
      }
      /* pass 2: weights and the weighted sum of values */
      double l = 0.0;
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        const int32_t blk = tables[(size_t)b * max_blocks + t / bs];
        const size_t vbase =
            (((size_t)blk * Hkv + g) * bs + (size_t)(t % bs)) * D;
        const double p = exp(scores[t] - m);
        l += p;
        for (int d = 0; d < D; ++d)
          acc[d] += p * load_elem(v_pool, kv_dtype, vbase + d, v_scales, D);
      }
      for (int d = 0; d < D; ++d) out[(size_t)r * D + d] = acc[d] / l;
      if (lse) lse[r] = m + log(l);
    }
    free(scores);
    free(acc);
  }
  return status;
}

int pkv_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
