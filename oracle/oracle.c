/*
 * oracle.c -- plain, slow, obviously correct CPU reference for paged MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only tests/, the smoke entry point and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, constant table or helper with
 * the HIP path.
 *
 * What it computes (the definition the fast method must reproduce):
 *
 *   For batch b, KV head k, query token s and query head h (h in the k-th group
 *   of h_q/h_kv heads), with L = cache_seqlens[b]:
 *     N     = L                       (non-causal)
 *           = max(0, L - s_q + s + 1) (causal: the s_q queries are the last s_q
 *                                      tokens of the cache, bottom-right aligned)
 *     K_t   = kcache[block_table[b][t / 64], t % 64, k, 0:576]   for t < N
 *     x_t   = scale * sum_d q[b,s,h,d] * K_t[d]                  (fp64)
 *     m     = max_t x_t,  Z = sum_t exp(x_t - m)
 *     out   = sum_t exp(x_t - m) / Z * K_t[0:dv]                 (V = first dv dims)
 *     lse   = m + ln Z ;  N == 0  =>  out = 0, lse = -inf
 *
 * Sources (cited by page title and section):
 *   - score against the cached latent through the absorbed query: the weight
 *     absorption identity q.(W_UK c) = (W_UK^T q).c, "FlashMLA inference
 *     acceleration" notes (dpshk.com/news/5996785), §2.1;
 *   - softmax over the whole cache, computed here in the two-pass textbook form
 *     that the online form must equal, same page §2.2, and the textbook einsum
 *     attention on the "FlashMLA technical principles / DeepSeek-V2-Lite cloud
 *     deployment" page (xfz.ruibaoantu.com article 3725620), §二.1;
 *   - paging: 64-token pages addressed through block_table and cache_seqlens,
 *     "OpenSourceWeek Day 1 -- Demystifying DeepSeek's FlashMLA"
 *     (deepseekonline.chat), §II.1-§II.2 and the API in §V.2; the variable-length
 *     paged cache of "Flash MLA: efficient MLA decoding kernel library for
 *     variable-length sequences" (developer.baidu.com article 7969948), §二-§三.1;
 *   - query-head folding (all q heads sharing one KV head are rows of one
 *     problem): Day-1 page §II.1.
 *
 * The scheduler twin at the bottom restates the split-KV partition that the
 * library's metadata call produces; the pages give only the call's signature
 * (Day-1 page §V.2), so the partition rule is this project's own reading and is
 * written out here independently of the GPU implementation.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 *
 * ORACLE_MUTANT (compile-time, default 0) plants one deliberate mistake so the
 * test suite can show that its pins catch it; the shipped build never sets it:
 *   1 rope dims dropped from the score     2 V read from the wrong end of a row
 *   3 causal mask aligned top-left         4 lse without the running max
 *   5 page index and slot swapped          6 query head -> KV head mapping wrong
 *   7 softmax scale not applied            8 slot off by one inside a page
 */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Full decode.  q: bf16 bits [batch, s_q, h_q, d_qk]; kcache: bf16 bits
 * [num_pages, page, h_kv, d_qk]; block_table: [batch, max_blocks].
 * sel: optional list of n_sel query indices (b*s_q*h_q + s*h_q + h); NULL means
 * all queries in order.  out: fp64 [n, dv]; lse: fp64 [n].
 * Returns 0, or -1 when a referenced page id is outside [0, num_pages).
 */
int oracle_decode(const uint16_t* q, const uint16_t* kcache, long long num_pages,
                  const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                  int batch, int s_q, int h_q, int h_kv, int d_qk, int dv, int page,
                  int causal, double scale, const long long* sel, long long n_sel,
                  double* out, double* lse) {
  const long long total = (long long)batch * s_q * h_q;
  const long long n = sel ? n_sel : total;
  const int group = h_q / h_kv;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long long idx = 0; idx < n; ++idx) {
    const long long qi = sel ? sel[idx] : idx;
    const int b = (int)(qi / ((long long)s_q * h_q));
    const int s = (int)((qi / h_q) % s_q);
    const int h = (int)(qi % h_q);
    const int k = (ORACLE_MUTANT == 6) ? h % h_kv : h / group;
    const long long L = cache_seqlens[b];
    long long N = L;
    if (causal) {
      N = (ORACLE_MUTANT == 3) ? (long long)s + 1 : L - s_q + s + 1;
      if (N > L) N = L;
      if (N < 0) N = 0;
    }
    double* o = out + idx * (long long)dv;
    for (int d = 0; d < dv; ++d) o[d] = 0.0;
    if (N == 0) {
      lse[idx] = -INFINITY;
      continue;
    }
    const uint16_t* qrow = q + qi * (long long)d_qk;
    double* qd = (double*)malloc(sizeof(double) * (size_t)d_qk);
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    const uint16_t** rows = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)N);
    for (int d = 0; d < d_qk; ++d) qd[d] = bf16_to_double(qrow[d]);

    /* gather each key row through the page table, then score it */
    double m = -INFINITY;
    for (long long t = 0; t < N; ++t) {
      const long long blk = (ORACLE_MUTANT == 5) ? (t % page) % max_blocks : t / page;
      const long long slot = (ORACLE_MUTANT == 5) ? t / page
                           : (ORACLE_MUTANT == 8) ? (t % page + 1) % page : t % page;
      const long long pid = block_table[(long long)b * max_blocks + blk];
      if (pid < 0 || pid >= num_pages) {
        bad |= 1;
        x[t] = -INFINITY;
        rows[t] = NULL;
        continue;
      }
      const uint16_t* kr = kcache + ((pid * page + slot % page) * h_kv + k) * (long long)d_qk;
      rows[t] = kr;
      double acc = 0.0;
      const int dscore = (ORACLE_MUTANT == 1) ? dv : d_qk;
      for (int d = 0; d < dscore; ++d) acc += qd[d] * bf16_to_double(kr[d]);
      x[t] = (ORACLE_MUTANT == 7) ? acc : scale * acc;
      if (x[t] > m) m = x[t];
    }
    /* two-pass softmax: normaliser first, then the weighted sum of V rows */
    double Z = 0.0;
    for (long long t = 0; t < N; ++t) Z += exp(x[t] - m);
    const int voff = (ORACLE_MUTANT == 2) ? d_qk - dv : 0;
    for (long long t = 0; t < N; ++t) {
      if (!rows[t]) continue;
      const double p = exp(x[t] - m) / Z;
      for (int d = 0; d < dv; ++d) o[d] += p * bf16_to_double(rows[t][voff + d]);
    }
    lse[idx] = (ORACLE_MUTANT == 4) ? log(Z) : m + log(Z);
    free(qd);
    free(x);
    free(rows);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Scheduler twin.                                                          */
/*
 * Work is counted in units of one 64-token page.  Sequence i needs
 * m_i = max(ceil(L_i / 64), 1) units (one unit even when empty, so that its
 * output is written), preceded by a fixed overhead of OVH units that prices the
 * query load and the split bookkeeping of starting a new chunk.  On the line
 *   C_0 = 0,  A_i = C_i + OVH,  B_i = A_i + m_i,  C_{i+1} = B_i,  T = C_b
 * parts of equal length q = max(ceil(T / P), QMIN) are cut: part(x) = floor(x / q).
 * Sequence i is split into chunks_i = part(B_i - 1) - part(A_i) + 1 chunks, and
 * num_splits is the exclusive prefix sum of chunks (length b + 1).
 * Part p covers [lo, hi) = [p q, min((p+1) q, T)).  Its metadata row is
 *   {i, first - A_i, j, last - A_j + 1, p - part(A_i), 0, 0, 0}
 * with i the first sequence whose work ends after lo, first = max(lo, A_i),
 * j the last sequence whose work starts before hi, last = min(hi, B_j) - 1;
 * an empty part (lo >= T) is {b, 0, b, 0, 0, 0, 0, 0}.
 *
 * Tile rows and the constants: rows <= 16 -> 16, rows <= 128 -> 64, else 128
 * (the row tile one workgroup owns); OVH = 3 for the 16-row tile, tile / 16
 * otherwise; QMIN = 2 * OVH.
 * Written with plain loops over all sequences for every part.
 */
static int twin_tile_rows(int rows) { return rows <= 16 ? 16 : rows <= 128 ? 64 : 128; }

int oracle_tile_rows(int rows) { return twin_tile_rows(rows); }

int oracle_schedule(const int32_t* cache_seqlens, int batch, int rows, int num_parts,
                    int32_t* tile_metadata, int32_t* num_splits) {
  if (batch <= 0 || num_parts <= 0 || rows <= 0) return -1;
  const int tile = twin_tile_rows(rows);
  const long long ovh = tile == 16 ? 3 : tile / 16;
  const long long qmin = 2 * ovh;
  long long* A = (long long*)malloc(sizeof(long long) * (size_t)batch);
  long long* B = (long long*)malloc(sizeof(long long) * (size_t)batch);
  long long c = 0;
  for (int i = 0; i < batch; ++i) {
    long long L = cache_seqlens[i] < 0 ? 0 : cache_seqlens[i];
    long long nb = (L + 63) / 64;
    long long m = nb > 1 ? nb : 1;
    A[i] = c + ovh;
    B[i] = A[i] + m;
    c = B[i];
  }
  const long long T = c;
  long long q = (T + num_parts - 1) / num_parts;
  if (q < qmin) q = qmin;

  num_splits[0] = 0;
  for (int i = 0; i < batch; ++i) {
    long long chunks = (B[i] - 1) / q - A[i] / q + 1;
    num_splits[i + 1] = (int32_t)(num_splits[i] + chunks);
  }
  for (int p = 0; p < num_parts; ++p) {
    int32_t* row = tile_metadata + (long long)p * 8;
    const long long lo = (long long)p * q;
    long long hi = lo + q;
    if (hi > T) hi = T;
    int i = batch;
    for (int t = 0; t < batch; ++t)
      if (B[t] > lo) { i = t; break; }
    if (lo >= T || i == batch) {
      row[0] = batch; row[1] = 0; row[2] = batch; row[3] = 0;
      row[4] = 0; row[5] = 0; row[6] = 0; row[7] = 0;
      continue;
    }
    int j = -1;
    for (int t = 0; t < batch; ++t)
      if (A[t] < hi) j = t;
    const long long first = lo > A[i] ? lo : A[i];
    const long long last = (hi < B[j] ? hi : B[j]) - 1;
    row[0] = i;
    row[1] = (int32_t)(first - A[i]);
    row[2] = j;
    row[3] = (int32_t)(last - A[j] + 1);
    row[4] = (int32_t)(p - A[i] / q);
    row[5] = 0; row[6] = 0; row[7] = 0;
  }
  free(A);
  free(B);
  return 0;
}
