/*
 * Driver for the sanitizer build of the CPU oracle (oracle/oracle.c), linked
 * with -fsanitize=address,undefined by tests/test_sanitizers_cpu.py.  Test
 * infrastructure only.  It runs the oracle's decode and scheduler twin over
 * small cases that reach every branch -- empty and one-token sequences, page
 * edges, causal rows with no key, two KV heads, a selection of rows, a page
 * id outside the cache, scheduler parts past the work -- so that an
 * out-of-bounds access, a leak or undefined behaviour in the oracle stops the
 * run.  Exit status 0 when every call returns what its contract says.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_decode(const uint16_t* q, const uint16_t* kcache, long long num_pages, const int32_t* block_table,
                  int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv, int d_qk,
                  int dv, int page, int causal, double scale, const long long* sel, long long n_sel, double* out,
                  double* lse);
int oracle_schedule(const int32_t* cache_seqlens, int batch, int rows, int num_parts, int32_t* tile_metadata,
                    int32_t* num_splits);
void oracle_set_threads(int n);

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state;
}
/* a bf16 pattern of modest magnitude: sign, exponent 120..129, random mantissa */
static uint16_t rand_bf16(void) {
  uint32_t r = next_u32();
  return (uint16_t)(((r >> 31) << 15) | ((120u + (r >> 8) % 10u) << 7) | (r & 0x7Fu));
}

static int fails = 0;
#define CHECK(c, ...)                     \
  do {                                    \
    if (!(c)) {                           \
      fprintf(stderr, __VA_ARGS__);       \
      fputc('\n', stderr);                \
      ++fails;                            \
    }                                     \
  } while (0)

static void decode_case(const int* lens, int batch, int s_q, int h_q, int h_kv, int causal, int bad_page) {
  const int D = 576, DV = 512, PG = 64;
  int max_blocks = 1;
  long long pages = 0;
  for (int b = 0; b < batch; ++b) {
    int nb = (lens[b] + PG - 1) / PG;
    if (nb > max_blocks) max_blocks = nb;
    pages += nb;
  }
  if (pages == 0) pages = 1;
  int32_t* bt = malloc(sizeof(int32_t) * (size_t)batch * max_blocks);
  long long next = 0;
  for (int b = 0; b < batch; ++b)
    for (int j = 0; j < max_blocks; ++j)
      bt[b * max_blocks + j] = j < (lens[b] + PG - 1) / PG ? (int32_t)((next++ * 7) % pages) : -1;
  if (bad_page && lens[0] > 0) bt[0] = (int32_t)(pages + 3);
  int32_t* sl = malloc(sizeof(int32_t) * (size_t)batch);
  for (int b = 0; b < batch; ++b) sl[b] = lens[b];
  size_t nq = (size_t)batch * s_q * h_q * D, nk = (size_t)pages * PG * h_kv * D;
  uint16_t* q = malloc(sizeof(uint16_t) * nq);
  uint16_t* kc = malloc(sizeof(uint16_t) * nk);
  for (size_t i = 0; i < nq; ++i) q[i] = rand_bf16();
  for (size_t i = 0; i < nk; ++i) kc[i] = rand_bf16();
  long long rows = (long long)batch * s_q * h_q;
  double* out = malloc(sizeof(double) * (size_t)rows * DV);
  double* lse = malloc(sizeof(double) * (size_t)rows);
  int rc = oracle_decode(q, kc, pages, bt, max_blocks, sl, batch, s_q, h_q, h_kv, D, DV, PG, causal,
                         1.0 / sqrt(192.0), NULL, 0, out, lse);
  CHECK(rc == (bad_page && lens[0] > 0 ? -1 : 0), "decode status %d", rc);
  for (long long r = 0; r < rows; ++r) {
    CHECK(!isnan(lse[r]), "lse NaN at row %lld", r);
    for (int d = 0; d < DV; ++d) CHECK(isfinite(out[r * DV + d]), "out not finite at row %lld", r);
  }
  /* a selection: every third row, in reverse */
  long long nsel = (rows + 2) / 3;
  long long* sel = malloc(sizeof(long long) * (size_t)nsel);
  for (long long i = 0; i < nsel; ++i) sel[i] = rows - 1 - 3 * i;
  double* out2 = malloc(sizeof(double) * (size_t)nsel * DV);
  double* lse2 = malloc(sizeof(double) * (size_t)nsel);
  rc = oracle_decode(q, kc, pages, bt, max_blocks, sl, batch, s_q, h_q, h_kv, D, DV, PG, causal,
                     1.0 / sqrt(192.0), sel, nsel, out2, lse2);
  for (long long i = 0; i < nsel; ++i) {
    CHECK(lse2[i] == lse[sel[i]] || (isinf(lse2[i]) && isinf(lse[sel[i]])), "selected lse differs");
    for (int d = 0; d < DV; ++d) CHECK(out2[i * DV + d] == out[sel[i] * DV + d], "selected out differs");
  }
  free(sel); free(out2); free(lse2);
  free(bt); free(sl); free(q); free(kc); free(out); free(lse);
}

static void schedule_case(const int32_t* lens, int batch, int rows, int parts) {
  int32_t* md = malloc(sizeof(int32_t) * 8 * (size_t)parts);
  int32_t* ns = malloc(sizeof(int32_t) * (size_t)(batch + 1));
  int rc = oracle_schedule(lens, batch, rows, parts, md, ns);
  CHECK(rc == 0, "schedule status %d", rc);
  CHECK(ns[0] == 0, "num_splits[0]");
  for (int i = 0; i < batch; ++i) CHECK(ns[i + 1] > ns[i], "num_splits not increasing");
  for (int p = 0; p < parts; ++p) CHECK(md[8 * p] >= 0 && md[8 * p] <= batch, "first sequence out of range");
  free(md);
  free(ns);
}

int main(void) {
  oracle_set_threads(2);
  const int l1[] = {0, 1, 63, 64, 65, 200};
  decode_case(l1, 6, 1, 4, 1, 0, 0);
  decode_case(l1, 6, 2, 4, 1, 1, 0);     /* causal: rows of the 1-token sequence see 0 or 1 key */
  const int l2[] = {130, 5};
  decode_case(l2, 2, 3, 4, 2, 1, 0);     /* two KV heads */
  decode_case(l2, 2, 1, 2, 1, 0, 1);     /* a page id outside the cache */
  const int l3[] = {0, 0};
  decode_case(l3, 2, 1, 2, 1, 0, 0);     /* nothing cached */

  for (int k = 0; k < 200; ++k) {
    int batch = 1 + (int)(next_u32() % 60);
    int32_t* lens = malloc(sizeof(int32_t) * (size_t)batch);
    for (int i = 0; i < batch; ++i) lens[i] = (int32_t)(next_u32() % (k % 3 == 0 ? 3u : 20000u));
    int rows = (k % 2) ? 16 : 256;
    int parts = 1 + (int)(next_u32() % 400);
    schedule_case(lens, batch, rows, parts);
    free(lens);
  }
  int32_t dummy = 5, md[8], ns[2];
  CHECK(oracle_schedule(&dummy, 0, 16, 1, md, ns) != 0, "empty batch accepted");
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
