/*
 * sanitize_oracle_driver.c -- runs every entry point of the fp64 oracle
 * (oracle/fd_oracle.c) on small seeded inputs, for a build with
 * -fsanitize=address,undefined (tests/test_sanitizers.py).  Test
 * infrastructure: memory errors and undefined behaviour abort the run; the
 * checks here are consistency checks between entry points (split against
 * unsplit, paged and multi-token against the plain decode), not parity.
 * Exits 0 when every call returns 0 and every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int fdo_decode(const void *q, const void *k, const void *v,
               const int32_t *seqlens, int B, int Hq, int Hkv, int D,
               int Lmax, double scale, int dtype, int nthreads, double *out,
               double *lse);
int fdo_decode_split(const void *q, const void *k, const void *v,
                     const int32_t *seqlens, int B, int Hq, int Hkv, int D,
                     int Lmax, double scale, int dtype, int chunk,
                     int nthreads, double *out, double *lse);
int fdo_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                     const int32_t *block_table, int max_pages, int page_size,
                     int num_pages, int head_major, const int32_t *seqlens,
                     int B, int Tq, int Hq, int Hkv, int D, double scale,
                     int dtype, int nthreads, double *out, double *lse);
int fdo_decode_multiquery(const void *q, const void *k, const void *v,
                          const int32_t *seqlens, int B, int Tq, int Hq,
                          int Hkv, int D, int Lmax, double scale, int dtype,
                          int nthreads, double *out, double *lse);

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* xorshift64*, in [-2, 2) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 2685821657736338717ull) >> 11) * 0x1.0p-51 - 2.0;
}

static uint16_t bf16(double x) { /* truncation is enough for test data */
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int failures = 0;

static void expect(const char *what, int ok) {
  if (!ok) {
    printf("FAIL %s\n", what);
    ++failures;
  }
}

static double max_diff(const double *a, const double *b, size_t n) {
  double m = 0.0;
  for (size_t i = 0; i < n; ++i) {
    if (isinf(a[i]) && isinf(b[i]) && a[i] == b[i]) continue;
    const double d = fabs(a[i] - b[i]);
    if (!(d <= m)) m = d; /* NaN propagates as a failure */
  }
  return m;
}

int main(void) {
  enum { B = 3, Hq = 8, Hkv = 2, D = 64, Lmax = 200, P = 16, Tq = 3 };
  const int32_t seqlens[B] = {200, 37, 0};
  const size_t nq = (size_t)B * Hq * D, nkv = (size_t)B * Hkv * Lmax * D;
  uint16_t *q = malloc(nq * 2), *k = malloc(nkv * 2), *v = malloc(nkv * 2);
  uint16_t *qm = malloc(nq * Tq * 2);
  double *o1 = malloc(nq * 8), *o2 = malloc(nq * 8);
  double *l1 = malloc((size_t)B * Hq * 8), *l2 = malloc((size_t)B * Hq * 8);
  double *om = malloc(nq * Tq * 8), *lm = malloc((size_t)B * Tq * Hq * 8);
  if (!q || !k || !v || !qm || !o1 || !o2 || !l1 || !l2 || !om || !lm)
    return 2;
  for (size_t i = 0; i < nq; ++i) q[i] = bf16(uniform());
  for (size_t i = 0; i < nq * Tq; ++i) qm[i] = bf16(uniform());
  /* rows past a sequence's length hold NaN bits: they must never be read */
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int j = 0; j < Lmax; ++j)
        for (int d = 0; d < D; ++d) {
          const size_t i = (((size_t)b * Hkv + g) * Lmax + j) * D + d;
          k[i] = j < seqlens[b] ? bf16(uniform()) : 0xFFFF;
          v[i] = j < seqlens[b] ? bf16(uniform()) : 0xFFFF;
        }
  const double scale = 0.125;

  expect("decode", fdo_decode(q, k, v, seqlens, B, Hq, Hkv, D, Lmax, scale,
                              0, 2, o1, l1) == 0);
  for (size_t i = 0; i < nq; ++i) expect("finite out", isfinite(o1[i]));
  for (int chunk = 1; chunk <= Lmax + 7; chunk += 41) {
    expect("split", fdo_decode_split(q, k, v, seqlens, B, Hq, Hkv, D, Lmax,
                                     scale, 0, chunk, 2, o2, l2) == 0);
    expect("split out", max_diff(o1, o2, nq) < 1e-12);
    expect("split lse", max_diff(l1, l2, (size_t)B * Hq) < 1e-12);
  }
  /* the same bits read as fp16 (finite values; the NaN padding too) */
  expect("decode f16", fdo_decode(q, k, v, seqlens, B, Hq, Hkv, D, Lmax,
                                  scale, 2, 2, o2, l2) == 0);
  for (size_t i = 0; i < nq; ++i) expect("finite f16 out", isfinite(o2[i]));
  /* lengths beyond Lmax are clamped */
  const int32_t too_long[B] = {Lmax + 50, 37, 0};
  expect("clamped", fdo_decode(q, k, v, too_long, B, Hq, Hkv, D, Lmax, scale,
                               0, 1, o2, l2) == 0);
  expect("clamped out", max_diff(o1, o2, nq) == 0.0);

  /* the same cache in pages (token-major, then head-major), pages of P
     keys in reverse order in the pool */
  const int max_pages = (Lmax + P - 1) / P, num_pages = B * max_pages;
  int32_t *table = malloc((size_t)B * max_pages * 4);
  uint16_t *kp = malloc((size_t)num_pages * P * Hkv * D * 2);
  uint16_t *vp = malloc((size_t)num_pages * P * Hkv * D * 2);
  if (!table || !kp || !vp) return 2;
  for (int hm = 0; hm < 2; ++hm) {
    memset(kp, 0xFF, (size_t)num_pages * P * Hkv * D * 2);
    memset(vp, 0xFF, (size_t)num_pages * P * Hkv * D * 2);
    for (int b = 0; b < B; ++b)
      for (int pg = 0; pg < max_pages; ++pg) {
        const int phys = num_pages - 1 - (b * max_pages + pg);
        table[b * max_pages + pg] = phys;
        for (int t = 0; t < P; ++t) {
          const int j = pg * P + t;
          if (j >= Lmax) continue;
          for (int g = 0; g < Hkv; ++g) {
            const size_t src = (((size_t)b * Hkv + g) * Lmax + j) * D;
            const size_t dst =
                hm ? (((size_t)phys * Hkv + g) * P + t) * D
                   : (((size_t)phys * P + t) * Hkv + g) * D;
            memcpy(kp + dst, k + src, (size_t)D * 2);
            memcpy(vp + dst, v + src, (size_t)D * 2);
          }
        }
      }
    expect("paged", fdo_decode_paged(q, kp, vp, table, max_pages, P,
                                     num_pages, hm, seqlens, B, 1, Hq, Hkv,
                                     D, scale, 0, 2, o2, l2) == 0);
    expect("paged out", max_diff(o1, o2, nq) < 1e-12);
    expect("paged lse", max_diff(l1, l2, (size_t)B * Hq) < 1e-12);
  }

  /* several new tokens; the newest sees every key, as the plain decode */
  expect("multiquery", fdo_decode_multiquery(qm, k, v, seqlens, B, Tq, Hq,
                                             Hkv, D, Lmax, scale, 0, 2, om,
                                             lm) == 0);
  for (int b = 0; b < B; ++b)
    memcpy(q + (size_t)b * Hq * D, qm + ((size_t)b * Tq + Tq - 1) * Hq * D,
           (size_t)Hq * D * 2);
  expect("decode newest", fdo_decode(q, k, v, seqlens, B, Hq, Hkv, D, Lmax,
                                     scale, 0, 1, o1, l1) == 0);
  for (int b = 0; b < B; ++b) {
    const double *a = om + ((size_t)b * Tq + Tq - 1) * Hq * D;
    expect("newest token out",
           max_diff(a, o1 + (size_t)b * Hq * D, (size_t)Hq * D) < 1e-12);
  }

  /* argument errors are reported, not run */
  expect("bad dims", fdo_decode(q, k, v, seqlens, B, 6, 4, D, Lmax, scale, 0,
                                1, o1, l1) != 0);

  free(q); free(k); free(v); free(qm); free(o1); free(o2); free(l1);
  free(l2); free(om); free(lm); free(table); free(kp); free(vp);
  printf("%s\n", failures ? "failures" : "ok");
  return failures ? 1 : 0;
}
