/*
 * fd_oracle.c -- exact fp64 CPU oracle for single-query decode attention.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
 * smoke check and the benchmark's CPU-baseline leg may load this library.
 * It shares no source, header, table or helper with the GPU library; it
 * decodes bf16 and fp16 itself and needs nothing but libc, libm and
 * OpenMP.
 *
 * What it computes.  "Flash-Decoding for long-context inference" (Dao,
 * Haziza, Massa, Sizov; Stanford CRFM blog), section "Multi-head attention
 * for decoding": while decoding, the one new query of a head attends to
 * every earlier token held in the KV cache.  The page's formula did not
 * survive extraction; the plain reading taken here is softmax attention
 * with a caller-given scale and no mask:
 *
 *     s_j  = scale * sum_d q[d] * K[j][d]          j = 0 .. L-1
 *     m    = max_j s_j
 *     l    = sum_j exp(s_j - m)
 *     out  = (sum_j exp(s_j - m) * V[j]) / l
 *     lse  = m + ln(l)                              (natural log)
 *     L = 0  ->  out = 0, lse = -inf
 *
 * Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 * Cache layout K, V: [B][Hkv][Lmax][D], contiguous; q, out: [B][Hq][D].
 * seqlens (optional) gives the valid prefix of each sequence; rows at or
 * beyond it are never read.  A seqlen outside [0, Lmax] is clamped.
 *
 * Two cache variants the pages point to (a note on the Flash-Decoding
 * search-result page that frameworks store the KV cache very differently,
 * and that decoding may process several new query tokens at once, as in
 * speculative decoding):
 *   paged:       row j of sequence b lives in page block_table[b][j /
 *                page_size], token j % page_size, of a page pool laid out
 *                token-major, K, V [num_pages][page_size][Hkv][D], or
 *                head-major, K, V [num_pages][Hkv][page_size][D] (two of
 *                the ways frameworks store it).  Same definition over the
 *                same rows.
 *   multi-query: q [B][Tq][Hq][D] holds the Tq newest tokens of each
 *                sequence, whose K/V are the last Tq rows of its cache;
 *                query t sees rows j < seqlens[b] - (Tq - 1 - t) (causal).
 *
 * The split/combine twin follows the section "A faster attention for
 * decoding: Flash-Decoding" of the same page: the keys/values are cut into
 * contiguous chunks, each chunk's attention is computed on its own together
 * with one log-sum-exp per row and chunk, and the chunks are then merged by
 * weighting each chunk's output with exp(its lse - max lse).  It exists so
 * that tests can check that splitting and merging reproduce the exact
 * result; it is written in fp64 with nothing reordered beyond that.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (never
 * -ffast-math: exp/log/max must keep IEEE semantics, NaN included).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define FDO_BF16 0
#define FDO_F32 1
#define FDO_F16 2

#define FDO_OK 0
#define FDO_EINVAL -1
#define FDO_ENOMEM -2

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 holds zero and the subnormals (fraction * 2^-24), exponent 31
 * infinity (fraction 0) and NaN; otherwise the value is
 * (1024 + fraction) * 2^(exponent - 25).  Every binary16 value is exact in
 * a double. */
static double half_to_double(uint16_t h)
{
    const int e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return (h & 0x8000) ? -v : v;
}

static int dtype_ok(int dtype)
{
    return dtype == FDO_BF16 || dtype == FDO_F32 || dtype == FDO_F16;
}

static size_t elem_bytes(int dtype)
{
    return dtype == FDO_F32 ? 4 : 2;
}

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double load_elem(const void *base, size_t idx, int dtype)
{
    if (dtype == FDO_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == FDO_F16)
        return half_to_double(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/*
 * One query row against L rows of K/V.  q_off is the element offset of the
 * query in q.  Row j starts at element row_off[j] of k and v, or, when
 * row_off is NULL, at kv_off + j * D (a contiguous slab).  scratch must hold
 * L doubles.  Two exact passes: scores and their max, then the exp-weighted
 * sums.
 */
static void attend_row(const void *q, size_t q_off, const void *k,
                       const void *v, size_t kv_off, const size_t *row_off,
                       int L, int D, double scale, int dtype, double *out,
                       double *lse, double *scratch)
{
    if (L <= 0) {
        for (int d = 0; d < D; ++d)
            out[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    int saw_nan = 0;
    for (int j = 0; j < L; ++j) {
        const size_t r = row_off ? row_off[j] : kv_off + (size_t)j * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += load_elem(q, q_off + d, dtype) * load_elem(k, r + d, dtype);
        double s = scale * dot;
        scratch[j] = s;
        if (isnan(s))
            saw_nan = 1;
        else if (s > m)
            m = s;
    }
    if (saw_nan)
        m = NAN; /* a NaN score makes the whole row NaN */
    double l = 0.0;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    for (int j = 0; j < L; ++j) {
        const size_t r = row_off ? row_off[j] : kv_off + (size_t)j * D;
        double p = exp(scratch[j] - m);
        l += p;
        for (int d = 0; d < D; ++d)
            out[d] += p * load_elem(v, r + d, dtype);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= l;
    *lse = m + log(l);
}

static int clamp_len(const int32_t *seqlens, int b, int Lmax)
{
    if (!seqlens)
        return Lmax;
    int L = seqlens[b];
    if (L < 0)
        L = 0;
    if (L > Lmax)
        L = Lmax;
    return L;
}

static int check_dims(int B, int Hq, int Hkv, int D, int Lmax, int dtype)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax <= 0)
        return FDO_EINVAL;
    if (Hq % Hkv != 0)
        return FDO_EINVAL;
    if (!dtype_ok(dtype))
        return FDO_EINVAL;
    return FDO_OK;
}

/*
 * Whole batch, exact definition.  out: [B][Hq][D] doubles, lse: [B][Hq].
 * nthreads <= 0 lets OpenMP choose.
 */
int fdo_decode(const void *q, const void *k, const void *v,
               const int32_t *seqlens, int B, int Hq, int Hkv, int D,
               int Lmax, double scale, int dtype, int nthreads, double *out,
               double *lse)
{
    int rc = check_dims(B, Hq, Hkv, D, Lmax, dtype);
    if (rc)
        return rc;
    const int G = Hq / Hkv;
    const long rows = (long)B * Hq;
    int failed = 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double *scratch = malloc(sizeof(double) * (size_t)Lmax);
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < rows; ++r) {
            if (!scratch)
                continue;
            int b = (int)(r / Hq), h = (int)(r % Hq);
            int g = h / G;
            size_t q_off = ((size_t)b * Hq + h) * D;
            size_t kv_off = ((size_t)b * Hkv + g) * (size_t)Lmax * D;
            attend_row(q, q_off, k, v, kv_off, NULL,
                       clamp_len(seqlens, b, Lmax), D, scale, dtype,
                       out + (size_t)r * D, lse + r, scratch);
        }
        free(scratch);
    }
    return failed ? FDO_ENOMEM : FDO_OK;
}

/*
 * One query row against one slab given directly ([L][D] rows, D apart).
 * Used to check single outputs of full-size runs without materialising
 * the whole cache on the host.
 */
int fdo_attend_row(const void *q_row, const void *k_slab, const void *v_slab,
                   int L, int D, double scale, int dtype, double *out,
                   double *lse)
{
    if (D <= 0 || L < 0 || !dtype_ok(dtype))
        return FDO_EINVAL;
    double *scratch = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    if (!scratch)
        return FDO_ENOMEM;
    attend_row(q_row, 0, k_slab, v_slab, 0, NULL, L, D, scale, dtype, out,
               lse, scratch);
    free(scratch);
    return FDO_OK;
}

/*
 * Split/combine twin for one row.  Chunk c covers keys
 * [c*chunk, min((c+1)*chunk, L)); chunks past L are empty and skipped.
 * If part_out / part_lse are given they receive each chunk's normalised
 * output ([nchunks][D]) and log-sum-exp ([nchunks]); empty chunks get
 * out = 0 and lse = -inf there.
 */
int fdo_attend_row_split(const void *q_row, const void *k_slab,
                         const void *v_slab, int L, int D, double scale,
                         int dtype, int chunk, int nchunks, double *out,
                         double *lse, double *part_out, double *part_lse)
{
    if (D <= 0 || L < 0 || chunk <= 0 || nchunks <= 0 ||
        !dtype_ok(dtype))
        return FDO_EINVAL;
    if ((long)chunk * nchunks < L)
        return FDO_EINVAL;
    double *scratch = malloc(sizeof(double) * (size_t)chunk);
    double *po = malloc(sizeof(double) * (size_t)nchunks * D);
    double *pl = malloc(sizeof(double) * (size_t)nchunks);
    if (!scratch || !po || !pl) {
        free(scratch);
        free(po);
        free(pl);
        return FDO_ENOMEM;
    }
    /* Step 1: each chunk on its own, with its own log-sum-exp. */
    for (int c = 0; c < nchunks; ++c) {
        long lo = (long)c * chunk;
        long n = L - lo;
        if (n > chunk)
            n = chunk;
        if (n < 0)
            n = 0;
        attend_row(q_row, 0, k_slab, v_slab, (size_t)lo * D, NULL, (int)n, D,
                   scale, dtype, po + (size_t)c * D, pl + c, scratch);
    }
    /* Step 2: merge the chunks, weighting each by exp(lse_c - max lse). */
    double M = -INFINITY;
    int any = 0, saw_nan = 0;
    for (int c = 0; c < nchunks; ++c) {
        if ((long)c * chunk >= L)
            continue;
        any = 1;
        if (isnan(pl[c]))
            saw_nan = 1;
        else if (pl[c] > M)
            M = pl[c];
    }
    if (saw_nan)
        M = NAN;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (!any) {
        *lse = -INFINITY;
    } else {
        double W = 0.0;
        for (int c = 0; c < nchunks; ++c) {
            if ((long)c * chunk >= L)
                continue;
            double w = exp(pl[c] - M);
            W += w;
            for (int d = 0; d < D; ++d)
                out[d] += w * po[(size_t)c * D + d];
        }
        for (int d = 0; d < D; ++d)
            out[d] /= W;
        *lse = M + log(W);
    }
    if (part_out)
        memcpy(part_out, po, sizeof(double) * (size_t)nchunks * D);
    if (part_lse)
        memcpy(part_lse, pl, sizeof(double) * (size_t)nchunks);
    free(scratch);
    free(po);
    free(pl);
    return FDO_OK;
}

/* Whole batch through the split/combine twin, chunk keys per split. */
int fdo_decode_split(const void *q, const void *k, const void *v,
                     const int32_t *seqlens, int B, int Hq, int Hkv, int D,
                     int Lmax, double scale, int dtype, int chunk,
                     int nthreads, double *out, double *lse)
{
    int rc = check_dims(B, Hq, Hkv, D, Lmax, dtype);
    if (rc)
        return rc;
    if (chunk <= 0)
        return FDO_EINVAL;
    const int G = Hq / Hkv;
    const int nchunks = (Lmax + chunk - 1) / chunk;
    const long rows = (long)B * Hq;
    const size_t elem = elem_bytes(dtype);
    int err = 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long r = 0; r < rows; ++r) {
        int b = (int)(r / Hq), h = (int)(r % Hq);
        int g = h / G;
        const char *qr = (const char *)q + ((size_t)b * Hq + h) * D * elem;
        size_t kv = ((size_t)b * Hkv + g) * (size_t)Lmax * D * elem;
        int e = fdo_attend_row_split(qr, (const char *)k + kv,
                                     (const char *)v + kv,
                                     clamp_len(seqlens, b, Lmax), D, scale,
                                     dtype, chunk, nchunks,
                                     out + (size_t)r * D, lse + r, NULL, NULL);
        if (e) {
#pragma omp atomic write
            err = e;
        }
    }
    return err;
}

/*
 * Paged cache, block_table [B][max_pages].  With pg = block_table[b][j /
 * page_size] and t = j % page_size, row j of (b, kv-head g) starts at element
 *   token-major (head_major = 0), K, V [num_pages][page_size][Hkv][D]:
 *       ((pg * page_size + t) * Hkv + g) * D
 *   head-major  (head_major = 1), K, V [num_pages][Hkv][page_size][D]:
 *       ((pg * Hkv + g) * page_size + t) * D
 * seqlens is required; a length beyond max_pages * page_size is clamped, and
 * a page index outside [0, num_pages) is an error (FDO_EINVAL).
 * Tq new tokens per sequence, as in fdo_decode_multiquery: q, out
 * [B][Tq][Hq][D], lse [B][Tq][Hq]; token t sees the first
 * L - (Tq - 1 - t) of the sequence's rows (Tq = 1: plain decode).
 */
int fdo_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                     const int32_t *block_table, int max_pages, int page_size,
                     int num_pages, int head_major, const int32_t *seqlens,
                     int B, int Tq, int Hq, int Hkv, int D, double scale,
                     int dtype, int nthreads, double *out, double *lse)
{
    if (max_pages <= 0 || page_size <= 0 || num_pages <= 0 || !seqlens)
        return FDO_EINVAL;
    if (Tq <= 0)
        return FDO_EINVAL;
    if (head_major != 0 && head_major != 1)
        return FDO_EINVAL;
    const int Lcap = max_pages * page_size;
    int rc = check_dims(B, Hq, Hkv, D, Lcap, dtype);
    if (rc)
        return rc;
    for (int b = 0; b < B; ++b) {
        int L = clamp_len(seqlens, b, Lcap);
        for (int p = 0; p < (L + page_size - 1) / page_size; ++p) {
            int pg = block_table[(size_t)b * max_pages + p];
            if (pg < 0 || pg >= num_pages)
                return FDO_EINVAL;
        }
    }
    const int G = Hq / Hkv;
    const long rows = (long)B * Tq * Hq;
    int failed = 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double *scratch = malloc(sizeof(double) * (size_t)Lcap);
        size_t *roff = malloc(sizeof(size_t) * (size_t)Lcap);
        if (!scratch || !roff) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < rows; ++r) {
            if (!scratch || !roff)
                continue;
            int b = (int)(r / ((long)Tq * Hq)), h = (int)(r % Hq);
            int tok = (int)((r / Hq) % Tq);
            int g = h / G;
            int L = clamp_len(seqlens, b, Lcap);
            /* causal among the new tokens: later ones' rows are not seen */
            L -= Tq - 1 - tok;
            if (L < 0)
                L = 0;
            for (int j = 0; j < L; ++j) {
                size_t pg = (size_t)block_table[(size_t)b * max_pages +
                                                j / page_size];
                size_t t = (size_t)(j % page_size);
                if (head_major)
                    roff[j] = ((pg * Hkv + g) * page_size + t) * (size_t)D;
                else
                    roff[j] = ((pg * page_size + t) * Hkv + g) * (size_t)D;
            }
            attend_row(q, (size_t)r * D, k_pages, v_pages, 0, roff, L, D,
                       scale, dtype, out + (size_t)r * D, lse + r, scratch);
        }
        free(scratch);
        free(roff);
    }
    return failed ? FDO_ENOMEM : FDO_OK;
}

/*
 * Multi-query decode: q, out [B][Tq][Hq][D], lse [B][Tq][Hq].  The Tq query
 * tokens are the newest Tq tokens of the sequence (already in the cache);
 * query t sees rows j < seqlens[b] - (Tq - 1 - t), clamped at 0.
 */
int fdo_decode_multiquery(const void *q, const void *k, const void *v,
                          const int32_t *seqlens, int B, int Tq, int Hq,
                          int Hkv, int D, int Lmax, double scale, int dtype,
                          int nthreads, double *out, double *lse)
{
    int rc = check_dims(B, Hq, Hkv, D, Lmax, dtype);
    if (rc)
        return rc;
    if (Tq <= 0)
        return FDO_EINVAL;
    const int G = Hq / Hkv;
    const long rows = (long)B * Tq * Hq;
    int failed = 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double *scratch = malloc(sizeof(double) * (size_t)Lmax);
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < rows; ++r) {
            if (!scratch)
                continue;
            int b = (int)(r / ((long)Tq * Hq));
            int t = (int)((r / Hq) % Tq), h = (int)(r % Hq);
            int g = h / G;
            int L = clamp_len(seqlens, b, Lmax) - (Tq - 1 - t);
            if (L < 0)
                L = 0;
            size_t kv_off = ((size_t)b * Hkv + g) * (size_t)Lmax * D;
            attend_row(q, (size_t)r * D, k, v, kv_off, NULL, L, D, scale,
                       dtype, out + (size_t)r * D, lse + r, scratch);
        }
        free(scratch);
    }
    return failed ? FDO_ENOMEM : FDO_OK;
}
