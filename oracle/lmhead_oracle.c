/*
 * Plain fp64 CPU oracle for the chunked LM-head + loss computation.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library.
 *
 * The three contractions of the method, each written as its plain definition:
 *
 *   logits  z[n, v]  = sum_h H[n, h] * W[v, h]            (ascending h)
 *   input grad dH[n, h] = sum_v dZ[n, v] * W[v, h]          (ascending v)
 *   weight grad dW[v, h] = sum_n dZ[n, v] * H[n, h]          (ascending n)
 *
 * (FlashInfer PR #8059 "det names for the chunked LM-head + loss backend":
 * the backend projects hidden states through the vocabulary matrix and
 * returns gradients for both; miles-ext-kernels PR #14, lm_head op commit:
 * the weight gradient is the BF16 cast of an FP32 [V, H] accumulator. The
 * oracle keeps everything in fp64 and does not chunk: chunking and the online
 * logsumexp are exact rewrites of these sums.)
 *
 * Operands are given either as bf16 bit patterns (uint16, widened exactly to
 * fp64) or as fp64 (used by finite-difference checks). Threads only split
 * independent outputs between them; every sum runs in the stated order.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

static double widen_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Row r of a [rows x cols] operand, widened to fp64 into dst[cols]. */
static void load_row(const void* base, int is_f64, int64_t cols, int64_t r, double* dst) {
    if (is_f64) {
        memcpy(dst, (const double*)base + r * cols, (size_t)cols * sizeof(double));
    } else {
        const uint16_t* src = (const uint16_t*)base + r * cols;
        for (int64_t c = 0; c < cols; ++c) dst[c] = widen_bf16(src[c]);
    }
}

static int pick_threads(int threads) {
    if (threads > 0) return threads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

typedef void (*work_fn)(void* ctx, int64_t begin, int64_t end);

typedef struct {
    work_fn fn;
    void* ctx;
    int64_t begin, end;
} span_arg;

static void* span_main(void* p) {
    span_arg* a = (span_arg*)p;
    a->fn(a->ctx, a->begin, a->end);
    return NULL;
}

/* Split [0, total) into contiguous spans, one per thread. */
static int run_spans(work_fn fn, void* ctx, int64_t total, int threads) {
    threads = pick_threads(threads);
    if (threads > total) threads = (int)(total > 0 ? total : 1);
    pthread_t* tid = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
    span_arg* args = (span_arg*)calloc((size_t)threads, sizeof(span_arg));
    if (!tid || !args) { free(tid); free(args); return -1; }
    int started = 0, rc = 0;
    for (int t = 0; t < threads; ++t) {
        args[t].fn = fn;
        args[t].ctx = ctx;
        args[t].begin = total * t / threads;
        args[t].end = total * (t + 1) / threads;
        if (pthread_create(&tid[t], NULL, span_main, &args[t]) != 0) { rc = -1; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    free(tid);
    free(args);
    return rc;
}

/* ------------------------------------------------------------------ logits */

typedef struct {
    const double* hrows;  /* [nr x hidden], selected rows of H in fp64 */
    int64_t nr, hidden, vocab;
    const void* W;
    int w_f64;
    double* z;            /* [nr x vocab] */
} logits_ctx;

static void logits_span(void* p, int64_t v0, int64_t v1) {
    logits_ctx* c = (logits_ctx*)p;
    const int64_t hd = c->hidden;
    double* wrow = (double*)malloc((size_t)hd * sizeof(double));
    if (!wrow) return;
    for (int64_t v = v0; v < v1; ++v) {
        load_row(c->W, c->w_f64, hd, v, wrow);
        int64_t i = 0;
        /* four independent dot products at a time; each keeps ascending h */
        for (; i + 4 <= c->nr; i += 4) {
            const double* h0 = c->hrows + (i + 0) * hd;
            const double* h1 = c->hrows + (i + 1) * hd;
            const double* h2 = c->hrows + (i + 2) * hd;
            const double* h3 = c->hrows + (i + 3) * hd;
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
            for (int64_t h = 0; h < hd; ++h) {
                const double w = wrow[h];
                s0 += h0[h] * w;
                s1 += h1[h] * w;
                s2 += h2[h] * w;
                s3 += h3[h] * w;
            }
            c->z[(i + 0) * c->vocab + v] = s0;
            c->z[(i + 1) * c->vocab + v] = s1;
            c->z[(i + 2) * c->vocab + v] = s2;
            c->z[(i + 3) * c->vocab + v] = s3;
        }
        for (; i < c->nr; ++i) {
            const double* hr = c->hrows + i * hd;
            double s = 0.0;
            for (int64_t h = 0; h < hd; ++h) s += hr[h] * wrow[h];
            c->z[i * c->vocab + v] = s;
        }
    }
    free(wrow);
}

/* z[i, v] = sum_h H[rows[i], h] * W[v, h] for the nr selected rows. */
int oracle_logits(const void* H, int h_f64, int64_t n, int64_t hidden,
                  const int64_t* rows, int64_t nr,
                  const void* W, int w_f64, int64_t vocab,
                  double* z, int threads) {
    if (nr < 0 || hidden <= 0 || vocab <= 0) return -1;
    if (nr == 0) return 0;
    double* hrows = (double*)malloc((size_t)(nr * hidden) * sizeof(double));
    if (!hrows) return -2;
    for (int64_t i = 0; i < nr; ++i) {
        if (rows[i] < 0 || rows[i] >= n) { free(hrows); return -1; }
        load_row(H, h_f64, hidden, rows[i], hrows + i * hidden);
    }
    logits_ctx c = {hrows, nr, hidden, vocab, W, w_f64, z};
    int rc = run_spans(logits_span, &c, vocab, threads);
    free(hrows);
    return rc;
}

/* ---------------------------------------------------------------------- dH */

typedef struct {
    const double* dz;     /* [nr x vocab] */
    int64_t nr, vocab, hidden;
    const void* W;
    int w_f64;
    double* dh;           /* [nr x hidden] */
} dh_ctx;

/* Each thread owns a block of hidden columns for every row. */
static void dh_span(void* p, int64_t h0, int64_t h1) {
    dh_ctx* c = (dh_ctx*)p;
    const int64_t hd = c->hidden, w = h1 - h0;
    double* wseg = (double*)malloc((size_t)w * sizeof(double));
    if (!wseg) return;
    for (int64_t i = 0; i < c->nr; ++i)
        for (int64_t h = h0; h < h1; ++h) c->dh[i * hd + h] = 0.0;
    for (int64_t v = 0; v < c->vocab; ++v) {   /* ascending v */
        if (c->w_f64) {
            memcpy(wseg, (const double*)c->W + v * hd + h0, (size_t)w * sizeof(double));
        } else {
            const uint16_t* src = (const uint16_t*)c->W + v * hd + h0;
            for (int64_t h = 0; h < w; ++h) wseg[h] = widen_bf16(src[h]);
        }
        for (int64_t i = 0; i < c->nr; ++i) {
            const double g = c->dz[i * c->vocab + v];
            if (g == 0.0) continue;  /* adding an exact zero product changes nothing */
            double* out = c->dh + i * hd + h0;
            for (int64_t h = 0; h < w; ++h) out[h] += g * wseg[h];
        }
    }
    free(wseg);
}

/* dh[i, h] = sum_v dz[i, v] * W[v, h]. */
int oracle_dh(const double* dz, int64_t nr, const void* W, int w_f64,
              int64_t vocab, int64_t hidden, double* dh, int threads) {
    if (nr < 0 || hidden <= 0 || vocab <= 0) return -1;
    if (nr == 0) return 0;
    dh_ctx c = {dz, nr, vocab, hidden, W, w_f64, dh};
    return run_spans(dh_span, &c, hidden, threads);
}

/* ---------------------------------------------------------------------- dW */

typedef struct {
    const double* dzt;    /* [nv x nr]: dZ[rows[i], vsel[j]] at dzt[j * nr + i] */
    int64_t nv, nr, hidden;
    const double* hrows;  /* [nr x hidden] */
    double* dw;           /* [nv x hidden] */
} dw_ctx;

static void dw_span(void* p, int64_t j0, int64_t j1) {
    dw_ctx* c = (dw_ctx*)p;
    const int64_t hd = c->hidden;
    for (int64_t j = j0; j < j1; ++j) {
        double* out = c->dw + j * hd;
        for (int64_t h = 0; h < hd; ++h) out[h] = 0.0;
        for (int64_t i = 0; i < c->nr; ++i) {   /* ascending row order */
            const double g = c->dzt[j * c->nr + i];
            if (g == 0.0) continue;
            const double* hr = c->hrows + i * hd;
            for (int64_t h = 0; h < hd; ++h) out[h] += g * hr[h];
        }
    }
}

/* dw[j, h] = sum_i dzt[j, i] * H[rows[i], h] (rows ascending). */
int oracle_dw(const double* dzt, int64_t nv, const void* H, int h_f64,
              int64_t n, int64_t hidden, const int64_t* rows, int64_t nr,
              double* dw, int threads) {
    if (nv < 0 || nr < 0 || hidden <= 0) return -1;
    if (nv == 0) return 0;
    double* hrows = (double*)malloc((size_t)((nr > 0 ? nr : 1) * hidden) * sizeof(double));
    if (!hrows) return -2;
    for (int64_t i = 0; i < nr; ++i) {
        if (rows[i] < 0 || rows[i] >= n) { free(hrows); return -1; }
        load_row(H, h_f64, hidden, rows[i], hrows + i * hidden);
    }
    dw_ctx c = {dzt, nv, nr, hidden, hrows, dw};
    int rc = run_spans(dw_span, &c, nv, threads);
    free(hrows);
    return rc;
}
