/*
 * zio.c -- CPU oracle primitives for memory-centric tiling of Y = XW.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * loads it.
 *
 * What lives here is deliberately small and plain:
 *   - decode of IEEE-754 binary16 and bfloat16 into double (exact),
 *   - round-to-nearest-even encode of double into binary16 / bfloat16,
 *     written from the format definitions (sign, biased exponent, fraction;
 *     subnormals; overflow to infinity),
 *   - a gather that decodes an arbitrary row/column subset of a strided
 *     16-bit matrix into a dense double matrix (data movement only),
 *   - one matrix product  C[r][c] = sum_{i<k} A[r][i] * B[c][i]  in double,
 *     each dot product summed in ascending i,
 *   - GeLU and its derivative in the exact (erf) form, via libm erfc.
 * The method's steps (the untiled product, its adjoints, the FFN chain) are
 * composed from these in oracle/__init__.py, in the order the pages give.
 *
 * Threads split the output grid only; every output element is one dot
 * product computed by one thread in ascending order, so the result does not
 * depend on the thread count.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ZIO_F16 1
#define ZIO_BF16 2

/* ------------------------------------------------------------------ */
/* threads                                                             */
/* ------------------------------------------------------------------ */

static int g_threads = 0;

static int default_threads(void) {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0) return n;
    }
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

int zio_set_threads(int n) {
    g_threads = n > 0 ? n : default_threads();
    return g_threads;
}

int zio_get_threads(void) {
    if (g_threads <= 0) g_threads = default_threads();
    return g_threads;
}

typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);

typedef struct {
    range_fn fn;
    void *ctx;
    int64_t lo, hi;
} range_job;

static void *range_thunk(void *p) {
    range_job *j = (range_job *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

/* Run fn over [0, n) split into contiguous ranges, one per thread. */
static void parallel_range(int64_t n, range_fn fn, void *ctx) {
    int nt = zio_get_threads();
    if (n <= 0) return;
    if (nt > n) nt = (int)n;
    if (nt <= 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t *tid = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    range_job *jobs = (range_job *)calloc((size_t)nt, sizeof(range_job));
    char *live = (char *)calloc((size_t)nt, 1);
    for (int i = 0; i < nt; ++i) {
        jobs[i].fn = fn;
        jobs[i].ctx = ctx;
        jobs[i].lo = n * i / nt;
        jobs[i].hi = n * (i + 1) / nt;
        if (pthread_create(&tid[i], NULL, range_thunk, &jobs[i]) == 0)
            live[i] = 1;
        else
            range_thunk(&jobs[i]); /* run inline if a thread cannot start */
    }
    for (int i = 0; i < nt; ++i)
        if (live[i]) pthread_join(tid[i], NULL);
    free(live);
    free(tid);
    free(jobs);
}

/* ------------------------------------------------------------------ */
/* binary16 / bfloat16                                                 */
/* ------------------------------------------------------------------ */

/* Format parameters: fraction bits and exponent bits. */
static int frac_bits(int dt) { return dt == ZIO_F16 ? 10 : 7; }
static int exp_bits(int dt) { return dt == ZIO_F16 ? 5 : 8; }

/* Exact value of a 16-bit pattern: (-1)^s * 2^(e-bias) * 1.f for normal
 * numbers, (-1)^s * 2^(1-bias) * 0.f for subnormals, inf/NaN at e = max. */
double zio_decode1(int dt, uint16_t bits) {
    int mb = frac_bits(dt), eb = exp_bits(dt);
    int bias = (1 << (eb - 1)) - 1;
    int s = (bits >> 15) & 1;
    int e = (bits >> mb) & ((1 << eb) - 1);
    int f = bits & ((1 << mb) - 1);
    double v;
    if (e == 0)
        v = ldexp((double)f, 1 - bias - mb);
    else if (e == (1 << eb) - 1)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + (1 << mb)), e - bias - mb);
    return s ? -v : v;
}

/* Round x to the nearest representable value, ties to the even fraction,
 * and return its bit pattern.  Magnitudes past the largest finite value
 * after rounding become infinity; NaN becomes a quiet NaN. */
uint16_t zio_encode1(int dt, double x) {
    int mb = frac_bits(dt), eb = exp_bits(dt);
    int bias = (1 << (eb - 1)) - 1;
    int emin = 1 - bias;
    uint16_t sign = signbit(x) ? (uint16_t)0x8000 : (uint16_t)0;
    uint16_t exp_all = (uint16_t)(((1 << eb) - 1) << mb);
    if (isnan(x)) return (uint16_t)(sign | exp_all | (1 << (mb - 1)));
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | exp_all);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < emin) E = emin; /* subnormal range: spacing of the smallest binade */
    double q = ldexp(1.0, E - mb);   /* spacing of representable values at a */
    double r = nearbyint(a / q) * q; /* a/q is exact; nearbyint rounds half to even */
    double max_finite = ldexp(2.0 - ldexp(1.0, -mb), bias);
    if (r > max_finite) return (uint16_t)(sign | exp_all);
    if (r < ldexp(1.0, emin)) {
        /* subnormal: fraction counts units of 2^(emin - mb) */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, emin - mb)));
    }
    frexp(r, &e2);
    E = e2 - 1;
    uint32_t frac = (uint32_t)(r / ldexp(1.0, E - mb)) - (1u << mb);
    return (uint16_t)(sign | (uint16_t)((E + bias) << mb) | (uint16_t)frac);
}

int zio_decode(int dt, const uint16_t *src, int64_t n, double *dst) {
    if (dt != ZIO_F16 && dt != ZIO_BF16) return 1;
    for (int64_t i = 0; i < n; ++i) dst[i] = zio_decode1(dt, src[i]);
    return 0;
}

int zio_encode(int dt, const double *src, int64_t n, uint16_t *dst) {
    if (dt != ZIO_F16 && dt != ZIO_BF16) return 1;
    for (int64_t i = 0; i < n; ++i) dst[i] = zio_encode1(dt, src[i]);
    return 0;
}

/* ------------------------------------------------------------------ */
/* gather: dst[r][c] = decode(base[rows[r]*row_stride + cols[c]*col_stride]) */
/* ------------------------------------------------------------------ */

typedef struct {
    int dt;
    const uint16_t *base;
    int64_t rs, cs, nc;
    const int64_t *rows, *cols;
    double *dst;
    double lut[65536];
} gather_ctx;

static void gather_rows(void *p, int64_t lo, int64_t hi) {
    gather_ctx *g = (gather_ctx *)p;
    for (int64_t r = lo; r < hi; ++r) {
        int64_t ri = g->rows ? g->rows[r] : r;
        const uint16_t *row = g->base + ri * g->rs;
        double *out = g->dst + r * g->nc;
        for (int64_t c = 0; c < g->nc; ++c) {
            int64_t ci = g->cols ? g->cols[c] : c;
            out[c] = g->lut[row[ci * g->cs]];
        }
    }
}

int zio_gather(int dt, const uint16_t *base, int64_t row_stride, int64_t col_stride,
               int64_t nr, const int64_t *rows, int64_t nc, const int64_t *cols,
               double *dst) {
    if (dt != ZIO_F16 && dt != ZIO_BF16) return 1;
    if (!base || !dst || nr < 0 || nc < 0) return 1;
    gather_ctx *g = (gather_ctx *)malloc(sizeof(gather_ctx));
    if (!g) return 2;
    g->dt = dt;
    g->base = base;
    g->rs = row_stride;
    g->cs = col_stride;
    g->nc = nc;
    g->rows = rows;
    g->cols = cols;
    g->dst = dst;
    /* the table is the decode function evaluated at every pattern */
    for (int i = 0; i < 65536; ++i) g->lut[i] = zio_decode1(dt, (uint16_t)i);
    parallel_range(nr, gather_rows, g);
    free(g);
    return 0;
}

/* ------------------------------------------------------------------ */
/* C[r][c] = sum_{i<k} A[r][i] * B[c][i]                               */
/* ------------------------------------------------------------------ */

typedef struct {
    int64_t nr, nc, k;
    const double *A, *B;
    double *C;
} mm_ctx;

/* Each output element is its own ascending-order sum.  Four columns are
 * carried at once only so that four independent sums are in flight; the
 * order inside each sum is untouched. */
static void mm_rows(void *p, int64_t lo, int64_t hi) {
    mm_ctx *m = (mm_ctx *)p;
    const int64_t k = m->k;
    for (int64_t r = lo; r < hi; ++r) {
        const double *a = m->A + r * k;
        double *out = m->C + r * m->nc;
        int64_t c = 0;
        for (; c + 4 <= m->nc; c += 4) {
            const double *b0 = m->B + (c + 0) * k;
            const double *b1 = m->B + (c + 1) * k;
            const double *b2 = m->B + (c + 2) * k;
            const double *b3 = m->B + (c + 3) * k;
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                double x = a[i];
                s0 += x * b0[i];
                s1 += x * b1[i];
                s2 += x * b2[i];
                s3 += x * b3[i];
            }
            out[c + 0] = s0;
            out[c + 1] = s1;
            out[c + 2] = s2;
            out[c + 3] = s3;
        }
        for (; c < m->nc; ++c) {
            const double *b = m->B + c * k;
            double s = 0.0;
            for (int64_t i = 0; i < k; ++i) s += a[i] * b[i];
            out[c] = s;
        }
    }
}

static void mm_cols(void *p, int64_t lo, int64_t hi) {
    mm_ctx *m = (mm_ctx *)p;
    const int64_t k = m->k;
    for (int64_t r = 0; r < m->nr; ++r) {
        const double *a = m->A + r * k;
        for (int64_t c = lo; c < hi; ++c) {
            const double *b = m->B + c * k;
            double s = 0.0;
            for (int64_t i = 0; i < k; ++i) s += a[i] * b[i];
            m->C[r * m->nc + c] = s;
        }
    }
}

int zio_matmul_nt(int64_t nr, int64_t nc, int64_t k, const double *A, const double *B,
                  double *C) {
    if (nr < 0 || nc < 0 || k < 0 || !A || !B || !C) return 1;
    mm_ctx m = {nr, nc, k, A, B, C};
    /* split whichever output axis gives the threads more to do */
    if (nr >= zio_get_threads() || nr >= nc)
        parallel_range(nr, mm_rows, &m);
    else
        parallel_range(nc, mm_cols, &m);
    return 0;
}

/* ------------------------------------------------------------------ */
/* GeLU, exact (erf) form: gelu(a) = a * Phi(a), Phi the standard normal CDF,  */
/* Phi(a) = (1 + erf(a/sqrt 2))/2 = erfc(-a/sqrt 2)/2.  The erfc spelling is     */
/* used because it keeps full relative accuracy in the negative tail, where    */
/* 1 + erf(.) cancels.                                                          */
/* gelu'(a) = Phi(a) + a * phi(a),  phi(a) = exp(-a^2/2) / sqrt(2 pi)           */
/* ------------------------------------------------------------------ */

void zio_gelu(const double *a, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) {
        double x = a[i];
        out[i] = x * (0.5 * erfc(-x / sqrt(2.0)));
    }
}

void zio_gelu_grad(const double *a, int64_t n, double *out) {
    const double inv_sqrt_2pi = 1.0 / sqrt(2.0 * M_PI);
    for (int64_t i = 0; i < n; ++i) {
        double x = a[i];
        double cdf = 0.5 * erfc(-x / sqrt(2.0));
        double pdf = exp(-0.5 * x * x) * inv_sqrt_2pi;
        out[i] = cdf + x * pdf;
    }
}
