/*
 * oracle.c -- plain, slow, FP64 CPU oracle for the LM-head path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the HIP path.
 *
 * Sources (cited by page title and section):
 *  [MIXED]  Megatron-LM pull request "Add mixed-precision (FP32) LM output
 *           logits" -- section "What does this PR do?" (the logits are the
 *           GEMM's FP32 accumulator, BF16 operands; the legacy path rounds
 *           each logit to BF16), section "Tests" (integer operands in
 *           [-8, 8], K * 8^2 < 2^24 makes every FP32 partial sum exact) and
 *           section "Method" (16 x K activations, 32,768 x K vocabulary
 *           weights, seed 1234).
 *  [XENT]   Transformer Engine issue "[Pytorch] change fused cross entropy
 *           backward grad to fp32 and reduce one read/..." -- section
 *           "Description" and "Changes" (backward gradient in FP32) and the
 *           discussion (the forward keeps the input, the n_rows x 1 target
 *           and the n_rows x 4 m_d_X_y statistics for the backward).
 *
 * Every routine is the plain definition written out in double precision:
 *   GEMM   C[i][j] = sum_p A(i,p) * B(j,p), summed in increasing p.
 *   CE fwd m = max_j z_j, d = sum_j exp(z_j - m), X = z_y,
 *          loss = (m - X) + log d; ignored rows give X = 0, loss = 0.
 *   CE bwd g_j = dloss * (exp(z_j - m) / d - [j == y]); ignored rows are 0.
 *   mean   n_valid = #{y != ignore}, mean = sum loss / n_valid,
 *          inv = 1 / n_valid (both 0 when n_valid == 0).
 *   split  per column block b of a row: m_b = max z_j, d_b = sum exp(z_j - m_b)
 *          over the block, X_b = z_y and own_b = 1 when the (global) target
 *          column lies in the block, else X_b = own_b = 0; merged over the
 *          blocks of a row: m = max m_b, d = sum d_b exp(m_b - m), X from the
 *          one owning block, loss = (m - X) + log d.  This is the per-shard
 *          form of the statistics of vocabulary-parallel cross entropy
 *          ([XENT] "Description" names Megatron's vocabulary-parallel CE as
 *          the FP32 reference): exp(z_j - m) = exp(z_j - m_b) exp(m_b - m).
 * The softmax-minus-one-hot form of the backward is the derivative of the
 * forward loss; the tests pin it by finite differences of the forward.
 *
 * Rows are split over POSIX threads; each output is computed by exactly one
 * thread in the fixed order above, so the thread count never changes a bit
 * of the result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---------------------------------------------------------------- helpers */

/* BF16 is the top half of an IEEE binary32 word; widening is exact. */
static double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int orc_default_threads(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

typedef void (*orc_row_fn)(void *ctx, int64_t r0, int64_t r1);

typedef struct {
    orc_row_fn fn;
    void *ctx;
    int64_t r0, r1;
} orc_span;

static void *orc_span_main(void *p)
{
    orc_span *s = (orc_span *)p;
    s->fn(s->ctx, s->r0, s->r1);
    return NULL;
}

/* Run fn over rows [0, n) split into nthreads contiguous spans. */
static void orc_parallel_rows(orc_row_fn fn, void *ctx, int64_t n, int nthreads)
{
    if (nthreads <= 0)
        nthreads = orc_default_threads();
    if (nthreads > n)
        nthreads = (int)(n > 0 ? n : 1);
    if (nthreads <= 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    orc_span *sp = (orc_span *)malloc(sizeof(orc_span) * (size_t)nthreads);
    char *live = (char *)calloc((size_t)nthreads, 1);
    for (int t = 0; t < nthreads; ++t) {
        sp[t].fn = fn;
        sp[t].ctx = ctx;
        sp[t].r0 = n * t / nthreads;
        sp[t].r1 = n * (t + 1) / nthreads;
        if (pthread_create(&th[t], NULL, orc_span_main, &sp[t]) == 0)
            live[t] = 1;
        else
            orc_span_main(&sp[t]); /* run inline if a thread cannot start */
    }
    for (int t = 0; t < nthreads; ++t)
        if (live[t])
            pthread_join(th[t], NULL);
    free(live);
    free(th);
    free(sp);
}

/* ------------------------------------------------------------------ GEMM */

/*
 * C[r][j] = sum_{p=0}^{np-1} A(i_r, p) * B(j, p)        (FP64)
 * S[r][j] = sum_{p=0}^{np-1} |A(i_r, p) * B(j, p)|      (FP64, may be NULL)
 * with A(i, p) = a[i * a_si + p * a_sp] and B(j, p) = b[j * b_sj + p * b_sp],
 * both BF16 bit patterns.  i_r = rows[r] if rows is given, else r.
 *
 * The logits GEMM of [MIXED] is A = activations x[M x K] (a_si = ldx,
 * a_sp = 1), B = vocabulary weights W[V x K] (b_sj = ldw, b_sp = 1).  The
 * input-gradient and weight-gradient GEMMs use the same definition with
 * other strides.  Each C[r][j] is accumulated in increasing p; when B is
 * contiguous in j the loops over p and j are nested the other way round
 * (one running sum per j, still in increasing p), which gives the same
 * bits and keeps the memory walk sequential.
 */
typedef struct {
    const uint16_t *a, *b;
    int64_t a_si, a_sp, b_sj, b_sp, nj, np;
    const int64_t *rows;
    double *c, *s;
} orc_gemm_ctx;

static void orc_gemm_rows(void *vctx, int64_t r0, int64_t r1)
{
    orc_gemm_ctx *g = (orc_gemm_ctx *)vctx;
    for (int64_t r = r0; r < r1; ++r) {
        int64_t i = g->rows ? g->rows[r] : r;
        double *crow = g->c + r * g->nj;
        double *srow = g->s ? g->s + r * g->nj : NULL;
        if (g->b_sp == 1 || g->b_sj != 1) {
            /* dot-product order: for each j, walk p */
            for (int64_t j = 0; j < g->nj; ++j) {
                double acc = 0.0, sabs = 0.0;
                for (int64_t p = 0; p < g->np; ++p) {
                    double prod = orc_bf16_to_double(g->a[i * g->a_si + p * g->a_sp]) *
                                  orc_bf16_to_double(g->b[j * g->b_sj + p * g->b_sp]);
                    acc += prod;
                    sabs += fabs(prod);
                }
                crow[j] = acc;
                if (srow)
                    srow[j] = sabs;
            }
        } else {
            /* B contiguous in j: one running sum per j, p outermost */
            for (int64_t j = 0; j < g->nj; ++j) {
                crow[j] = 0.0;
                if (srow)
                    srow[j] = 0.0;
            }
            for (int64_t p = 0; p < g->np; ++p) {
                double av = orc_bf16_to_double(g->a[i * g->a_si + p * g->a_sp]);
                const uint16_t *bp = g->b + p * g->b_sp;
                for (int64_t j = 0; j < g->nj; ++j) {
                    double prod = av * orc_bf16_to_double(bp[j]);
                    crow[j] += prod;
                    if (srow)
                        srow[j] += fabs(prod);
                }
            }
        }
    }
}

int orc_gemm_bf16(const uint16_t *a, int64_t a_si, int64_t a_sp,
                  const uint16_t *b, int64_t b_sj, int64_t b_sp,
                  int64_t n_out_rows, const int64_t *rows, int64_t nj, int64_t np,
                  double *c, double *s, int nthreads)
{
    if (n_out_rows < 0 || nj < 0 || np < 0)
        return -1;
    if ((n_out_rows > 0 && nj > 0) && (!c || (np > 0 && (!a || !b))))
        return -2;
    orc_gemm_ctx g = {a, b, a_si, a_sp, b_sj, b_sp, nj, np, rows, c, s};
    orc_parallel_rows(orc_gemm_rows, &g, n_out_rows, nthreads);
    return 0;
}

/* --------------------------------------------------------- cross entropy */

/* Row statistics of [XENT]'s saved m_d_X_y record, in FP64.
 * Returns 0, or -1 when the target is neither ignore_index nor in [0, V). */
static int orc_row_stats(const float *z, int64_t V, int32_t y, int32_t ignore_index,
                         double *m_out, double *d_out, double *x_out, double *loss_out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j)
        if ((double)z[j] > m)
            m = (double)z[j];
    /* A row whose logits are all -inf has no softmax: d is the empty sum 0
     * (not exp(-inf + inf) = NaN), and the loss below is NaN. */
    double d = 0.0;
    if (m != -INFINITY)
        for (int64_t j = 0; j < V; ++j)
            d += exp((double)z[j] - m);
    *m_out = m;
    *d_out = d;
    if (y == ignore_index) {
        *x_out = 0.0;
        *loss_out = 0.0;
        return 0;
    }
    if (y < 0 || (int64_t)y >= V)
        return -1;
    double x = (double)z[y];
    *x_out = x;
    *loss_out = (m - x) + log(d);
    return 0;
}

typedef struct {
    const float *z;
    int64_t ld, V;
    const int32_t *tgt;
    int32_t ignore_index;
    const int64_t *rows;
    double *stats;
    const double *dloss;
    int64_t dloss_stride;
    double *g;
    int bad; /* set (atomically) when a target is out of range */
} orc_xent_ctx;

static void orc_xent_fwd_rows(void *vctx, int64_t r0, int64_t r1)
{
    orc_xent_ctx *c = (orc_xent_ctx *)vctx;
    for (int64_t r = r0; r < r1; ++r) {
        int64_t i = c->rows ? c->rows[r] : r;
        double *st = c->stats + 4 * r;
        if (orc_row_stats(c->z + i * c->ld, c->V, c->tgt[i], c->ignore_index,
                          &st[0], &st[1], &st[2], &st[3]) != 0)
            __atomic_store_n(&c->bad, 1, __ATOMIC_RELAXED);
    }
}

/* stats[r] = {m, d, X_y, loss} for row i_r (FP64), per [XENT]'s n_rows x 4
 * record whose fourth column is the row loss. */
int orc_xent_fwd(const float *z, int64_t ld, int64_t V, const int32_t *tgt,
                 int32_t ignore_index, int64_t n_out_rows, const int64_t *rows,
                 double *stats, int nthreads)
{
    if (n_out_rows < 0 || V < 1 || ld < V)
        return -1;
    orc_xent_ctx c;
    memset(&c, 0, sizeof c);
    c.z = z, c.ld = ld, c.V = V, c.tgt = tgt, c.ignore_index = ignore_index;
    c.rows = rows, c.stats = stats;
    orc_parallel_rows(orc_xent_fwd_rows, &c, n_out_rows, nthreads);
    return c.bad ? -3 : 0;
}

static void orc_xent_bwd_rows(void *vctx, int64_t r0, int64_t r1)
{
    orc_xent_ctx *c = (orc_xent_ctx *)vctx;
    for (int64_t r = r0; r < r1; ++r) {
        int64_t i = c->rows ? c->rows[r] : r;
        const float *z = c->z + i * c->ld;
        double *g = c->g + r * c->V;
        int32_t y = c->tgt[i];
        if (y == c->ignore_index) {
            for (int64_t j = 0; j < c->V; ++j)
                g[j] = 0.0;
            continue;
        }
        double m, d, x, loss;
        if (orc_row_stats(z, c->V, y, c->ignore_index, &m, &d, &x, &loss) != 0) {
            __atomic_store_n(&c->bad, 1, __ATOMIC_RELAXED);
            continue;
        }
        double up = c->dloss[c->dloss_stride * i];
        for (int64_t j = 0; j < c->V; ++j) {
            double p = exp((double)z[j] - m) / d;
            g[j] = up * (p - (j == (int64_t)y ? 1.0 : 0.0));
        }
    }
}

/* g[r][j] = dloss_i * (softmax(z_i)_j - [j == y_i]) in FP64, recomputing the
 * row statistics from the logits; dloss_i = dloss[dloss_stride * i]. */
int orc_xent_bwd(const float *z, int64_t ld, int64_t V, const int32_t *tgt,
                 int32_t ignore_index, const double *dloss, int64_t dloss_stride,
                 int64_t n_out_rows, const int64_t *rows, double *g, int nthreads)
{
    if (n_out_rows < 0 || V < 1 || ld < V || (dloss_stride != 0 && dloss_stride != 1))
        return -1;
    orc_xent_ctx c;
    memset(&c, 0, sizeof c);
    c.z = z, c.ld = ld, c.V = V, c.tgt = tgt, c.ignore_index = ignore_index;
    c.rows = rows, c.dloss = dloss, c.dloss_stride = dloss_stride, c.g = g;
    orc_parallel_rows(orc_xent_bwd_rows, &c, n_out_rows, nthreads);
    return c.bad ? -3 : 0;
}

/* ------------------------------------------ split-vocabulary cross entropy */

typedef struct {
    const float *z;
    int64_t ld, ncols, col0, bc, nb;
    const int32_t *tgt;
    int32_t ignore_index;
    const int64_t *rows;
    int64_t n_out;
    double *part;
} orc_part_ctx;

static void orc_xent_partial_rows(void *vctx, int64_t r0, int64_t r1)
{
    orc_part_ctx *c = (orc_part_ctx *)vctx;
    for (int64_t r = r0; r < r1; ++r) {
        int64_t i = c->rows ? c->rows[r] : r;
        const float *z = c->z + i * c->ld;
        int32_t y = c->tgt[i];
        for (int64_t b = 0; b < c->nb; ++b) {
            int64_t j0 = b * c->bc;
            int64_t j1 = j0 + c->bc < c->ncols ? j0 + c->bc : c->ncols;
            double m = -INFINITY;
            for (int64_t j = j0; j < j1; ++j)
                if ((double)z[j] > m)
                    m = (double)z[j];
            /* A block whose logits are all -inf (masked columns) holds no
             * probability mass: its pair is the empty one, m = -inf, d = 0. */
            double d = 0.0;
            if (m != -INFINITY)
                for (int64_t j = j0; j < j1; ++j)
                    d += exp((double)z[j] - m);
            double x = 0.0, own = 0.0;
            if (y != c->ignore_index) {
                int64_t loc = (int64_t)y - c->col0; /* column within the slice */
                if (loc >= j0 && loc < j1) {
                    x = (double)z[loc];
                    own = 1.0;
                }
            }
            double *pp = c->part + 4 * (b * c->n_out + r);
            pp[0] = m, pp[1] = d, pp[2] = x, pp[3] = own;
        }
    }
}

/* Partial statistics of a slice of a logits row holding the global columns
 * [col0, col0 + ncols), split into blocks of bc columns (the last one
 * shorter): part[b][r] = {m_b, d_b, X_b, own_b} for row i_r (FP64). */
int orc_xent_partial(const float *z, int64_t ld, int64_t ncols, int64_t col0, int64_t bc,
                     const int32_t *tgt, int32_t ignore_index, int64_t n_out_rows,
                     const int64_t *rows, double *part, int nthreads)
{
    if (n_out_rows < 0 || ncols < 1 || ld < ncols || bc < 1 || col0 < 0)
        return -1;
    orc_part_ctx c;
    memset(&c, 0, sizeof c);
    c.z = z, c.ld = ld, c.ncols = ncols, c.col0 = col0, c.bc = bc;
    c.nb = (ncols + bc - 1) / bc;
    c.tgt = tgt, c.ignore_index = ignore_index, c.rows = rows, c.n_out = n_out_rows;
    c.part = part;
    orc_parallel_rows(orc_xent_partial_rows, &c, n_out_rows, nthreads);
    return 0;
}

/* Merge n_parts partial records per row (part + p * part_stride + 4 r) into
 * stats[r] = {m, d, X_y, loss}.  Ignored rows: X = loss = 0.  A target
 * outside [0, vocab), or one not owned by exactly one part, gives X = loss =
 * NaN (m and d are still the merged values). */
void orc_xent_merge(const double *part, int64_t n_parts, int64_t part_stride, int64_t n_rows,
                    const int32_t *tgt, int32_t ignore_index, int64_t vocab, double *stats)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        double m = -INFINITY;
        for (int64_t p = 0; p < n_parts; ++p)
            if (part[p * part_stride + 4 * r] > m)
                m = part[p * part_stride + 4 * r];
        double d = 0.0, x = 0.0;
        int64_t owners = 0;
        for (int64_t p = 0; p < n_parts; ++p) {
            const double *pp = part + p * part_stride + 4 * r;
            if (pp[0] != -INFINITY) /* an empty block adds nothing to d */
                d += pp[1] * exp(pp[0] - m);
            if (pp[3] != 0.0) {
                x = pp[2];
                ++owners;
            }
        }
        double *st = stats + 4 * r;
        st[0] = m;
        st[1] = d;
        int32_t y = tgt[r];
        if (y == ignore_index) {
            st[2] = 0.0;
            st[3] = 0.0;
        } else if (y < 0 || (int64_t)y >= vocab || owners != 1) {
            st[2] = NAN;
            st[3] = NAN;
        } else {
            st[2] = x;
            st[3] = (m - x) + log(d);
        }
    }
}

/* out = {mean over non-ignored rows, 1 / n_valid, n_valid}; zeros if none. */
int orc_xent_mean(const double *loss, const int32_t *tgt, int32_t ignore_index,
                  int64_t n, double *out)
{
    double sum = 0.0;
    int64_t nv = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (tgt[i] == ignore_index)
            continue;
        sum += loss[i];
        ++nv;
    }
    out[0] = nv ? sum / (double)nv : 0.0;
    out[1] = nv ? 1.0 / (double)nv : 0.0;
    out[2] = (double)nv;
    return 0;
}

/* ------------------------------------------------------ BF16 rounding */

/*
 * Round a double to the nearest BF16 value, ties to even, and return its bit
 * pattern.  BF16 keeps 8 significant bits and binary32's exponent range, so
 * the spacing of representable values near |v| in [2^(e-1), 2^e) is
 * 2^(e-8), never finer than the smallest subnormal spacing 2^-133.  Values
 * that round past the largest finite BF16 become infinity; NaN becomes the
 * quiet NaN 0x7FC0 with the input's sign.
 */
uint16_t orc_round_bf16(double v)
{
    uint32_t u;
    float f;
    if (isnan(v)) {
        return signbit(v) ? (uint16_t)0xFFC0 : (uint16_t)0x7FC0;
    }
    if (isinf(v) || v == 0.0) {
        f = (float)v; /* exact */
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    int e;
    (void)frexp(v, &e); /* |v| = f * 2^e, f in [0.5, 1) */
    int q = e - 8;
    if (q < -133)
        q = -133;
    double scaled = ldexp(v, -q);          /* exact */
    double r = ldexp(nearbyint(scaled), q); /* ties-to-even under default mode */
    if (fabs(r) >= ldexp(1.0, 128))
        r = r > 0 ? INFINITY : -INFINITY;
    f = (float)r; /* exact: r has at most 8 significant bits */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void orc_round_bf16_array(const double *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_round_bf16(in[i]);
}
