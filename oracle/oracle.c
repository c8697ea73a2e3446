/*
 * oracle.c -- plain, slow, single-threaded CPU definition of the RTPurbo
 * sparse decode attention path ("Full Attention Strikes Back: Transferring
 * Full Attention into Sparse within Hundred Training Steps", arXiv 2605.16928).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Compiled with -O2 -ffp-contract=off -fno-fast-math: every floating point
 * operation below is the IEEE operation written, in the order written.
 *
 * What each function follows (citations name the page and its section):
 *   orc_scores      -- 16-dim low-rank indexer score of every cached token,
 *                      taken before RoPE (gist.science summary, method
 *                      section 2 "low-dimensional token indexing"; the arXiv
 *                      abstract gives the indexer's width as 16).  The pages give
 *                      no formula; the score is the plain dot product
 *                      q_r . k_r in fp32, accumulated as one fused
 *                      multiply-add per dimension, dimensions 0..15 in order.
 *   orc_scores_bf16 -- orc_scores over bf16 indexer keys, each widened
 *                      exactly to fp32 first (a storage variant of the same
 *                      definition, halving the key bytes).
 *   orc_topp        -- dynamic top-p selection: accumulate low-dimensional
 *                      attention mass, largest first, until the cumulative
 *                      mass reaches p (gist.science summary, method
 *                      section 3 "dynamic top-p vs static top-k").  Mass is
 *                      the unit-temperature softmax of the scores over all N
 *                      cached tokens, in fp64; order is a full sort by score,
 *                      ties to the lower token index; the set is the shortest
 *                      prefix whose mass is >= p * Z.  p >= 1 keeps all.
 *   orc_topk        -- static top-k selection, the fixed budget that dynamic
 *                      top-p is set against (same section): the k highest
 *                      scores, in the same order as orc_topp (the pages give
 *                      no tie rule for either; ties go to the lower index).
 *                      k >= N keeps all.
 *   orc_project     -- the indexer's low-dim projection of pre-RoPE query or
 *                      key features (summary section 2: a 16-dim projector
 *                      before RoPE): out[t][j] = sum_c W[j][c] * x[t][c] for
 *                      bf16 W [r][d] and x [T][d], every product and the
 *                      sum in fp64, c = 0..d-1 in order (the pages fix no
 *                      precision; fp64 stands in for the exact sum).
 *   orc_attention   -- exact softmax attention of one query row over a given
 *                      set of cached rows, in fp64 (arXiv abstract: sparse
 *                      attention over the indexer's tokens; summary
 *                      section 5 "sparse decode").
 *   orc_local_rows  -- the rows a local head attends: attention sinks plus a
 *                      sliding window (summary section 1, head roles).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

/* bf16 bit pattern -> its exact value (bf16 is the top half of an fp32). */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Neumaier-compensated running sum. */
typedef struct { double sum, comp; } ksum;

static void ksum_add(ksum *k, double x)
{
    double t = k->sum + x;
    if (fabs(k->sum) >= fabs(x))
        k->comp += (k->sum - t) + x;
    else
        k->comp += (x - t) + k->sum;
    k->sum = t;
}

static double ksum_value(const ksum *k) { return k->sum + k->comp; }

/* -------------------------------------------------------------- O1 scores */

/* s[i] = q . k_r[i] for i in [0, N): fp32, one fmaf per dimension, j = 0..15
 * in order, starting from +0; a zero result is stored as +0.
 * q: [16]; k: [N][16] row-major. */
void orc_scores(const float *q, const float *k, int64_t N, float *s)
{
    for (int64_t i = 0; i < N; ++i) {
        const float *row = k + i * 16;
        float acc = 0.0f;
        for (int j = 0; j < 16; ++j)
            acc = fmaf(q[j], row[j], acc);
        if (acc == 0.0f)
            acc = 0.0f; /* -0 becomes +0 */
        s[i] = acc;
    }
}

/* The same scores from bf16 keys (bit patterns), widened to fp32. */
void orc_scores_bf16(const float *q, const uint16_t *k, int64_t N, float *s)
{
    for (int64_t i = 0; i < N; ++i) {
        const uint16_t *row = k + i * 16;
        float acc = 0.0f;
        for (int j = 0; j < 16; ++j)
            acc = fmaf(q[j], (float)bf16_value(row[j]), acc);
        if (acc == 0.0f)
            acc = 0.0f; /* -0 becomes +0 */
        s[i] = acc;
    }
}

/* --------------------------------------------------------- O2-O4 top-p set */

typedef struct {
    int64_t k;          /* size of the selected set                       */
    float tau;          /* score of the last selected token (threshold)   */
    double max_score;   /* M                                              */
    double Z;           /* sum of exp(s_i - M) over all N tokens          */
    double mass;        /* mass of the selected set / Z                   */
    double last_mass;   /* mass of the last selected token / Z            */
    double slack;       /* mass of the set without its last token / Z     */
} orc_topp_report;

typedef struct { float s; int64_t i; } scored;

/* Full order: larger score first; equal scores, lower index first. */
static int by_score_desc(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    if (a->i < b->i) return -1;
    if (a->i > b->i) return 1;
    return 0;
}

/* Selects the top-p set of one head.  sel must hold N entries; it receives
 * the selected token indices in selection order (largest score first).
 * Returns the set size, or -1 if memory runs out. */
int64_t orc_topp(const float *s, int64_t N, float p, int64_t *sel,
                 orc_topp_report *rep)
{
    orc_topp_report r;
    memset(&r, 0, sizeof r);

    /* O2: M, e_i = exp(s_i - M), Z by compensated sum in index order. */
    double M = -INFINITY;
    for (int64_t i = 0; i < N; ++i)
        if ((double)s[i] > M) M = (double)s[i];
    ksum zs = {0.0, 0.0};
    for (int64_t i = 0; i < N; ++i)
        ksum_add(&zs, exp((double)s[i] - M));
    double Z = ksum_value(&zs);
    r.max_score = M;
    r.Z = Z;

    /* O3: full sort, descending score, ties by ascending index. */
    scored *order = (scored *)malloc((size_t)N * sizeof *order);
    if (!order) return -1;
    for (int64_t i = 0; i < N; ++i) {
        order[i].s = s[i];
        order[i].i = i;
    }
    qsort(order, (size_t)N, sizeof *order, by_score_desc);

    /* O4: shortest prefix with cumulative mass >= p * Z (p >= 1: all). */
    int64_t k;
    ksum ps = {0.0, 0.0};
    double before_last = 0.0, last = 0.0;
    if ((double)p >= 1.0) {
        for (int64_t t = 0; t < N; ++t) {
            before_last = ksum_value(&ps);
            last = exp((double)order[t].s - M);
            ksum_add(&ps, last);
        }
        k = N;
    } else {
        double target = (double)p * Z;
        k = N;
        for (int64_t t = 0; t < N; ++t) {
            before_last = ksum_value(&ps);
            last = exp((double)order[t].s - M);
            ksum_add(&ps, last);
            if (ksum_value(&ps) >= target) {
                k = t + 1;
                break;
            }
        }
    }
    for (int64_t t = 0; t < k; ++t)
        sel[t] = order[t].i;
    r.k = k;
    r.tau = order[k - 1].s;
    r.mass = ksum_value(&ps) / Z;
    r.last_mass = last / Z;
    r.slack = before_last / Z;
    free(order);
    if (rep) *rep = r;
    return k;
}

/* Selects the top-k set of one head: the first min(k, N) tokens of the full
 * order used by orc_topp.  sel must hold N entries; it receives them in that
 * order.  Returns the set size (0 for k <= 0), or -1 if memory runs out. */
int64_t orc_topk(const float *s, int64_t N, int64_t k, int64_t *sel)
{
    scored *order = (scored *)malloc((size_t)(N > 0 ? N : 1) * sizeof *order);
    if (!order) return -1;
    for (int64_t i = 0; i < N; ++i) {
        order[i].s = s[i];
        order[i].i = i;
    }
    qsort(order, (size_t)N, sizeof *order, by_score_desc);
    const int64_t n = k < 0 ? 0 : (k < N ? k : N);
    for (int64_t t = 0; t < n; ++t)
        sel[t] = order[t].i;
    free(order);
    return n;
}

/* out[t][j] = sum_c W[j][c] * x[t][c] in fp64, for t < T, j < r. */
void orc_project(const uint16_t *x, int64_t T, int64_t d, const uint16_t *W, int64_t r,
                 double *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c)
                acc += bf16_value(W[j * d + c]) * bf16_value(x[t * d + c]);
            out[t * r + j] = acc;
        }
}

/* Mass of an arbitrary set of tokens, as a fraction of Z (O2 definitions).
 * Used to judge a set produced elsewhere. */
double orc_set_mass(const float *s, int64_t N, const int64_t *set, int64_t n)
{
    double M = -INFINITY;
    for (int64_t i = 0; i < N; ++i)
        if ((double)s[i] > M) M = (double)s[i];
    ksum zs = {0.0, 0.0}, ms = {0.0, 0.0};
    for (int64_t i = 0; i < N; ++i)
        ksum_add(&zs, exp((double)s[i] - M));
    for (int64_t t = 0; t < n; ++t)
        ksum_add(&ms, exp((double)s[set[t]] - M));
    return ksum_value(&ms) / ksum_value(&zs);
}

/* --------------------------------------------------- O5 exact attention */

/* out[c] = sum_{i in rows} w_i V[i][c], w = softmax over rows of
 * scale * (q . K[i]), all in fp64 from the exact bf16 values.
 * q: [d] bf16; K, V: row-major [*][d] bf16 (row i at K + i*d).
 * rows: n row indices (n >= 1). */
void orc_attention(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                   int64_t d, const int64_t *rows, int64_t n, float scale,
                   double *out)
{
    double *logit = (double *)malloc((size_t)n * sizeof *logit);
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *krow = K + rows[t] * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += bf16_value(q[c]) * bf16_value(krow[c]);
        logit[t] = (double)scale * dot;
        if (logit[t] > mx) mx = logit[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        logit[t] = exp(logit[t] - mx);
        den += logit[t];
    }
    for (int64_t c = 0; c < d; ++c)
        out[c] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *vrow = V + rows[t] * d;
        double w = logit[t] / den;
        for (int64_t c = 0; c < d; ++c)
            out[c] += w * bf16_value(vrow[c]);
    }
    free(logit);
}

/* ------------------------------------------------------ O6 local rows */

/* Rows attended by a local head when the cache holds N tokens and the query
 * is the newest one: the first n_sink rows plus the newest `window` rows,
 * each row once.  rows must hold min(N, n_sink + window) entries; returns
 * the count, ascending. */
int64_t orc_local_rows(int64_t N, int64_t n_sink, int64_t window,
                       int64_t *rows)
{
    int64_t w_start = N - window;
    if (w_start < 0) w_start = 0;
    int64_t n = 0;
    for (int64_t i = 0; i < N; ++i)
        if (i < n_sink || i >= w_start)
            rows[n++] = i;
    return n;
}
