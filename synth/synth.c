/*
 * synth.c -- seeded, counter-based, random-access input generator.
 *
 * Serves both the GPU path (its inputs are generated here on the host and
 * uploaded) and the CPU oracle (which regenerates only the rows it reads).
 * It holds none of the attention method's arithmetic: only pseudo-random
 * numbers and the fixed maps that turn them into N(0,1) samples.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Value c of a stream with key k is
 * mix64(k + (c + 1) * GAMMA), so any element can be produced on its own.
 *
 *   uniform(k, c)  = ((mix64(...) >> 11) + 0.5) * 2^-53         in (0, 1)
 *   normal_f32     = fp32(sqrt(-2 ln u1) * cos(2 pi u2)),         Box-Muller,
 *                    u1 = uniform(k, 2i), u2 = uniform(k, 2i + 1)
 *   normal_bf16    = Q[j], j = 16-bit field (i mod 4) of mix64 at counter i/4,
 *                    Q[j] = bf16(inverse normal CDF at (j + 0.5) / 65536):
 *                    N(0,1) over 65536 equiprobable cells, rounded to bf16.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t c)
{
    return mix64(key + (c + 1) * GAMMA);
}

static inline double uniform(uint64_t key, uint64_t c)
{
    return ((double)(draw(key, c) >> 11) + 0.5) * 0x1.0p-53;
}

/* Key of one stream: (seed, stream id, layer, batch row, head). */
uint64_t synth_key(uint64_t seed, uint32_t stream, uint32_t layer, uint32_t b,
                   uint32_t head)
{
    uint64_t k = mix64(seed * GAMMA + 0x5EEDULL);
    k = mix64(k ^ ((uint64_t)stream << 48));
    k = mix64(k ^ ((uint64_t)layer << 32));
    k = mix64(k ^ (((uint64_t)b << 20) | (uint64_t)head));
    return k;
}

double synth_uniform(uint64_t key, uint64_t c) { return uniform(key, c); }

/* ---------------------------------------------------------------- fp32 */

static float normal_f32(uint64_t key, uint64_t i)
{
    double u1 = uniform(key, 2 * i), u2 = uniform(key, 2 * i + 1);
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

/* ---------------------------------------------------------------- bf16 */

static uint16_t table_q[65536];
static pthread_once_t table_once = PTHREAD_ONCE_INIT;

static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u); /* round to nearest even */
    return (uint16_t)(u >> 16);
}

static double norm_cdf(double x) { return 0.5 * erfc(-x * 0.7071067811865476); }

static void build_table(void)
{
    /* Upper half by bisection on the CDF; lower half by symmetry. */
    for (int j = 32768; j < 65536; ++j) {
        double u = ((double)j + 0.5) / 65536.0;
        double lo = 0.0, hi = 9.0;
        for (int it = 0; it < 64; ++it) {
            double mid = 0.5 * (lo + hi);
            if (norm_cdf(mid) < u) lo = mid; else hi = mid;
        }
        double x = 0.5 * (lo + hi);
        uint16_t pos = f32_to_bf16((float)x);
        table_q[j] = pos;
        table_q[65535 - j] = (uint16_t)(pos ^ 0x8000u);
    }
}

const uint16_t *synth_bf16_table(void)
{
    pthread_once(&table_once, build_table);
    return table_q;
}

static inline uint16_t normal_bf16(uint64_t key, uint64_t i)
{
    uint64_t w = draw(key, i >> 2);
    return table_q[(w >> (16 * (i & 3))) & 0xFFFFu];
}

/* ------------------------------------------------------------ threaded */

typedef struct {
    uint64_t key;
    int64_t start, count;
    void *out;
    int kind; /* 0 f32 normal, 1 bf16 normal */
} job;

static void *run_job(void *arg)
{
    job *jb = (job *)arg;
    if (jb->kind == 0) {
        float *o = (float *)jb->out;
        for (int64_t t = 0; t < jb->count; ++t)
            o[t] = normal_f32(jb->key, (uint64_t)(jb->start + t));
    } else {
        uint16_t *o = (uint16_t *)jb->out;
        for (int64_t t = 0; t < jb->count; ++t)
            o[t] = normal_bf16(jb->key, (uint64_t)(jb->start + t));
    }
    return NULL;
}

static void run_parallel(uint64_t key, int64_t start, int64_t count, void *out,
                         int kind, int nthreads)
{
    enum { MAXT = 64 };
    size_t esize = kind == 0 ? 4 : 2;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > MAXT) nthreads = MAXT;
    if (count < 65536) nthreads = 1;
    job jobs[MAXT];
    pthread_t th[MAXT];
    int64_t per = (count + nthreads - 1) / nthreads;
    per = (per + 3) & ~(int64_t)3;
    int used = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t s = (int64_t)t * per;
        if (s >= count) break;
        int64_t c = count - s < per ? count - s : per;
        jobs[t].key = key;
        jobs[t].start = start + s;
        jobs[t].count = c;
        jobs[t].out = (char *)out + (size_t)s * esize;
        jobs[t].kind = kind;
        used = t + 1;
    }
    if (used == 1) {
        run_job(&jobs[0]);
        return;
    }
    for (int t = 0; t < used; ++t)
        pthread_create(&th[t], NULL, run_job, &jobs[t]);
    for (int t = 0; t < used; ++t)
        pthread_join(th[t], NULL);
}

/* Elements [start, start + count) of an fp32 N(0,1) stream. */
void synth_normal_f32(uint64_t key, int64_t start, int64_t count, float *out,
                      int nthreads)
{
    run_parallel(key, start, count, out, 0, nthreads);
}

/* Elements [start, start + count) of a bf16 N(0,1) stream (bit patterns). */
void synth_normal_bf16(uint64_t key, int64_t start, int64_t count,
                       uint16_t *out, int nthreads)
{
    synth_bf16_table();
    run_parallel(key, start, count, out, 1, nthreads);
}

/* Rows rows[0..n) of a bf16 stream laid out as [*][row_len]. */
void synth_bf16_rows(uint64_t key, const int64_t *rows, int64_t n,
                     int64_t row_len, uint16_t *out)
{
    synth_bf16_table();
    for (int64_t t = 0; t < n; ++t)
        for (int64_t c = 0; c < row_len; ++c)
            out[t * row_len + c] =
                normal_bf16(key, (uint64_t)(rows[t] * row_len + c));
}

/* Rows rows[0..n) of an fp32 stream laid out as [*][row_len]. */
void synth_f32_rows(uint64_t key, const int64_t *rows, int64_t n,
                    int64_t row_len, float *out)
{
    for (int64_t t = 0; t < n; ++t)
        for (int64_t c = 0; c < row_len; ++c)
            out[t * row_len + c] =
                normal_f32(key, (uint64_t)(rows[t] * row_len + c));
}
