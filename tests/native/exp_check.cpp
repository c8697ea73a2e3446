// Host check of rtp::exp_tang (the selector's fp64 exp) against expl:
// prints the largest error in ulps of the exact result over a dense sweep of
// [-745, 0] and over edge points, and the table's largest error.
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rtp_exp.h"

static const double kTbl[rtp::kExpTable] = RTP_EXP2_TABLE;

// Error of `got` in units of the last place of the exact value `want`.
static long double ulps(double got, long double want)
{
    if (want == 0.0L) return got == 0.0 ? 0.0L : 1e30L;
    int e;
    frexpl(want, &e);
    long double ulp = ldexpl(1.0L, e - 53);
    const long double min_ulp = ldexpl(1.0L, -1074);  // subnormal spacing
    if (ulp < min_ulp) ulp = min_ulp;
    return fabsl((long double)got - want) / ulp;
}

int main()
{
    long double tmax = 0;
    for (int j = 0; j < rtp::kExpTable; ++j) {
        long double u = ulps(kTbl[j], exp2l((long double)j / (long double)rtp::kExpTable));
        if (u > tmax) tmax = u;
    }
    long double emax = 0, smax = 0;
    double worst = 0;
    uint64_t state = 0x9E3779B97F4A7C15ull;
    for (int i = 0; i < 4000000; ++i) {
        double x;
        if (i < 2000000) {
            x = -745.0 * (double)i / 2000000.0;
        } else {  // random points, including small magnitudes
            state = state * 6364136223846793005ull + 1442695040888963407ull;
            const double u = (double)(state >> 11) * 0x1p-53;
            x = (i & 1) ? -745.0 * u : -exp2(-60.0 * u);
        }
        const long double want = expl((long double)x);
        const long double e = ulps(rtp::exp_tang(x, kTbl), want);
        if (want >= (long double)DBL_MIN) {
            if (e > emax) { emax = e; worst = x; }
        } else if (e > smax) {
            smax = e;
        }
    }
    const double edges[] = {0.0, -0.0, -1e-300, -0x1p-1074, -1e-17, -0.5, -1.0, -708.0,
                            -708.39, -744.4, -745.1, -745.13, 1.0, 20.0, 709.0};
    for (double x : edges) {
        const long double e = ulps(rtp::exp_tang(x, kTbl), expl((long double)x));
        const long double want = expl((long double)x);
        if (want >= (long double)DBL_MIN) {
            if (e > emax) { emax = e; worst = x; }
        } else if (e > smax) {
            smax = e;
        }
    }
    const bool zero_ok = rtp::exp_tang(-746.0, kTbl) == 0.0 &&
                         rtp::exp_tang(-745.5, kTbl) == 0.0 &&
                         rtp::exp_tang(-1e300, kTbl) == 0.0 &&
                         rtp::exp_tang(-INFINITY, kTbl) == 0.0 &&
                         rtp::exp_tang(NAN, kTbl) == 0.0;
    printf("table_max_ulp %.6Lf\nnormal_max_ulp %.6Lf\nsubnormal_max_ulp %.6Lf\nworst_x %.17g\n"
           "specials_ok %d\n", tmax, emax, smax, worst, zero_ok ? 1 : 0);
    return 0;
}
