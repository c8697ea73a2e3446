// fp64 exponential for the selector's mass terms exp(s - ref).  The top-p
// boundary is decided on fp64 masses, and the library exp costs several
// times the fp64 instructions of this one, which made it the bound of the
// histogram pass.
//
// Method: Tang's table-driven exponential (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989).  x = (64 m + j) ln2/64 + r with
// |r| <= ln2/128; exp(x) = 2^m * 2^(j/64) * exp(r), where exp(r) is its
// Taylor polynomial of degree 5 (truncation error below 4e-17 relative).
// ln2/64 is split in two so that n * hi is exact for every |n| < 2^17.
// Measured error against expl: below 1.3 ulp over [-745, 0] (host test).
//
// Plain C++ so that the host can test it; the kernels pass a copy of the
// table in LDS.
#pragma once

#include <math.h>

#ifdef __HIPCC__
#define RTP_HD __host__ __device__
#else
#define RTP_HD
#endif

namespace rtp {

// 2^(j/64) for j = 0..63, each rounded to the nearest double.
#define RTP_EXP2_TABLE                                                                   \
    {                                                                                    \
        0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0, \
        0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0, \
        0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0, \
        0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0, \
        0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0, \
        0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0, \
        0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0, \
        0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0, \
        0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0, \
        0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0, \
        0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0, \
        0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0, \
        0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0, \
        0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0, \
        0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0, \
        0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0, \
    }

constexpr int kExpTable = 64;
constexpr double kExpInvStep = 0x1.71547652b82fep+6;  // 64 / ln 2
constexpr double kExpStepHi = 0x1.62e42fefa0000p-7;   // ln2/64 to 36 significant bits
constexpr double kExpStepLo = 0x1.cf79abc9e3b3ap-46;  // ln2/64 - kExpStepHi

// exp(x) for x <= 709; `tbl` holds RTP_EXP2_TABLE.  The reduction runs on
// max(x, -745.5), whose exp rounds to +0, so the result is +0 for every x
// below that, for x = -inf, and for NaN (max returns the other operand): a
// mass term of a NaN score is 0.  No branch and no select, so the callers'
// loops stay free of divergence.
RTP_HD inline double exp_tang(double x, const double *tbl)
{
    x = fmax(x, -745.5);
    const double n = rint(x * kExpInvStep);
    double r = fma(-n, kExpStepHi, x);
    r = fma(-n, kExpStepLo, r);
    const int ni = (int)n;
    // exp(r) - 1, then t * exp(r) as t + t * (exp(r) - 1) in one rounding.
    double pm = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    pm = fma(r, pm, 1.0 / 6.0);
    pm = fma(r, pm, 0.5);
    pm = fma(r, pm, 1.0);
    pm *= r;
    const double t = tbl[ni & (kExpTable - 1)];
    return ldexp(fma(t, pm, t), ni >> 6);
}

}  // namespace rtp
