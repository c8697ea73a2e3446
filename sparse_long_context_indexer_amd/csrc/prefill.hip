// Prefill attention (gist.science summary, method section 1: retrieval heads
// keep full attention, local heads a sliding window with attention sinks;
// the arXiv abstract credits the prefill speed-up at 1M context to this
// split).  Query token t of a head attends the keys its role allows:
//
//   dense (window <= 0)   keys [0, t]
//   local (window >= 1)   keys [0, min(n_sink, w0)) and [w0, t],
//                         w0 = max(0, t + 1 - window)
//
// with softmax(scale * q . k) over those keys, fp32 softmax and output.
//
// Matrix cores (fp32 accumulate), flash-style.  A block takes 32 query
// positions and up to 8 query heads of one KV head, one wave per head, and
// walks the allowed keys in tiles of 64.  Each tile's K rows and V^T (V
// transposed: one row per dimension, converted to fp16) are staged once in
// LDS for all the block's heads: waves 0-3 stage K, waves 4-7 V.  Per wave
// and tile:
//
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, 2 key halves x 8 dim steps:
//                 A = 8 dims of one key row (one 16-B LDS read), B = Q^T (the
//                 wave's 32 queries, held in registers).  Lane l then holds
//                 query l%32 and keys 8i + 4(l/32) + j of each half (i, j < 4).
//   O^T += V^T P^T  v_mfma_f32_32x32x16_f16, 4 dim tiles x 4 key steps of 16.
//                 The 16 keys of a step enter in the order the lanes already
//                 hold them: a lane of half g supplies keys 4g + (0..3) and
//                 8 + 4g + (0..3), as B = its own probabilities and as A =
//                 one 16-B read of V^T, whose key blocks are stored in that
//                 order.
//
// The two products of an iteration belong to different tiles: S^T of tile
// it + 1 is issued in the same basic block as the exponentials of tile it,
// and O^T += V^T P^T of tile it beside the fp16 rounding of its P, so each
// wave's matrix-core work overlaps its own vector work.  K is staged one
// tile ahead of V (two buffers each).
//
// O^T's columns are queries, so each lane's accumulators belong to its own
// query: the online-softmax rescale needs no exchange, and a query's max and
// sum combine the lane's 32 values with those of lane l ^ 32 (a permlane32
// swap).  Two tiles per loop trip, with the S^T registers of the current and
// the next tile trading roles.  The softmax
// reference moves up only when a tile's max exceeds it by more than 8 (log2
// units), so probabilities stay below 2^8 and the rescale of O is rare.
// Precision: V's bf16 values are exact in fp16 between 2^-14 and 2^16 in
// magnitude (a dimension tile whose largest value lies outside [2^-10,
// 2^16) is staged scaled by a power of two, see v_store).  P is
// rounded to fp16 (at most 2^-11 relative) and the softmax sum l adds the
// same rounded values, so each output is an exact average of V rows under
// weights within 2^-10 (relative) of the true ones: its error is at most
// 2^-10 of the weighted mean of |v - out|.  P carries a factor 2^7, which l
// cancels, so that fp16 keeps weights at full precision down to 2^-21 of
// the reference's.
#include <math.h>
#include <stddef.h>

#include "rtp_device.h"
#include "rtp_launch.h"

namespace rtp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfWaves = 8;                   // query heads per block, one per wave
constexpr int kPfThreads = kPfWaves * kWave;  // 512
constexpr int kPfQ = 32;                      // query positions per block
constexpr int kPfK = 64;                      // keys per tile
constexpr int kKRow = 128 + 8;                // bf16 per staged K row (272 B: rows 4 banks apart)
constexpr int kVRow = kPfK + 8;               // bf16 per staged V^T row (144 B, 16-B aligned)
constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfPScale = 7.0f;              // log2 of the factor carried by P

struct PfArgs {
    const uint16_t *q, *K, *V;
    float *out;
    int Hq, Hkv, T, head_begin, n_heads, n_sink, window;
    int G;        // query heads per KV head
    int hc;       // chunks of up to kPfWaves heads per KV head
    int c_first;  // first chunk (g * hc + s) that holds a head of the range
    int nc;       // chunks that do
    int64_t kv_cap;
    float qscale;    // |scale| * log2(e), at least 1e-30 (a masked score of -inf gives 0)
    uint32_t qsign;  // 0x80008000 when scale < 0: Q's signs are flipped instead
};

constexpr int kPfHalf = kPfThreads / 2;       // threads of one wave group
constexpr int kKBuf = kPfK * kKRow;           // bf16 per K buffer
constexpr int kVBuf = 128 * kVRow;            // bf16 per V^T buffer

struct PfShared {
    uint16_t k[2][kKBuf];
    uint16_t vt[2][kVBuf];  // V^T in fp16, each dimension tile scaled by 2^-vshift
    // Per buffer, one byte per dimension tile: its scale shift (0 almost
    // always); read as one word, which every lane of a wave loads at once
    // without bank conflicts.
    int8_t vshift[2][kPfWaves / 2];
};

static_assert(offsetof(PfShared, vshift) % 4 == 0, "each buffer's shifts are one aligned word");

// Magnitude bits of the smallest bf16 value that fp16 cannot hold (2^16).
constexpr uint32_t kBf16F16Over = 0x4780u;
// Biased binade below which a dimension tile's largest value is scaled up
// (2^-10), and the largest upward shift (the tile's scale factor 2^-k must
// stay a finite float).
constexpr int kSmallBinade = 117;
constexpr int kMaxUp = 100;

// v of this lane and of lane l ^ 32 (a VALU swap of the wave's halves).
struct X32 {
    float a, b;
};
__device__ __forceinline__ X32 pair_x32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

__device__ __forceinline__ float max3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

struct HalfRegs {
    uint4 r[4];
};

// The first wave group stages K rows, the second V rows.  Thread t of a
// group loads, for j < 4: K row 16 j + t / 16, dims 8 (t % 16) .. +7 (each
// load covers whole rows); or V row 4 (t % 16) + j, dims 8 (t / 16) .. +7
// (64-B pieces of 16 rows, so that the transposing LDS stores of a wave
// spread over every bank).  Rows past the prompt read row T - 1 (their keys
// are masked).
__device__ __forceinline__ HalfRegs k_load(const uint16_t *Kb, int k0, int T)
{
    const int t = threadIdx.x & (kPfHalf - 1);
    HalfRegs h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kr = min(k0 + 16 * j + (t >> 4), T - 1);
        h.r[j] = *(reinterpret_cast<const uint4 *>(Kb + (int64_t)kr * 128) + (t & 15));
    }
    return h;
}

__device__ __forceinline__ HalfRegs v_load(const uint16_t *Vb, int k0, int T)
{
    const int t = threadIdx.x & (kPfHalf - 1);
    HalfRegs h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int vr = min(k0 + 4 * (t & 15) + j, T - 1);
        h.r[j] = *(reinterpret_cast<const uint4 *>(Vb + (int64_t)vr * 128) + (t >> 4));
    }
    return h;
}

__device__ __forceinline__ void k_store(const HalfRegs &h, PfShared &sh, int buf)
{
    const int t = threadIdx.x & (kPfHalf - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint4 *>(&sh.k[buf][(16 * j + (t >> 4)) * kKRow + 8 * (t & 15)]) = h.r[j];
}

// Two bf16 values as two fp16 values (round to nearest even): exact for
// magnitudes in [2^-14, 2^16), where fp16 holds every bf16 value.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w)
{
    const f16x2 c = {static_cast<_Float16>(__uint_as_float(w << 16)),
                     static_cast<_Float16>(__uint_as_float(w & 0xFFFF0000u))};
    return __builtin_bit_cast(uint32_t, c);
}

// Two bf16 values scaled by 2^-k, still as bf16: exact while the results
// are normal floats (a scaled value keeps its 8 significant bits); results
// below 2^-126 lose low bits, far below what fp16 keeps anyway.
__device__ __forceinline__ uint32_t bf16x2_scale(uint32_t w, int k)
{
    const float lo = __builtin_amdgcn_ldexpf(__uint_as_float(w << 16), -k);
    const float hi = __builtin_amdgcn_ldexpf(__uint_as_float(w & 0xFFFF0000u), -k);
    return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

// V transposed, in fp16: per dimension, the thread's four keys as one 8-B
// store; the 16 lanes of a dimension row write 128 contiguous bytes.  Within
// each 16-key group the 4-key blocks 1 and 2 trade places, so a lane's 8
// keys of a product step are contiguous (one 16-B read).  Staging wave i
// holds dimensions 32 i .. 32 i + 31 of the tile's 64 keys, which is one
// dimension tile of the second product.  If their largest magnitude is 2^16
// or more (beyond fp16) or below 2^-10, the wave stores them all scaled by
// 2^-k, the shift that brings the largest into [2^15, 2^16), and records k:
// the product then scales that tile's accumulators by 2^-k before and 2^k
// after (exact in fp32).  Every value keeps its bf16 bits unless it lies
// below fp16's normal range after the shift, and then stays within 2^-40 of
// the largest magnitude of its dimension tile (2^-25 absolute when the
// largest is at least 2^-10 and no shift is applied).
__device__ __forceinline__ void v_store(HalfRegs h, PfShared &sh, int buf)
{
    const int t = threadIdx.x & (kPfHalf - 1);
    const int d0 = 8 * (t >> 4), sb = t & 3;
    const int kk = 16 * ((t >> 2) & 3) + 4 * ((sb == 1) ? 2 : (sb == 2) ? 1 : sb);
    u16x2 mag = {0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2, h.r[j][c] & 0x7FFF7FFFu));
    const uint32_t mx = mag.x > mag.y ? mag.x : mag.y;
    // Scaled down when the largest magnitude is 2^16 or more (beyond fp16),
    // up when it is below 2^-10 (so that values near it stay in fp16's
    // normal range): either way the largest lands in [2^15, 2^16).  All-zero
    // tiles stay.
    const bool big = __ballot(mx >= kBf16F16Over) != 0;
    const bool small = __ballot(mx >= (uint32_t)(kSmallBinade << 7)) == 0 && __ballot(mx != 0u) != 0;
    int k = 0;
    if (big || small) {
        // The largest magnitude (as floats, these bit patterns order like
        // the magnitudes) and its biased binade e.
        const uint32_t wm = __float_as_uint(wave_max(__uint_as_float(mx << 16))) >> 16;
        const int e = (int)(wm >> 7);
        k = e - 142 > -kMaxUp ? e - 142 : -kMaxUp;
    }
    k = __builtin_amdgcn_readfirstlane(k);  // one value per wave
    if (k != 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) h.r[j][c] = bf16x2_scale(h.r[j][c], k);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) h.r[j][c] = bf16x2_to_f16x2(h.r[j][c]);
    if (lane_id() == 0) sh.vshift[buf][(threadIdx.x >> 6) & (kPfWaves / 2 - 1)] = (int8_t)k;
    uint16_t *vt = sh.vt[buf];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        *reinterpret_cast<uint2 *>(&vt[(d0 + 2 * c) * kVRow + kk]) =
            make_uint2(__builtin_amdgcn_perm(h.r[1][c], h.r[0][c], 0x05040100u),
                       __builtin_amdgcn_perm(h.r[3][c], h.r[2][c], 0x05040100u));
        *reinterpret_cast<uint2 *>(&vt[(d0 + 2 * c + 1) * kVRow + kk]) =
            make_uint2(__builtin_amdgcn_perm(h.r[1][c], h.r[0][c], 0x07060302u),
                       __builtin_amdgcn_perm(h.r[3][c], h.r[2][c], 0x07060302u));
    }
}

__global__ __launch_bounds__(kPfThreads) void prefill_kernel(PfArgs a)
{
    __shared__ PfShared sh;
    // Heaviest query tiles (the latest positions) first.
    const int q0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * kPfQ;
    const int chunk = a.c_first + (int)blockIdx.y % a.nc, b = (int)blockIdx.y / a.nc;
    const int g = chunk / a.hc, hs = (chunk % a.hc) * kPfWaves;
    const int lane = lane_id(), w = threadIdx.x / kWave, gl = lane >> 5;
    const int h = g * a.G + hs + w;
    const bool active = hs + w < a.G && h >= a.head_begin && h < a.head_begin + a.n_heads;
    const bool vgrp = w >= kPfWaves / 2;

    const uint16_t *Kb = a.K + ((int64_t)b * a.Hkv + g) * a.kv_cap * 128;
    const uint16_t *Vb = a.V + ((int64_t)b * a.Hkv + g) * a.kv_cap * 128;

    // Tiles: the sink tiles, then the causal / window range.
    const int q_last = min(q0 + kPfQ - 1, a.T - 1);
    const bool local = a.window >= 1;
    const int w0_first = local ? max(0, q0 + 1 - a.window) : 0;
    const int w0_last = local ? max(0, q_last + 1 - a.window) : 0;
    const int sink_hi = local ? min(a.n_sink, w0_last) : 0;  // keys below: some query's sink
    const int ns = (sink_hi + kPfK - 1) / kPfK;
    const int kt_first = max(ns, w0_first / kPfK), kt_last = q_last / kPfK;
    const int nt = ns + max(0, kt_last - kt_first + 1);
    auto tile_k0 = [&](int it) { return (it < ns ? it : kt_first + it - ns) * kPfK; };

    // B operand of S^T: query q0 + l%32 (rows past T repeat T - 1), dims
    // 16 ks + 8 (l/32) .. +7.
    const int my_q = q0 + (lane & 31);
    const int qc = min(my_q, a.T - 1);
    bf16x8 qb[8];
    if (active) {
        const uint16_t *Qr = a.q + (((int64_t)b * a.Hq + h) * (int64_t)a.T + qc) * 128;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 u = *reinterpret_cast<const uint4 *>(Qr + 16 * ks + 8 * gl);
            u.x ^= a.qsign;
            u.y ^= a.qsign;
            u.z ^= a.qsign;
            u.w ^= a.qsign;
            qb[ks] = __builtin_bit_cast(bf16x8, u);
        }
    }
    const int my_w0 = local ? max(0, qc + 1 - a.window) : 0;
    const int my_sink = local ? min(a.n_sink, my_w0) : 0;

    float m = -INFINITY, l = 0.0f;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.0f;

    const char *lds = reinterpret_cast<const char *>(&sh);
    const int kl = 2 * ((lane & 31) * kKRow + 8 * gl);
    const int vl = 2 * (2 * kKBuf + (lane & 31) * kVRow + 8 * gl);
    // S^T = K Q^T from K buffer kb.
    auto product_qk = [&](f32x16 (&acc)[2], int kb) {
        const char *kp = lds + __builtin_amdgcn_readfirstlane(kb * 2 * kKBuf) + kl;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[st][e] = 0.0f;
#pragma unroll
        for (int kq = 0; kq < 8; ++kq)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kp + 2 * (32 * st * kKRow + 16 * kq));
                acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kq], acc[st], 0, 0, 0);
            }
    };

    // K runs one tile ahead of V: the products of an iteration are S^T of
    // tile it + 1 (K buffer (it + 1) % 2) and O^T += V^T P^T of tile it (V
    // buffer it % 2); the first group then stages K of tile it + 2 and the
    // second V of tile it + 1, into the buffers the previous iteration read.
    HalfRegs rg;
    if (!vgrp) {
        k_store(k_load(Kb, tile_k0(0), a.T), sh, 0);
        if (nt > 1) k_store(k_load(Kb, tile_k0(1), a.T), sh, 1);
    } else {
        v_store(v_load(Vb, tile_k0(0), a.T), sh, 0);
    }
    __syncthreads();
    f32x16 s[2], sn[2];
    if (active) product_qk(s, 0);
    __syncthreads();
    // One tile: cur holds its S^T, nxt receives the next tile's.  Two tiles
    // per loop trip with the roles swapped, so no copy moves nxt to cur.
    auto step = [&](int it, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        const bool ld = vgrp ? it + 1 < nt : it + 2 < nt;
        if (ld) rg = vgrp ? v_load(Vb, tile_k0(it + 1), a.T) : k_load(Kb, tile_k0(it + 2), a.T);
        if (active) {
            const int k0 = tile_k0(it);
            // Masked keys score -inf (their probability is exactly 0); a tile
            // whose every key is allowed for every query of the block skips
            // the test.
            const bool full = k0 + kPfK - 1 <= q0 &&
                              (!local || k0 >= w0_last || k0 + kPfK <= min(a.n_sink, w0_first));
            if (!full) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = k0 + 32 * st + 8 * (e >> 2) + 4 * gl + (e & 3);
                        const bool ok = (key <= qc) & (!local | (key < my_sink) | (key >= my_w0));
                        cur[st][e] = ok ? cur[st][e] : -INFINITY;
                    }
            }
            // The query's max over the tile (both lane halves), in log2 units.
            float tmax = fmaxf(cur[0][0], cur[1][0]);
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 1; e < 16; e += 2) tmax = max3(tmax, cur[st][e], cur[st][e + (e < 15)]);
            const X32 tp = pair_x32(tmax);
            tmax = fmaxf(tp.a, tp.b) * a.qscale;
            // The reference m moves up only when the tile's max exceeds it by
            // more than 8 (so probabilities stay below 2^8): the rescale of
            // O and l is rare after the first tiles.
            if (__ballot(tmax > m + 8.0f)) {
                const float mn = tmax > m + 8.0f ? tmax : m;
                const float corr = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
                l *= corr;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[dt][e] *= corr;
                m = mn;
            }
            // S^T of the next tile (on the last tile, of a stale buffer,
            // unused) while p = 2^(s * qscale - m) is taken.
            product_qk(nxt, (it + 1) & 1);
            // Probabilities carry a factor 2^7 (cancelled by l): they lie
            // in (0, 2^15], and fp16 keeps them to 2^-11 relative down to
            // 2^-21 of the reference's weight.
            const float nm = m == -INFINITY ? 0.0f : kPfPScale - m;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    cur[st][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[st][e], a.qscale, nm));
            // O^T += V^T P^T; key-step ks takes elements 8 (ks % 2) .. +7 of
            // cur[ks / 2].  P enters as fp16 (round to nearest even) and l
            // sums the same rounded values.
            const uint32_t vsh = __builtin_amdgcn_readfirstlane(
                *reinterpret_cast<const uint32_t *>(sh.vshift[it & 1]));
            const bool scaled = vsh != 0u;
            auto shift_of = [&](int dp) { return (int)(int8_t)(vsh >> (8 * dp)); };
            if (scaled) {
#pragma unroll
                for (int dp = 0; dp < 4; ++dp) {
                    const float f = __builtin_amdgcn_ldexpf(1.0f, -shift_of(dp));
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[dp][e] *= f;
                }
            }
            const char *vp = lds + __builtin_amdgcn_readfirstlane((it & 1) * 2 * kVBuf) + vl;
            const f16x2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
            float psum = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int st = ks >> 1, e0 = 8 * (ks & 1);
                f16x8 ph;
#pragma unroll
                for (int t = 0; t < 8; ++t) ph[t] = static_cast<_Float16>(cur[st][e0 + t]);
#pragma unroll
                for (int t = 0; t < 8; t += 2) {
                    const f16x2 pr = {ph[t], ph[t + 1]};
                    psum = __builtin_amdgcn_fdot2(pr, one, psum, false);
                }
#pragma unroll
                for (int dp = 0; dp < 4; dp += 2) {
                    const f16x8 v0 = *reinterpret_cast<const f16x8 *>(vp + 2 * (32 * dp * kVRow + 16 * ks));
                    const f16x8 v1 =
                        *reinterpret_cast<const f16x8 *>(vp + 2 * (32 * (dp + 1) * kVRow + 16 * ks));
                    o[dp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v0, ph, o[dp], 0, 0, 0);
                    o[dp + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v1, ph, o[dp + 1], 0, 0, 0);
                }
            }
            if (scaled) {
#pragma unroll
                for (int dp = 0; dp < 4; ++dp) {
                    const float f = __builtin_amdgcn_ldexpf(1.0f, shift_of(dp));
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[dp][e] *= f;
                }
            }
            const X32 pp = pair_x32(psum);
            l += pp.a + pp.b;
        }
        if (ld) {
            if (vgrp)
                v_store(rg, sh, (it + 1) & 1);
            else
                k_store(rg, sh, it & 1);
        }
        __syncthreads();
    };
    int it = 0;
    for (; it + 1 < nt; it += 2) {
        step(it, s, sn);
        step(it + 1, sn, s);
    }
    if (it < nt) step(it, s, sn);
    if (!active || my_q >= a.T) return;
    // out[q][dim] = O / l: lane l holds dims 32 dt + 8 i + 4 (l/32) + j.
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float *orow = a.out + (((int64_t)b * a.Hq + h) * (int64_t)a.T + my_q) * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<float4 *>(orow + 32 * dt + 8 * i + 4 * gl) =
                make_float4(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv, o[dt][4 * i + 2] * inv,
                            o[dt][4 * i + 3] * inv);
}

}  // namespace

hipError_t launch_prefill_attend(const uint16_t *q, const uint16_t *K, const uint16_t *V, int B,
                                 int Hq, int Hkv, int T, int64_t kv_cap, int head_begin,
                                 int n_heads, int n_sink, int window, float scale, float *out,
                                 hipStream_t stream)
{
    PfArgs a;
    a.q = q;
    a.K = K;
    a.V = V;
    a.out = out;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.T = T;
    a.head_begin = head_begin;
    a.n_heads = n_heads;
    a.n_sink = n_sink;
    a.window = window;
    a.kv_cap = kv_cap;
    // Clamped above zero so that -inf * qscale stays -inf.  At the clamp,
    // s * qscale - m is below 1e-8 in magnitude for any scores within 1e22
    // of each other, so 2^x rounds to exactly 1, as scale = 0 requires.
    a.qscale = fmaxf(fabsf(scale) * kPfLog2e, 1e-30f);
    a.qsign = scale < 0.0f ? 0x80008000u : 0u;
    a.G = Hq / Hkv;
    a.hc = (a.G + kPfWaves - 1) / kPfWaves;
    const int h_last = head_begin + n_heads - 1;
    a.c_first = (head_begin / a.G) * a.hc + (head_begin % a.G) / kPfWaves;
    const int c_last = (h_last / a.G) * a.hc + (h_last % a.G) / kPfWaves;
    a.nc = c_last - a.c_first + 1;
    const int gx = (T + kPfQ - 1) / kPfQ;
    return launch(prefill_kernel, dim3((unsigned)gx, (unsigned)(B * a.nc)), dim3(kPfThreads), 0,
                  stream, a);
}

}  // namespace rtp
