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
// Matrix cores (bf16 in, fp32 accumulate), flash-style: each wave owns 16
// queries and walks the allowed key tiles of 16 keys with an online softmax.
//   S^T = K Q^T      4 x v_mfma_f32_16x16x32_bf16: lane l holds dims
//                    32ks + 8(l/16) .. +7 of key l%16 (A, one 16-B load) and
//                    of query l%16 (B, kept in registers); the result gives
//                    lane l keys 4(l/16) + j of query l%16.
//   O += P V         8 x v_mfma_f32_16x16x16_bf16: P's A operand is exactly
//                    the lane's own scores (query l%16, keys 4(l/16) + i);
//                    V's B operand (keys 4(l/16) + i, one dim) is gathered
//                    from the tile staged in this wave's LDS slice.  O's
//                    rows are queries 4(l/16) + j, so each query's softmax
//                    factors are fetched from lane q with a shuffle.
// P is rounded to bf16 for its MFMA (hi part) and the rounding residue is
// added by a second MFMA (lo part), so P is carried to about 2^-17.
#include <math.h>

#include "rtp_device.h"
#include "rtp_launch.h"

namespace rtp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / kWave;
constexpr int kPfQ = 16 * kPfWaves;  // queries per block
constexpr float kPfLog2e = 1.4426950408889634f;

struct PfArgs {
    const uint16_t *q, *K, *V;
    float *out;
    int Hq, Hkv, T, head_begin, n_heads, n_sink, window;
    int64_t kv_cap;
    float qscale;  // scale * log2(e)
};

struct PfShared {
    uint16_t v[kPfWaves][16][128];  // each wave's V tile
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// bf16 of x, rounded to nearest even (finite x).
__device__ __forceinline__ uint32_t bf16_rne(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float shfl(float v, int src)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

__global__ __launch_bounds__(kPfThreads) void prefill_kernel(PfArgs a)
{
    __shared__ PfShared sh;
    const int hh = blockIdx.y % a.n_heads, b = blockIdx.y / a.n_heads;
    const int h = a.head_begin + hh, g = h / (a.Hq / a.Hkv);
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int row = lane & 15, quad = lane >> 4;
    const int q0 = (int)blockIdx.x * kPfQ + w * 16;
    if (q0 >= a.T) return;  // whole wave; no block barrier below

    const uint16_t *Qb = a.q + ((int64_t)b * a.Hq + h) * (int64_t)a.T * 128;
    const uint16_t *Kb = a.K + ((int64_t)b * a.Hkv + g) * a.kv_cap * 128;
    const uint16_t *Vb = a.V + ((int64_t)b * a.Hkv + g) * a.kv_cap * 128;
    // B operand of S^T: query q0 + row (rows past T repeat T - 1), dims
    // 32 ks + 8 quad .. +7.
    const int my_q = q0 + row;
    const int64_t qr = my_q < a.T ? my_q : a.T - 1;
    bf16x8 qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qb[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(Qb + qr * 128 + 32 * ks + 8 * quad));

    // Key ranges of this wave's queries: the union over its 16 queries.
    const int q_last = min(q0 + 15, a.T - 1);
    const bool local = a.window >= 1;
    const int w0_first = local ? max(0, q0 + 1 - a.window) : 0;  // smallest w0 of the wave
    const int sink_hi = local ? min(a.n_sink, max(0, q_last + 1 - a.window)) : 0;
    // This lane's query: its allowed keys.
    const int my_w0 = local ? max(0, my_q + 1 - a.window) : 0;
    const int my_sink = local ? min(a.n_sink, my_w0) : 0;

    float m = -INFINITY, l = 0.0f;  // softmax state of query my_q (lanes with row = q)
    f32x4 o[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto tile = [&](int k0) {
        // S^T for keys k0 .. k0 + 15.
        uint4 ka[4];
        const int kr = k0 + row;
        const int64_t krc = kr < a.T ? kr : a.T - 1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            ka[ks] = *reinterpret_cast<const uint4 *>(Kb + krc * 128 + 32 * ks + 8 * quad);
        // Stage the V tile: lane l moves pieces l, l + 64, l + 128, l + 192
        // (key = piece / 16, 16-B piece = piece % 16).
        uint4 vx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pc = lane + 64 * i, key = k0 + (pc >> 4);
            const int64_t kc = key < a.T ? key : a.T - 1;
            vx[i] = *reinterpret_cast<const uint4 *>(Vb + kc * 128 + (pc & 15) * 8);
        }
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[ks]), qb[ks], s, 0, 0, 0);
        // Lane l: keys k0 + 4 quad + j of query my_q, in log2 units.
        float p[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = k0 + 4 * quad + j;
            const bool ok = my_q < a.T && key <= my_q &&
                            (!local || key < my_sink || key >= my_w0);
            p[j] = ok ? s[j] * a.qscale : -INFINITY;
            tmax = fmaxf(tmax, p[j]);
        }
        tmax = fmaxf(tmax, shfl(tmax, lane ^ 16));
        tmax = fmaxf(tmax, shfl(tmax, lane ^ 32));
        const float mn = fmaxf(m, tmax);
        const float corr = (m == -INFINITY) ? (mn == -INFINITY ? 1.0f : 0.0f) : exp2f(m - mn);
        float psum = 0.0f;
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e = p[j] == -INFINITY ? 0.0f : exp2f(p[j] - mn);
            psum += e;
            ph[j] = bf16_rne(e);
            pl[j] = bf16_rne(e - __uint_as_float(ph[j] << 16));
        }
        psum += shfl(psum, lane ^ 16);
        psum += shfl(psum, lane ^ 32);
        l = l * corr + psum;
        m = mn;
        // O rows are queries 4 quad + j: their factors come from lane
        // 4 quad + j (row = that query).
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float cj = shfl(corr, 4 * quad + j);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) o[nt][j] *= cj;
        }
        // V tile into this wave's LDS slice, then the B operands.
        uint4 *vs = reinterpret_cast<uint4 *>(&sh.v[w][0][0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) vs[lane + 64 * i] = vx[i];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const i16x4 ahi = {(short)ph[0], (short)ph[1], (short)ph[2], (short)ph[3]};
        const i16x4 alo = {(short)pl[0], (short)pl[1], (short)pl[2], (short)pl[3]};
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            i16x4 bv;
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = (short)sh.v[w][4 * quad + i][16 * nt + row];
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bv, o[nt], 0, 0, 0);
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bv, o[nt], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();  // reads done before the next tile's writes
    };

    // Sink tiles first (local heads), then the window / causal range.
    int k_begin = 0;
    if (local) {
        for (int k0 = 0; k0 < sink_hi; k0 += 16) tile(k0);
        k_begin = max((w0_first / 16) * 16, ((sink_hi + 15) / 16) * 16);
    }
    for (int k0 = k_begin; k0 <= q_last; k0 += 16) tile(k0);

    // out[q][dim] = O / l for queries 4 quad + j.
    float *ob = a.out + ((int64_t)b * a.Hq + h) * (int64_t)a.T * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int qq = q0 + 4 * quad + j;
        const float lj = shfl(l, 4 * quad + j);
        const float inv = lj > 0.0f ? 1.0f / lj : 0.0f;
        if (qq < a.T) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) ob[(int64_t)qq * 128 + 16 * nt + row] = o[nt][j] * inv;
        }
    }
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
    a.qscale = scale * kPfLog2e;
    const int gx = (T + kPfQ - 1) / kPfQ;
    return launch(prefill_kernel, dim3((unsigned)gx, (unsigned)(B * n_heads)), dim3(kPfThreads), 0,
                  stream, a);
}

}  // namespace rtp
