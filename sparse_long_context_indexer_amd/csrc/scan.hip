// Indexer scan: fp32 score of every cached token for the retrieval query
// heads of one KV head, from the 16-dim pre-RoPE indexer keys (gist.science
// summary of arXiv 2605.16928, method section 2).
//
// HBM-bound: each 64-B k_r row is read once and scored against every query
// head of its group (up to 8 per block), so the group shares one streaming
// read.  Each score is one lane's sequential fused multiply-add chain over
// dimensions 0..15: splitting the dot product across lanes would change its
// rounding.  Coalescing comes from the layout instead: lane l of a wave
// reads row base+l, so one wave instruction covers 64 consecutive rows, and
// each score store covers 64 consecutive floats.
#include "rtp_device.h"
#include "rtp_launch.h"

namespace rtp {

constexpr int kScanThreads = 256;
constexpr int kScanTPT = 2;                          // tokens per thread
constexpr int kScanTile = kScanThreads * kScanTPT;   // tokens per block

template <int G>
__global__ __launch_bounds__(kScanThreads) void index_scores_kernel(
    const float *__restrict__ q_r, const float *__restrict__ k_r,
    float *__restrict__ scores, int N, int64_t kr_cap, int Hq_r, int Hkv_r,
    int group, int head_chunks)
{
    const int y = blockIdx.y;
    const int chunk = y % head_chunks;
    const int bg = y / head_chunks;  // b * Hkv_r + g
    const int g = bg % Hkv_r;
    const int b = bg / Hkv_r;
    const int h0 = g * group + chunk * G;
    const int nh = min(G, group - chunk * G);

    const float4 *krow = reinterpret_cast<const float4 *>(k_r + (int64_t)bg * kr_cap * 16);
    const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x;

    float4 kv[kScanTPT][4];
#pragma unroll
    for (int t = 0; t < kScanTPT; ++t) {
        const int64_t i = base + (int64_t)t * kScanThreads;
        if (i < N) {
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[t][j] = krow[i * 4 + j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[t][j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }

    const float *qb = q_r + ((int64_t)b * Hq_r + h0) * 16;
    float *sb = scores + ((int64_t)b * Hq_r + h0) * (int64_t)N;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (h >= nh) break;
        float q[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) q[j] = qb[h * 16 + j];
#pragma unroll
        for (int t = 0; t < kScanTPT; ++t) {
            const int64_t i = base + (int64_t)t * kScanThreads;
            const float k[16] = {kv[t][0].x, kv[t][0].y, kv[t][0].z, kv[t][0].w,
                                 kv[t][1].x, kv[t][1].y, kv[t][1].z, kv[t][1].w,
                                 kv[t][2].x, kv[t][2].y, kv[t][2].z, kv[t][2].w,
                                 kv[t][3].x, kv[t][3].y, kv[t][3].z, kv[t][3].w};
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) acc = __builtin_fmaf(q[j], k[j], acc);
            acc = (acc == 0.0f) ? 0.0f : acc;  // -0 becomes +0
            if (i < N) sb[(int64_t)h * N + i] = acc;
        }
    }
}

hipError_t launch_index_scores(const float *q_r, const float *k_r, float *scores,
                               int B, int Hq_r, int Hkv_r, int N, int64_t kr_cap,
                               hipStream_t stream)
{
    const int group = Hq_r / Hkv_r;
    const int gx = (int)((N + (int64_t)kScanTile - 1) / kScanTile);
    auto go = [&](auto kern, int G) {
        const int chunks = (group + G - 1) / G;
        dim3 grid(gx, B * Hkv_r * chunks);
        return launch(kern, grid, dim3(kScanThreads), 0, stream, q_r, k_r, scores, N, kr_cap,
                      Hq_r, Hkv_r, group, chunks);
    };
    if (group == 1) return go(index_scores_kernel<1>, 1);
    if (group == 2) return go(index_scores_kernel<2>, 2);
    if (group <= 4) return go(index_scores_kernel<4>, 4);
    return go(index_scores_kernel<8>, 8);
}

}  // namespace rtp
