// One tile of the indexer scan (gist.science summary of arXiv 2605.16928,
// method section 2: a 16-dim projector applied to queries and keys before
// RoPE gives the indexer logits).  Shared by the scan kernel and by the
// kernel that runs the scan together with the local heads.
//
// HBM-bound: each 64-B k_r row is read once and scored against every query
// head of its group (up to G per tile), so the group shares one streaming
// read.  Each score is one lane's sequential fused multiply-add chain over
// dimensions 0..15: splitting the dot product across lanes would change its
// rounding.  Coalescing comes from the layout instead: lane l of a wave
// reads row base+l, so one wave instruction covers 64 consecutive rows, and
// each score store covers 64 consecutive floats.
#pragma once

#include "rtp_device.h"

namespace rtp {

constexpr int kScanThreads = 256;

// Launch geometry of the scan: tiles of kScanThreads * tpt tokens (x) times
// (batch row, KV group, chunk of up to G query heads) (y).
struct ScanGeom {
    int group;        // query heads per KV group
    int head_chunks;  // chunks of up to G heads per group
    int gx;           // token tiles per row
    int gy;           // B * Hkv_r * head_chunks
};

inline ScanGeom scan_geom(int B, int Hq_r, int Hkv_r, int N, int G, int tpt)
{
    ScanGeom g;
    g.group = Hq_r / Hkv_r;
    g.head_chunks = (g.group + G - 1) / G;
    const int64_t tile = (int64_t)kScanThreads * tpt;
    g.gx = (int)(((int64_t)N + tile - 1) / tile);
    g.gy = B * Hkv_r * g.head_chunks;
    return g;
}

// Tile (bx, y): thread t scores tokens bx*tile + t + k*kScanThreads,
// k < TPT, for the heads of chunk y % head_chunks of group y / head_chunks.
// k_r rows are 16 fp32 (64 B), or with kBf16 16 bf16 (32 B) widened exactly
// to fp32 before the same fma chain.
template <int G, int TPT, bool kBf16 = false>
__device__ __forceinline__ void scan_tile(const float *__restrict__ q_r,
                                          const void *__restrict__ k_r,
                                          float *__restrict__ scores, int N, int64_t kr_cap,
                                          int Hq_r, int Hkv_r, int group, int head_chunks,
                                          int bx, int y)
{
    constexpr int kTile = kScanThreads * TPT;
    const int chunk = y % head_chunks;
    const int bg = y / head_chunks;  // b * Hkv_r + g
    const int g = bg % Hkv_r;
    const int b = bg / Hkv_r;
    const int h0 = g * group + chunk * G;
    const int nh = min(G, group - chunk * G);

    const int64_t base = (int64_t)bx * kTile + threadIdx.x;

    float4 kv[TPT][4];
    if constexpr (kBf16) {
        const uint4 *krow = reinterpret_cast<const uint4 *>(
            static_cast<const uint16_t *>(k_r) + (int64_t)bg * kr_cap * 16);
        uint4 kw[TPT][2];
#pragma unroll
        for (int t = 0; t < TPT; ++t) {
            const int64_t i = base + (int64_t)t * kScanThreads;
            if (i < N) {
                kw[t][0] = krow[i * 2];
                kw[t][1] = krow[i * 2 + 1];
            } else {
                kw[t][0] = kw[t][1] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        // Word e of a 16-B piece holds dims 2e (low half) and 2e + 1.
#pragma unroll
        for (int t = 0; t < TPT; ++t)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 w = kw[t][j];
                kv[t][2 * j] = make_float4(__uint_as_float(w.x << 16),
                                           __uint_as_float(w.x & 0xFFFF0000u),
                                           __uint_as_float(w.y << 16),
                                           __uint_as_float(w.y & 0xFFFF0000u));
                kv[t][2 * j + 1] = make_float4(__uint_as_float(w.z << 16),
                                               __uint_as_float(w.z & 0xFFFF0000u),
                                               __uint_as_float(w.w << 16),
                                               __uint_as_float(w.w & 0xFFFF0000u));
            }
    } else {
        const float4 *krow = reinterpret_cast<const float4 *>(
            static_cast<const float *>(k_r) + (int64_t)bg * kr_cap * 16);
#pragma unroll
        for (int t = 0; t < TPT; ++t) {
            const int64_t i = base + (int64_t)t * kScanThreads;
            if (i < N) {
#pragma unroll
                for (int j = 0; j < 4; ++j) kv[t][j] = krow[i * 4 + j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) kv[t][j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
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
        for (int t = 0; t < TPT; ++t) {
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

}  // namespace rtp
