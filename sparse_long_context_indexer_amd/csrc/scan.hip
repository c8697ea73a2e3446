// Indexer scan: fp32 score of every cached token for the retrieval query
// heads of one KV head, from the 16-dim pre-RoPE indexer keys (gist.science
// summary of arXiv 2605.16928, method section 2).  The tile itself is
// scan_tile (scan_tile.h); this launch runs tiles only.
#include "rtp_launch.h"
#include "scan_tile.h"

namespace rtp {

constexpr int kScanTPT = 2;  // tokens per thread

template <int G, bool kBf16 = false>
__global__ __launch_bounds__(kScanThreads) void index_scores_kernel(
    const float *__restrict__ q_r, const void *__restrict__ k_r,
    float *__restrict__ scores, int N, int64_t kr_cap, int Hq_r, int Hkv_r,
    int group, int head_chunks)
{
    scan_tile<G, kScanTPT, kBf16>(q_r, k_r, scores, N, kr_cap, Hq_r, Hkv_r, group, head_chunks,
                                  blockIdx.x, blockIdx.y);
}

// The scan over bf16 k_r rows (32 B per token instead of 64).
hipError_t launch_index_scores_bf16(const float *q_r, const uint16_t *k_r, float *scores,
                                    int B, int Hq_r, int Hkv_r, int N, int64_t kr_cap,
                                    hipStream_t stream)
{
    auto go = [&](auto kern, int G) {
        const ScanGeom g = scan_geom(B, Hq_r, Hkv_r, N, G, kScanTPT);
        return launch(kern, dim3(g.gx, g.gy), dim3(kScanThreads), 0, stream, q_r,
                      static_cast<const void *>(k_r), scores, N, kr_cap, Hq_r, Hkv_r, g.group,
                      g.head_chunks);
    };
    const int group = Hq_r / Hkv_r;
    if (group == 1) return go(index_scores_kernel<1, true>, 1);
    if (group == 2) return go(index_scores_kernel<2, true>, 2);
    if (group <= 4) return go(index_scores_kernel<4, true>, 4);
    return go(index_scores_kernel<8, true>, 8);
}

hipError_t launch_index_scores(const float *q_r, const float *k_r, float *scores,
                               int B, int Hq_r, int Hkv_r, int N, int64_t kr_cap,
                               hipStream_t stream)
{
    auto go = [&](auto kern, int G) {
        const ScanGeom g = scan_geom(B, Hq_r, Hkv_r, N, G, kScanTPT);
        return launch(kern, dim3(g.gx, g.gy), dim3(kScanThreads), 0, stream, q_r,
                      static_cast<const void *>(k_r), scores, N, kr_cap, Hq_r, Hkv_r, g.group,
                      g.head_chunks);
    };
    const int group = Hq_r / Hkv_r;
    if (group == 1) return go(index_scores_kernel<1>, 1);
    if (group == 2) return go(index_scores_kernel<2>, 2);
    if (group <= 4) return go(index_scores_kernel<4>, 4);
    return go(index_scores_kernel<8>, 8);
}

}  // namespace rtp
