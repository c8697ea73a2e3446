// Indexer projections (gist.science summary, method section 2: a 16-dim
// projector is applied to query and key features before RoPE; the arXiv
// abstract gives the indexer's width as 16).  For token row x (128 bf16) of
// head h and that head's projector W_h (16 x 128 bf16):
//
//   out[j] = sum_c W_h[j][c] * x[c],   j < 16,
//
// with every bf16 product exact in fp32 and fp32 accumulation.  The same
// call projects one decode token (q_r of the retrieval query heads, or the
// new k_r row appended to the indexer key cache) or a whole prefill (the
// k_r cache of N tokens, a tokens x 128 by 128 x 16 product).
//
// A dense contraction on bf16 data, so it runs on the matrix cores: one wave
// takes 16 tokens at a time as the A operand of v_mfma_f32_16x16x32_bf16
// (lane l holds dims 8(l/16) .. +7 of token l%16 in each 32-dim step: one
// 16-B load), with the head's W^T as the B operand, loaded once and held in
// registers; four MFMAs cover the 128 input dims and leave lane l with
// outputs j = l%16 of tokens 4(l/16) .. +3.  The kernel is bound by reading
// x (256 B per token for 64 B written), so each wave puts kProjU tiles of
// loads in flight before its first MFMA.
#include "rtp_device.h"
#include "rtp_launch.h"

namespace rtp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kProjThreads = 256;
constexpr int kProjWaves = kProjThreads / kWave;
constexpr int kProjU = 4;                               // 16-token tiles per wave
constexpr int kProjTilesPerBlock = kProjWaves * kProjU;  // 16 tiles = 256 tokens

struct ProjArgs {
    const uint16_t *x;
    int64_t x_cap;
    int Hx, head_begin, H, T;
    const uint16_t *W;
    float *out;
    int64_t out_cap, out_pos;
    int tiles;  // 16-token tiles per (batch row, head)
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ __launch_bounds__(kProjThreads) void project_kernel(ProjArgs a)
{
    const int bh = blockIdx.y;  // b * H + h
    const int h = bh % a.H, b = bh / a.H;
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int row = lane & 15, quad = lane >> 4;
    const int tile0 = ((int)blockIdx.x * kProjWaves + w) * kProjU;
    if (tile0 >= a.tiles) return;  // whole wave

    const uint16_t *xb = a.x + ((int64_t)b * a.Hx + a.head_begin + h) * a.x_cap * 128;
    // This lane's A words of every tile: token 16 t + row (rows past T read
    // token T - 1 and are not stored), dims 32 ks + 8 quad .. +7.
    uint4 xa[kProjU][4];
#pragma unroll
    for (int u = 0; u < kProjU; ++u) {
        const int t = (tile0 + u) * 16 + row;
        const int64_t tt = t < a.T ? t : a.T - 1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            xa[u][ks] = *reinterpret_cast<const uint4 *>(xb + tt * 128 + 32 * ks + 8 * quad);
    }
    // B operand: W^T[c][j] = W_h[j][c] for j = row, c = 32 ks + 8 quad .. +7.
    const uint16_t *Wh = a.W + (int64_t)h * 16 * 128;
    bf16x8 wb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        wb[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(Wh + row * 128 + 32 * ks + 8 * quad));

    float *ob = a.out + ((int64_t)bh * a.out_cap + a.out_pos) * 16;
#pragma unroll
    for (int u = 0; u < kProjU; ++u) {
        if (tile0 + u >= a.tiles) break;
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u][ks]), wb[ks], c, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = (tile0 + u) * 16 + 4 * quad + j;
            if (t < a.T) ob[(int64_t)t * 16 + row] = c[j];
        }
    }
}

}  // namespace

hipError_t launch_index_project(const uint16_t *x, int B, int Hx, int64_t x_cap, int head_begin,
                                int H, int T, const uint16_t *W, float *out, int64_t out_cap,
                                int64_t out_pos, hipStream_t stream)
{
    ProjArgs a;
    a.x = x;
    a.x_cap = x_cap;
    a.Hx = Hx;
    a.head_begin = head_begin;
    a.H = H;
    a.T = T;
    a.W = W;
    a.out = out;
    a.out_cap = out_cap;
    a.out_pos = out_pos;
    a.tiles = (T + 15) / 16;
    const int gx = (a.tiles + kProjTilesPerBlock - 1) / kProjTilesPerBlock;
    return launch(project_kernel, dim3((unsigned)gx, (unsigned)(B * H)), dim3(kProjThreads), 0,
                  stream, a);
}

}  // namespace rtp
