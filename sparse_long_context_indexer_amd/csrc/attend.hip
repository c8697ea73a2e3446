// Exact decode attention over (a) each retrieval head's selected rows and
// (b) each local head's sinks plus sliding window (gist.science summary of
// arXiv 2605.16928, method sections 1 and 5).
//
// Both are HBM-bound GEMV-shaped work on bf16 K/V rows of 256 B, so no
// matrix cores: a row is spread over 16 lanes (16 B = 8 bf16 each), which
// makes every row read two whole 128-B lines; a wave works on 4 rows at a
// time and several rows are loaded before any is used, to keep enough
// gathers in flight.  Split-K: each block owns a contiguous slice of the
// row list and runs an online softmax over it (base-2 exponent, with
// scale*log2(e) folded into q); partial (max, sum, o[128]) records are
// merged across splits by combine_kernel.
//
// Local heads: the 8 query heads of a KV head share each row read.  Each lane
// forms 8 partial dot products; a butterfly over the 16 lanes of a row
// reduces all 8 in 8 exchanges (each step halves the heads a lane carries).
#include <float.h>
#include <math.h>

#include "rtp_device.h"
#include "rtp_launch.h"

namespace rtp {

constexpr int kAttThreads = 256;
constexpr int kGroups = kAttThreads / 16;  // 16-lane row groups per block
constexpr int kPart = 132;                 // floats per partial: m, l, pad, o[128]
constexpr int kSparseU = 4;                // rows per group per iteration
constexpr int kLocalU = 2;
constexpr int kLocalRows = 128;      // rows per local split (at least)
constexpr int kMaxLocalSplits = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float sum16(float v)
{
    v += __shfl_xor(v, 1, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 8, 16);
    return v;
}

__device__ __forceinline__ float rescale(float m_old, float m_new)
{
    return m_old == -INFINITY ? 0.0f : exp2f(m_old - m_new);
}

// ------------------------------------------------------------ sparse

// Work split: the kept rows of all B*n_q heads are cut into chunks of one
// common size, chosen on the device from the counts so that about
// kSparseTarget blocks have work whatever the per-head budgets are; block j
// takes chunk j of the concatenated per-head lists.  The grid is sized for
// the worst case (kSparseTarget + heads); blocks past the last chunk exit.
constexpr int kSparseTarget = 768;
constexpr int kSlice = 64;  // partials merged per block in the first merge level

int sparse_grid(int64_t R) { return (int)(kSparseTarget + R); }
int sparse_slices(int64_t R) { return (sparse_grid(R) + kSlice - 1) / kSlice; }

struct SparseWs {
    float *part;      // one partial per attention block
    float *super;     // [R][slices] first-level merges
    uint32_t *ctr;    // [R] slices merged so far
};

static size_t sparse_ws_layout(int64_t R, SparseWs *W, void *base)
{
    size_t off = 0;
    const size_t part = off;
    off += align_up((size_t)sparse_grid(R) * kPart * sizeof(float), 256);
    const size_t sup = off;
    off += align_up((size_t)R * sparse_slices(R) * kPart * sizeof(float), 256);
    const size_t ctr = off;
    off += align_up((size_t)R * sizeof(uint32_t), 256);
    if (W) {
        char *b = static_cast<char *>(base);
        W->part = reinterpret_cast<float *>(b + part);
        W->super = reinterpret_cast<float *>(b + sup);
        W->ctr = reinterpret_cast<uint32_t *>(b + ctr);
    }
    return off;
}

size_t sparse_ws_bytes(int64_t B, int64_t n_q, int N)
{
    (void)N;
    return sparse_ws_layout(B * n_q, nullptr, nullptr);
}

struct SplitPlan {
    int chunk;     // rows per split
    int r;         // head row (b * n_q + hr) of this block's split, -1 if none
    int first;     // index of the head row's first split
    int splits;    // splits of that head row
};

__device__ __forceinline__ int clamp_count(int c, int N) { return c < 0 ? 0 : (c > N ? N : c); }

// Every thread of the block must call this; all get the same plan.  Finds
// either the split that global index j falls in (j >= 0) or, for j < 0,
// the splits of head row `row`.
template <int NT>
__device__ SplitPlan plan_splits(const int32_t *count, int R, int N, int rows_per_iter, int j,
                                 int row, int64_t *s64, int *s32)
{
    // Total kept rows.
    int64_t tot = 0;
    for (int r = threadIdx.x; r < R; r += NT) tot += clamp_count(count[r], N);
    tot = wave_sum(tot);
    if (lane_id() == 0) s64[threadIdx.x / kWave] = tot;
    __syncthreads();
    int64_t T = 0;
    for (int w = 0; w < NT / kWave; ++w) T += s64[w];
    int64_t chunk = (T + kSparseTarget - 1) / kSparseTarget;
    if (chunk < rows_per_iter) chunk = rows_per_iter;
    chunk = (chunk + rows_per_iter - 1) / rows_per_iter * rows_per_iter;
    // Splits per head row over contiguous per-thread segments, then a scan.
    const int per = (R + NT - 1) / NT;
    const int r0 = threadIdx.x * per, r1 = min(R, r0 + per);
    int seg = 0;
    for (int r = r0; r < r1; ++r) seg += (int)((clamp_count(count[r], N) + chunk - 1) / chunk);
    int total;
    const int pre = block_exclusive_scan<NT>(seg, s32, &total);
    SplitPlan P;
    P.chunk = (int)chunk;
    __shared__ int sh_r, sh_first, sh_splits;
    if (threadIdx.x == 0) sh_r = -1;
    __syncthreads();
    int acc = pre;
    for (int r = r0; r < r1; ++r) {
        const int sp = (int)((clamp_count(count[r], N) + chunk - 1) / chunk);
        const bool hit = j >= 0 ? (j >= acc && j < acc + sp) : (r == row);
        if (hit) {
            sh_r = r;
            sh_first = acc;
            sh_splits = sp;
        }
        acc += sp;
    }
    __syncthreads();
    P.r = sh_r;
    P.first = sh_r >= 0 ? sh_first : 0;
    P.splits = sh_r >= 0 ? sh_splits : 0;
    __syncthreads();
    return P;
}

__global__ __launch_bounds__(kAttThreads) void sparse_attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ count, int N, int64_t kv_cap, int Hq, int Hkv,
    int q_head_begin, int n_q, int R, float qscale, float *__restrict__ part,
    uint32_t *__restrict__ ctr)
{
    __shared__ float wm[kAttThreads / kWave], wl[kAttThreads / kWave];
    __shared__ float wo[kAttThreads / kWave][128];
    __shared__ int64_t s64[kAttThreads / kWave];
    __shared__ int s32[kAttThreads / kWave + 1];
    constexpr int kRowsPerIter = kGroups * kSparseU;
    const int blk = blockIdx.x;
    if (blk == 0)  // the merge that follows counts slices from zero
        for (int i = threadIdx.x; i < R; i += kAttThreads) ctr[i] = 0u;
    const SplitPlan plan = plan_splits<kAttThreads>(count, R, N, kRowsPerIter, blk, -1, s64, s32);
    if (plan.r < 0) return;  // past the last split: no partial to write
    const int prow = plan.r;
    const int b = prow / n_q, hr = prow % n_q;
    const int h = q_head_begin + hr;
    const int g = h / (Hq / Hkv);
    float *pr = part + (int64_t)blk * kPart;
    const int cnt = clamp_count(count[prow], N);
    const int begin = (blk - plan.first) * plan.chunk;
    const int end = min(cnt, begin + plan.chunk);

    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int grp = lane >> 4, sub = lane & 15;
    float qf[8];
    {
        const uint4 qw = *reinterpret_cast<const uint4 *>(q + ((int64_t)b * Hq + h) * 128 + sub * 8);
        bf16x8_to_f32(qw, qf);
#pragma unroll
        for (int c = 0; c < 8; ++c) qf[c] *= qscale;
    }
    const int64_t kvb = ((int64_t)b * Hkv + g) * kv_cap * 128 + sub * 8;
    const uint16_t *Kb = K + kvb;
    const uint16_t *Vb = V + kvb;
    const int32_t *ir = idx + (int64_t)prow * N;

    float m = -INFINITY, l = 0.0f, o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = 0.0f;

    for (int base = begin; base < end; base += kRowsPerIter) {
        uint4 kw[kSparseU], vw[kSparseU];
        bool ok[kSparseU];
#pragma unroll
        for (int u = 0; u < kSparseU; ++u) {
            const int j = base + u * kGroups + w * 4 + grp;
            int t = j < end ? ir[j] : -1;
            ok[u] = (unsigned)t < (unsigned)N;
            const int64_t off = ok[u] ? (int64_t)t * 128 : 0;
            kw[u] = *reinterpret_cast<const uint4 *>(Kb + off);
            vw[u] = *reinterpret_cast<const uint4 *>(Vb + off);
        }
        float lg[kSparseU];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kSparseU; ++u) {
            float kf[8];
            bf16x8_to_f32(kw[u], kf);
            float d = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) d = fmaf(qf[c], kf[c], d);
            d = sum16(d);
            lg[u] = ok[u] ? d : -INFINITY;
            mx = fmaxf(mx, lg[u]);
        }
        const float mn = fmaxf(m, mx);
        if (mn == -INFINITY) continue;
        const float corr = rescale(m, mn);
        l *= corr;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] *= corr;
#pragma unroll
        for (int u = 0; u < kSparseU; ++u) {
            const float pw = ok[u] ? exp2f(lg[u] - mn) : 0.0f;
            float vf[8];
            bf16x8_to_f32(vw[u], vf);
            l += pw;
#pragma unroll
            for (int c = 0; c < 8; ++c) o[c] = fmaf(pw, vf[c], o[c]);
        }
        m = mn;
    }

    // Merge the 4 row groups of the wave, then the waves of the block.
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
        const float mo = __shfl_xor(m, off);
        const float lo = __shfl_xor(l, off);
        const float mn = fmaxf(m, mo);
        const float a = rescale(m, mn), bb = rescale(mo, mn);
        l = l * a + lo * bb;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float oo = __shfl_xor(o[c], off);
            o[c] = o[c] * a + oo * bb;
        }
        m = mn;
    }
    if (lane < 16) {
#pragma unroll
        for (int c = 0; c < 8; ++c) wo[w][sub * 8 + c] = o[c];
        if (lane == 0) {
            wm[w] = m;
            wl[w] = l;
        }
    }
    __syncthreads();
    if (threadIdx.x < 128) {
        float M = -INFINITY;
        for (int i = 0; i < kAttThreads / kWave; ++i) M = fmaxf(M, wm[i]);
        float L = 0.0f, O = 0.0f;
        for (int i = 0; i < kAttThreads / kWave; ++i) {
            const float f = rescale(wm[i], M);
            L += wl[i] * f;
            O += wo[i][threadIdx.x] * f;
        }
        pr[4 + threadIdx.x] = O;
        if (threadIdx.x == 0) {
            pr[0] = M;
            pr[1] = L;
        }
    }
}

// Merges n partials (max, sum, o[128]) with a block of kCombThreads:
// kCombGroups groups of 128 threads (one per dimension) take every
// kCombGroups-th partial, then the groups are summed.  Writes either a
// merged partial (dst_part) or the normalised output row (dst_out).
constexpr int kCombGroups = 4;
constexpr int kCombThreads = kCombGroups * 128;

struct CombShared {
    float f[kSlice > 128 ? kSlice : 128];
    float o[kCombGroups][128];
    float red[kCombThreads / kWave];
    int last;
};

__device__ void merge_partials(const float *__restrict__ pr, int n, float *dst_part,
                               float *dst_out, CombShared &S)
{
    constexpr int kNW = kCombThreads / kWave;
    const int tid = threadIdx.x;
    const int c = tid & 127, grp = tid >> 7;
    float m = -INFINITY;
    for (int k = tid; k < n; k += kCombThreads) m = fmaxf(m, pr[(int64_t)k * kPart]);
    m = wave_max(m);
    if (lane_id() == 0) S.red[tid / kWave] = m;
    __syncthreads();
    float M = S.red[0];
    for (int i = 1; i < kNW; ++i) M = fmaxf(M, S.red[i]);
    __syncthreads();
    float l = 0.0f;
    for (int k = tid; k < n; k += kCombThreads) {
        const float f = rescale(pr[(int64_t)k * kPart], M);
        S.f[k] = f;
        l += pr[(int64_t)k * kPart + 1] * f;
    }
    l = wave_sum(l);
    if (lane_id() == 0) S.red[tid / kWave] = l;
    __syncthreads();
    float L = 0.0f;
    for (int i = 0; i < kNW; ++i) L += S.red[i];
    float o = 0.0f;
#pragma unroll 16
    for (int k = grp; k < n; k += kCombGroups) o = fmaf(pr[(int64_t)k * kPart + 4 + c], S.f[k], o);
    S.o[grp][c] = o;
    __syncthreads();
    if (grp == 0) {
        float t = 0.0f;
#pragma unroll
        for (int g = 0; g < kCombGroups; ++g) t += S.o[g][c];
        if (dst_out) dst_out[c] = L > 0.0f ? t / L : 0.0f;
        if (dst_part) {
            dst_part[4 + c] = t;
            if (c == 0) {
                dst_part[0] = M;
                dst_part[1] = L;
            }
        }
    }
    __syncthreads();
}

// Sparse heads, block (q, r): merges slice q (up to kSlice partials) of head
// row r's splits; the block that completes the row's last slice merges the
// slices into the output.
__global__ __launch_bounds__(kCombThreads) void sparse_combine_kernel(
    const float *__restrict__ part, float *__restrict__ super, uint32_t *__restrict__ ctr,
    const int32_t *__restrict__ count, int N, int R, int Hq, int q_head_begin, int n_q,
    int max_slices, float *__restrict__ out)
{
    __shared__ CombShared S;
    __shared__ int64_t s64[kCombThreads / kWave];
    __shared__ int s32[kCombThreads / kWave + 1];
    const int q = blockIdx.x, r = blockIdx.y;
    const SplitPlan plan =
        plan_splits<kCombThreads>(count, R, N, kGroups * kSparseU, -1, r, s64, s32);
    const int b = r / n_q, hr = r % n_q;
    float *dst = out + ((int64_t)b * Hq + q_head_begin + hr) * 128;
    const int slices = (plan.splits + kSlice - 1) / kSlice;
    if (slices == 0) {  // an empty row: nothing was kept
        if (q == 0 && threadIdx.x < 128) dst[threadIdx.x] = 0.0f;
        return;
    }
    if (q >= slices) return;
    float *sp = super + ((int64_t)r * max_slices) * kPart;
    const int k0 = q * kSlice;
    merge_partials(part + (int64_t)(plan.first + k0) * kPart, min(kSlice, plan.splits - k0),
                   sp + (int64_t)q * kPart, nullptr, S);
    // Publish this slice, then count it; the last one merges them all.
    __threadfence();
    if (threadIdx.x == 0) S.last = atomicAdd(&ctr[r], 1u) == (uint32_t)(slices - 1);
    __syncthreads();
    if (!S.last) return;
    __threadfence();
    merge_partials(sp, slices, nullptr, dst, S);
}

// Local heads: S static splits per head row (S <= 128).
__global__ __launch_bounds__(kCombThreads) void local_combine_kernel(
    const float *__restrict__ part, int S_, int Hq, int q_head_begin, int n_q,
    float *__restrict__ out)
{
    __shared__ CombShared S;
    const int r = blockIdx.x;
    const int b = r / n_q, hr = r % n_q;
    merge_partials(part + (int64_t)r * S_ * kPart, S_, nullptr,
                   out + ((int64_t)b * Hq + q_head_begin + hr) * 128, S);
}

hipError_t launch_sparse_decode(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                const int32_t *idx, const int32_t *count, int B, int Hq,
                                int Hkv, int N, int64_t kv_cap, int q_head_begin,
                                int n_q_heads, float scale, float *out, void *ws,
                                hipStream_t stream)
{
    const int R = B * n_q_heads;
    SparseWs W;
    sparse_ws_layout(R, &W, ws);
    RTP_TRY(launch(sparse_attn_kernel, dim3(sparse_grid(R)), dim3(kAttThreads), 0, stream, q,
                   K, V, idx, count, N, kv_cap, Hq, Hkv, q_head_begin, n_q_heads, R,
                   scale * kLog2e, W.part, W.ctr));
    const int slices = sparse_slices(R);
    return launch(sparse_combine_kernel, dim3(slices, R), dim3(kCombThreads), 0, stream, W.part,
                  W.super, W.ctr, count, N, R, Hq, q_head_begin, n_q_heads, slices, out);
}

// ------------------------------------------------------------- local

static int64_t local_rows_count(int N, int n_sink, int window)
{
    const int64_t w_start = N > window ? (int64_t)N - window : 0;
    const int64_t sink_end = n_sink < w_start ? n_sink : w_start;
    return sink_end + (N - w_start);
}

int local_splits(int64_t n_rows)
{
    int64_t s = (n_rows + kLocalRows - 1) / kLocalRows;
    return (int)(s < 1 ? 1 : (s > kMaxLocalSplits ? kMaxLocalSplits : s));
}

size_t local_ws_bytes(int64_t B, int64_t n_q, int N)
{
    // The row list never exceeds N rows, so this bounds every n_sink/window.
    return align_up((size_t)(B * n_q * local_splits(N)) * kPart * sizeof(float), 256);
}

// Block (s, y, b): KV head g = g_first + y / chunks_per_g, query heads
// [h_lo, h_hi) of that head within the local range (at most 8), rows of
// split s of the local row list.
__global__ __launch_bounds__(kAttThreads) void local_attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int N, int64_t kv_cap, int Hq, int Hkv,
    int q_head_begin, int n_q, int n_sink, int window, float qscale, int S,
    int chunks_per_g, float *__restrict__ part)
{
    __shared__ float wm[kAttThreads / kWave][8], wl[kAttThreads / kWave][8];
    __shared__ float wo[kAttThreads / kWave][8][128];
    const int G = Hq / Hkv;
    const int s = blockIdx.x, b = blockIdx.z;
    const int g = q_head_begin / G + (int)blockIdx.y / chunks_per_g;
    const int ck = (int)blockIdx.y % chunks_per_g;
    const int h_lo = max(q_head_begin, g * G + ck * 8);
    const int h_hi = min(q_head_begin + n_q, min(g * G + G, g * G + ck * 8 + 8));
    const int nh = h_hi - h_lo;
    if (nh <= 0) return;

    const int64_t w_start = N > window ? (int64_t)N - window : 0;
    const int64_t sink_end = n_sink < w_start ? n_sink : w_start;
    const int64_t n_rows = sink_end + (N - w_start);
    constexpr int kRowsPerIter = kGroups * kLocalU;
    int64_t chunk = (n_rows + S - 1) / S;
    chunk = (chunk + kRowsPerIter - 1) / kRowsPerIter * kRowsPerIter;
    const int64_t begin = (int64_t)s * chunk;
    const int64_t end = min(n_rows, begin + chunk);

    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int grp = lane >> 4, sub = lane & 15;

    float qf[8][8];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        if (hh < nh) {
            const uint4 qw = *reinterpret_cast<const uint4 *>(
                q + ((int64_t)b * Hq + h_lo + hh) * 128 + sub * 8);
            bf16x8_to_f32(qw, qf[hh]);
#pragma unroll
            for (int c = 0; c < 8; ++c) qf[hh][c] *= qscale;
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) qf[hh][c] = 0.0f;
        }
    }
    const int64_t kvb = ((int64_t)b * Hkv + g) * kv_cap * 128 + sub * 8;
    const uint16_t *Kb = K + kvb;
    const uint16_t *Vb = V + kvb;

    float m[8], l[8], o[8][8];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[hh][c] = 0.0f;
    }
    const int b3 = (sub >> 3) & 1, b2 = (sub >> 2) & 1, b1 = (sub >> 1) & 1;

    for (int64_t base = begin; base < end; base += kRowsPerIter) {
        uint4 kw[kLocalU], vw[kLocalU];
        bool ok[kLocalU];
#pragma unroll
        for (int u = 0; u < kLocalU; ++u) {
            const int64_t j = base + u * kGroups + w * 4 + grp;
            ok[u] = j < end;
            const int64_t row = j < sink_end ? j : w_start + (j - sink_end);
            const int64_t off = ok[u] ? row * 128 : 0;
            kw[u] = *reinterpret_cast<const uint4 *>(Kb + off);
            vw[u] = *reinterpret_cast<const uint4 *>(Vb + off);
        }
        float lg[kLocalU][8];
#pragma unroll
        for (int u = 0; u < kLocalU; ++u) {
            float kf[8];
            bf16x8_to_f32(kw[u], kf);
            float d[8];
#pragma unroll
            for (int hh = 0; hh < 8; ++hh) {
                float a = 0.0f;
#pragma unroll
                for (int c = 0; c < 8; ++c) a = fmaf(qf[hh][c], kf[c], a);
                d[hh] = a;
            }
            // Butterfly: after the steps over lane bits 3, 2, 1 a lane holds
            // one head, 4*b3 + 2*b2 + b1, summed over 8 lanes; bit 0 finishes.
            float d4[4], d2[2], d1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float send = b3 ? d[k] : d[k + 4];
                const float keep = b3 ? d[k + 4] : d[k];
                d4[k] = keep + __shfl_xor(send, 8, 16);
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float send = b2 ? d4[k] : d4[k + 2];
                const float keep = b2 ? d4[k + 2] : d4[k];
                d2[k] = keep + __shfl_xor(send, 4, 16);
            }
            {
                const float send = b1 ? d2[0] : d2[1];
                const float keep = b1 ? d2[1] : d2[0];
                d1 = keep + __shfl_xor(send, 2, 16);
            }
            d1 += __shfl_xor(d1, 1, 16);
            // Head hh's logit sits in lanes 2*hh and 2*hh + 1 of the group.
#pragma unroll
            for (int hh = 0; hh < 8; ++hh) {
                const float v = __shfl(d1, 2 * hh, 16);
                lg[u][hh] = ok[u] ? v : -INFINITY;
            }
        }
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            float mx = lg[0][hh];
#pragma unroll
            for (int u = 1; u < kLocalU; ++u) mx = fmaxf(mx, lg[u][hh]);
            const float mn = fmaxf(m[hh], mx);
            if (mn == -INFINITY) continue;
            const float corr = rescale(m[hh], mn);
            l[hh] *= corr;
#pragma unroll
            for (int c = 0; c < 8; ++c) o[hh][c] *= corr;
            m[hh] = mn;
        }
#pragma unroll
        for (int u = 0; u < kLocalU; ++u) {
            float vf[8];
            bf16x8_to_f32(vw[u], vf);
#pragma unroll
            for (int hh = 0; hh < 8; ++hh) {
                const float pw = ok[u] ? exp2f(lg[u][hh] - m[hh]) : 0.0f;
                l[hh] += pw;
#pragma unroll
                for (int c = 0; c < 8; ++c) o[hh][c] = fmaf(pw, vf[c], o[hh][c]);
            }
        }
    }

    // Merge the 4 row groups of the wave, then the waves of the block.
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
#pragma unroll
        for (int off = 16; off < kWave; off <<= 1) {
            const float mo = __shfl_xor(m[hh], off);
            const float lo = __shfl_xor(l[hh], off);
            const float mn = fmaxf(m[hh], mo);
            const float a = rescale(m[hh], mn), bb = rescale(mo, mn);
            l[hh] = l[hh] * a + lo * bb;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float oo = __shfl_xor(o[hh][c], off);
                o[hh][c] = o[hh][c] * a + oo * bb;
            }
            m[hh] = mn;
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
#pragma unroll
            for (int c = 0; c < 8; ++c) wo[w][hh][sub * 8 + c] = o[hh][c];
            if (lane == 0) {
                wm[w][hh] = m[hh];
                wl[w][hh] = l[hh];
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nh * 128; e += kAttThreads) {
        const int hh = e / 128, c = e % 128;
        float M = -INFINITY;
        for (int i = 0; i < kAttThreads / kWave; ++i) M = fmaxf(M, wm[i][hh]);
        float L = 0.0f, O = 0.0f;
        for (int i = 0; i < kAttThreads / kWave; ++i) {
            const float f = rescale(wm[i][hh], M);
            L += wl[i][hh] * f;
            O += wo[i][hh][c] * f;
        }
        float *pr = part + (((int64_t)b * n_q + (h_lo - q_head_begin + hh)) * S + s) * kPart;
        pr[4 + c] = O;
        if (c == 0) {
            pr[0] = M;
            pr[1] = L;
        }
    }
}

hipError_t launch_local_decode(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                               int B, int Hq, int Hkv, int N, int64_t kv_cap,
                               int q_head_begin, int n_q_heads, int n_sink, int window,
                               float scale, float *out, void *ws, hipStream_t stream)
{
    const int G = Hq / Hkv;
    const int S = local_splits(local_rows_count(N, n_sink, window));
    const int g_first = q_head_begin / G;
    const int g_last = (q_head_begin + n_q_heads - 1) / G;
    const int chunks_per_g = (G + 7) / 8;
    const int ny = (g_last - g_first + 1) * chunks_per_g;
    float *part = static_cast<float *>(ws);
    RTP_TRY(launch(local_attn_kernel, dim3(S, ny, B), dim3(kAttThreads), 0, stream, q, K, V, N,
                   kv_cap, Hq, Hkv, q_head_begin, n_q_heads, n_sink, window, scale * kLog2e,
                   S, chunks_per_g, part));
    return launch(local_combine_kernel, dim3(B * n_q_heads), dim3(kCombThreads), 0, stream, part,
                  S, Hq, q_head_begin, n_q_heads, out);
}

}  // namespace rtp
