// Sort-free top-p selection (gist.science summary of arXiv 2605.16928,
// method section 3: keep adding low-dim attention mass until it reaches p;
// method section 5: a histogram-based, sort-free threshold).
//
// The kept set is the shortest prefix, in descending score order with ties
// to the lower token index, whose mass sum(exp(s - M)) reaches p * Z.  It is
// found exactly, without sorting, as a mass-weighted radix select over the
// 64-bit composite key (order-preserving score key, then token index):
//
//   max     row max M per chunk (and clears the histograms and counters)
//   hist1   fp64 mass and count per level-1 bin = score key bits [31:20],
//           LDS histogram per block, merged with global atomics
//   pick1   per row: Z, the target p*Z, the boundary bin j1 (the first bin,
//           from the top, where the cumulative mass reaches the target) and
//           the mass A above it
//   emit1   tokens in bins above j1 are kept; tokens of bin j1 become
//           candidates (key, index)
//   resolve one block per row: the same step over key bits [19:10], then
//           [9:0] (the boundary is now one score value tau), then how many
//           tokens of score tau are needed and, if not all of them, the
//           lowest indices among them by a count-only radix select over the
//           index bits
//
// Masses are fp64: exp(s - M) in fp64 and fp64 sums, so the running sums
// agree with an fp64 reference to ~1e-16 relative.  HBM traffic: the scores
// are read three times (max, hist1, emit1); candidates are few except for
// near-flat rows.
#include <float.h>

#include "rtp_device.h"
#include "rtp_launch.h"

namespace rtp {

constexpr int kSelThreads = 256;
constexpr int kSelPerThread = 32;
constexpr int64_t kSelChunk = kSelThreads * kSelPerThread;  // scores per block
constexpr int kBins1 = 4096;
constexpr int kResThreads = 1024;
constexpr int kResBins = 2048;

struct SelRow {
    double Z;        // sum of exp(s - M) over the row
    double A;        // mass above the level-1 boundary bin
    double T;        // p * Z
    float M;         // row max
    uint32_t j1;     // level-1 boundary bin
    uint32_t n_cand; // candidates appended by emit1
    uint32_t pad[7];
};
static_assert(sizeof(SelRow) == 64, "SelRow is one 64-B record");

SelLayout sel_layout(int64_t R, int64_t N)
{
    SelLayout L;
    L.nblk = (N + kSelChunk - 1) / kSelChunk;
    size_t off = 0;
    L.rows = off;
    off += align_up((size_t)R * sizeof(SelRow), 256);
    L.mass1 = off;
    off += align_up((size_t)R * kBins1 * sizeof(double), 256);
    L.cnt1 = off;
    off += align_up((size_t)R * kBins1 * sizeof(uint32_t), 256);
    L.zero_end = off;
    L.pmax = off;
    off += align_up((size_t)R * L.nblk * sizeof(float), 256);
    L.cand = off;
    off += align_up((size_t)R * N * sizeof(uint2), 256);
    L.total = off;
    return L;
}

struct SelPtrs {
    SelRow *rows;
    double *mass1;
    uint32_t *cnt1;
    float *pmax;
    uint2 *cand;
    uint4 *zero;
    int64_t zero_words;  // uint4 words to clear
    int64_t nblk;
};

static SelPtrs sel_ptrs(void *ws, int64_t R, int64_t N)
{
    SelLayout L = sel_layout(R, N);
    char *base = static_cast<char *>(ws);
    SelPtrs P;
    P.rows = reinterpret_cast<SelRow *>(base + L.rows);
    P.mass1 = reinterpret_cast<double *>(base + L.mass1);
    P.cnt1 = reinterpret_cast<uint32_t *>(base + L.cnt1);
    P.pmax = reinterpret_cast<float *>(base + L.pmax);
    P.cand = reinterpret_cast<uint2 *>(base + L.cand);
    P.zero = reinterpret_cast<uint4 *>(base + L.rows);
    P.zero_words = (int64_t)((L.zero_end - L.rows) / sizeof(uint4));
    P.nblk = L.nblk;
    return P;
}

// ---------------------------------------------------------------- max

__global__ __launch_bounds__(kSelThreads) void sel_max_kernel(
    const float *__restrict__ scores, int N, SelPtrs P, int32_t *__restrict__ count)
{
    __shared__ float red[kSelThreads / kWave];
    const int64_t r = blockIdx.y;
    const int64_t blk = blockIdx.x;
    // Clear histograms, row state and counters (grid-stride).
    {
        const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * kSelThreads;
        const int64_t gtid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kSelThreads + threadIdx.x;
        for (int64_t w = gtid; w < P.zero_words; w += nthreads) P.zero[w] = make_uint4(0, 0, 0, 0);
        if (blk == 0 && threadIdx.x == 0) count[r] = 0;
    }
    const float *sr = scores + r * (int64_t)N;
    const int64_t c0 = blk * kSelChunk;
    float m = -FLT_MAX;
#pragma unroll 8
    for (int t = 0; t < kSelPerThread; ++t) {
        const int64_t i = c0 + (int64_t)t * kSelThreads + threadIdx.x;
        if (i < N) m = fmaxf(m, sr[i]);
    }
    m = wave_max(m);
    if (lane_id() == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
        for (int i = 1; i < kSelThreads / kWave; ++i) b = fmaxf(b, red[i]);
        P.pmax[r * P.nblk + blk] = b;
    }
}

__device__ __forceinline__ float row_max(const SelPtrs &P, int64_t r, float *red)
{
    float m = -FLT_MAX;
    for (int64_t i = threadIdx.x; i < P.nblk; i += blockDim.x) m = fmaxf(m, P.pmax[r * P.nblk + i]);
    m = wave_max(m);
    if (lane_id() == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    float b = red[0];
    for (int i = 1; i < (int)(blockDim.x / kWave); ++i) b = fmaxf(b, red[i]);
    __syncthreads();
    return b;
}

// -------------------------------------------------------------- hist1

__global__ __launch_bounds__(kSelThreads) void sel_hist1_kernel(
    const float *__restrict__ scores, int N, SelPtrs P)
{
    __shared__ double hm[kBins1];
    __shared__ uint32_t hc[kBins1];
    __shared__ float red[kSelThreads / kWave];
    const int64_t r = blockIdx.y;
    const double M = (double)row_max(P, r, red);
    for (int i = threadIdx.x; i < kBins1; i += kSelThreads) {
        hm[i] = 0.0;
        hc[i] = 0u;
    }
    __syncthreads();
    const float *sr = scores + r * (int64_t)N;
    const int64_t c0 = (int64_t)blockIdx.x * kSelChunk;
#pragma unroll 4
    for (int t = 0; t < kSelPerThread; ++t) {
        const int64_t i = c0 + (int64_t)t * kSelThreads + threadIdx.x;
        if (i < N) {
            const float s = sr[i];
            const uint32_t bin = score_key(s) >> 20;
            atomicAdd(&hm[bin], exp((double)s - M));
            atomicAdd(&hc[bin], 1u);
        }
    }
    __syncthreads();
    double *gm = P.mass1 + r * kBins1;
    uint32_t *gc = P.cnt1 + r * kBins1;
    for (int i = threadIdx.x; i < kBins1; i += kSelThreads) {
        const uint32_t c = hc[i];
        if (c) {
            atomicAdd(&gm[i], hm[i]);
            atomicAdd(&gc[i], c);
        }
    }
}

// -------------------------------------------------------------- pick1

__global__ __launch_bounds__(kSelThreads) void sel_pick1_kernel(SelPtrs P, float p)
{
    constexpr int kPer = kBins1 / kSelThreads;  // bins per thread
    __shared__ double scan[kSelThreads / kWave + 1];
    __shared__ float red[kSelThreads / kWave];
    __shared__ int chosen;  // highest bin where the running mass crosses T
    __shared__ int lowest;  // lowest non-empty bin
    const int64_t r = blockIdx.x;
    const float M = row_max(P, r, red);
    const double *gm = P.mass1 + r * kBins1;
    const uint32_t *gc = P.cnt1 + r * kBins1;
    // Thread t owns bins top - t*kPer - [0, kPer): thread order is score order.
    const int top = kBins1 - 1 - (int)threadIdx.x * kPer;
    double w[kPer];
    uint32_t c[kPer];
    double local = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        w[k] = gm[top - k];
        c[k] = gc[top - k];
        local += w[k];
    }
    if (threadIdx.x == 0) {
        chosen = -1;
        lowest = kBins1;
    }
    double Z;
    const double before = block_exclusive_scan<kSelThreads>(local, scan, &Z);
    const double T = (double)p * Z;
    // Running sums restart from each thread's block prefix, so rounding may
    // show a crossing in two neighbouring threads; the highest bin wins.
    double cum = before;
    int my_cross = -1, my_lowest = -1;
    double cross_before = 0.0, lowest_before = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        if (c[k]) {
            if (my_cross < 0 && cum < T && cum + w[k] >= T) {
                my_cross = top - k;
                cross_before = cum;
            }
            my_lowest = top - k;
            lowest_before = cum;
        }
        cum += w[k];
    }
    if (my_cross >= 0) atomicMax(&chosen, my_cross);
    if (my_lowest >= 0) atomicMin(&lowest, my_lowest);
    __syncthreads();
    if (chosen >= 0) {
        if (my_cross == chosen) {
            P.rows[r].j1 = (uint32_t)my_cross;
            P.rows[r].A = cross_before;
        }
    } else if (my_lowest >= 0 && my_lowest == lowest) {
        // Rounding kept the running sum just below the target: keep all.
        P.rows[r].j1 = (uint32_t)my_lowest;
        P.rows[r].A = lowest_before;
    }
    if (threadIdx.x == 0) {
        P.rows[r].Z = Z;
        P.rows[r].T = T;
        P.rows[r].M = M;
    }
}

// -------------------------------------------------------------- emit1

__global__ __launch_bounds__(kSelThreads) void sel_emit1_kernel(
    const float *__restrict__ scores, int N, SelPtrs P, int32_t *__restrict__ idx,
    int32_t *__restrict__ count)
{
    const int64_t r = blockIdx.y;
    const uint32_t j1 = P.rows[r].j1;
    const float *sr = scores + r * (int64_t)N;
    int32_t *ir = idx + r * (int64_t)N;
    uint2 *cr = P.cand + r * (int64_t)N;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(count + r);
    const int64_t c0 = (int64_t)blockIdx.x * kSelChunk;
    for (int t = 0; t < kSelPerThread; ++t) {
        const int64_t i = c0 + (int64_t)t * kSelThreads + threadIdx.x;
        const bool valid = i < N;
        const uint32_t key = valid ? score_key(sr[i]) : 0u;
        const uint32_t bin = key >> 20;
        const int64_t pa = wave_append(valid && bin > j1, cnt);
        if (pa >= 0) ir[pa] = (int32_t)i;
        const int64_t pc = wave_append(valid && bin == j1, &P.rows[r].n_cand);
        if (pc >= 0) cr[pc] = make_uint2(key, (uint32_t)i);
    }
}

// ------------------------------------------------------------ resolve

struct ResShared {
    double hm[kResBins];
    uint32_t hc[kResBins];
    double dscan[kResThreads / kWave + 1];
    uint32_t uscan[kResThreads / kWave + 1];
    int chosen;
    double chosen_before;
    uint32_t chosen_cbefore;
    int lowest;
};

// Keeps candidates whose digit equals `keep_digit`, emits those on the kept
// side of it to idx, drops the rest; compacts survivors in place.  Returns
// the survivor count.  emit_above: digits above are emitted (score levels);
// otherwise digits below are emitted (index levels).
__device__ int64_t res_filter(uint2 *cr, int64_t n, int shift, uint32_t mask,
                              uint32_t keep_digit, bool emit_above, bool by_index,
                              int32_t *ir, uint32_t *cnt, ResShared &S)
{
    int64_t kept_total = 0;
    for (int64_t c0 = 0; c0 < n; c0 += kResThreads) {
        const int64_t k = c0 + threadIdx.x;
        const bool valid = k < n;
        uint2 e = valid ? cr[k] : make_uint2(0, 0);
        const uint32_t field = by_index ? e.y : e.x;
        const uint32_t dg = (field >> shift) & mask;
        const bool out = valid && (emit_above ? dg > keep_digit : dg < keep_digit);
        const bool keep = valid && dg == keep_digit;
        const int64_t pa = wave_append(out, cnt);
        if (pa >= 0) ir[pa] = (int32_t)e.y;
        uint32_t tot;
        const uint32_t pos = block_exclusive_scan<kResThreads>((uint32_t)keep, S.uscan, &tot);
        // All reads of this chunk are done (the scan synchronised the block),
        // and survivors land at or below their read position.
        if (keep) cr[kept_total + pos] = e;
        kept_total += tot;
        __syncthreads();
    }
    return kept_total;
}

__global__ __launch_bounds__(kResThreads) void sel_resolve_kernel(
    int N, SelPtrs P, int32_t *__restrict__ idx, int32_t *__restrict__ count)
{
    __shared__ ResShared S;
    const int64_t r = blockIdx.x;
    const SelRow row = P.rows[r];
    const double M = (double)row.M;
    const double T = row.T;
    double A = row.A;
    int64_t n = row.n_cand;
    uint2 *cr = P.cand + r * (int64_t)N;
    int32_t *ir = idx + r * (int64_t)N;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(count + r);
    const int tid = threadIdx.x;

    // Score levels: key bits [19:10], then [9:0].
    for (int level = 0; level < 2 && n > 0; ++level) {
        const int shift = level == 0 ? 10 : 0;
        for (int i = tid; i < 1024; i += kResThreads) {
            S.hm[i] = 0.0;
            S.hc[i] = 0u;
        }
        if (tid == 0) {
            S.chosen = -1;
            S.lowest = -1;
        }
        __syncthreads();
        for (int64_t k = tid; k < n; k += kResThreads) {
            const uint32_t key = cr[k].x;
            const uint32_t dg = (key >> shift) & 1023u;
            atomicAdd(&S.hm[dg], exp((double)key_score(key) - M));
            atomicAdd(&S.hc[dg], 1u);
        }
        __syncthreads();
        // Thread t owns digit 1023 - t: thread order is descending score.
        const int dg = 1023 - tid;
        const double w = S.hm[dg];
        const uint32_t c = S.hc[dg];
        double tot;
        const double before = block_exclusive_scan<kResThreads>(w, S.dscan, &tot);
        const double x = A + before;
        // Highest digit where the running mass crosses T (see pick1); if
        // rounding hides every crossing, the lowest non-empty digit.
        if (c && x < T && x + w >= T) atomicMax(&S.chosen, dg);
        if (c) atomicMax(&S.lowest, tid);
        __syncthreads();
        if (S.chosen < 0 && tid == S.lowest) S.chosen = dg;
        __syncthreads();
        if (dg == S.chosen) S.chosen_before = before;
        __syncthreads();
        const uint32_t j = (uint32_t)S.chosen;
        A += S.chosen_before;
        n = res_filter(cr, n, shift, 1023u, j, true, false, ir, cnt, S);
    }
    if (n == 0) return;

    // Every survivor now has the same score tau.  Keep the first c of them
    // in index order: the smallest c with A + c * e_tau >= T.
    const uint32_t tau_key = cr[0].x;
    const double e_tau = exp((double)key_score(tau_key) - M);
    int64_t c = 1;
    if (A + (double)n * e_tau < T) {
        c = n;
    } else {
        double need = (T - A) / e_tau;
        c = need < 1.0 ? 1 : (int64_t)ceil(need);
        if (c > n) c = n;
        while (c > 1 && A + (double)(c - 1) * e_tau >= T) --c;
        while (c < n && A + (double)c * e_tau < T) ++c;
    }
    if (c == n) {
        for (int64_t c0 = 0; c0 < n; c0 += kResThreads) {
            const int64_t k = c0 + tid;
            const bool valid = k < n;
            const uint32_t ix = valid ? cr[k].y : 0u;
            const int64_t pa = wave_append(valid, cnt);
            if (pa >= 0) ir[pa] = (int32_t)ix;
        }
        return;
    }
    // Count-only radix select of the c lowest indices: bits [30:20], [19:10],
    // [9:0].  Indices are distinct, so the last level leaves one token.
    const int shifts[3] = {20, 10, 0};
    const uint32_t masks[3] = {2047u, 1023u, 1023u};
    for (int level = 0; level < 3 && n > 0 && c > 0; ++level) {
        const int shift = shifts[level];
        const uint32_t mask = masks[level];
        const int nb = (int)mask + 1;
        for (int i = tid; i < nb; i += kResThreads) S.hc[i] = 0u;
        if (tid == 0) S.chosen = -1;
        __syncthreads();
        for (int64_t k = tid; k < n; k += kResThreads)
            atomicAdd(&S.hc[(cr[k].y >> shift) & mask], 1u);
        __syncthreads();
        // Thread t owns digits 2t, 2t+1 (ascending index order).
        const uint32_t c0 = (2 * tid < nb) ? S.hc[2 * tid] : 0u;
        const uint32_t c1 = (2 * tid + 1 < nb) ? S.hc[2 * tid + 1] : 0u;
        uint32_t tot;
        const uint32_t before = block_exclusive_scan<kResThreads>(c0 + c1, S.uscan, &tot);
        if (c0 && before < (uint64_t)c && before + c0 >= (uint64_t)c) {
            S.chosen = 2 * tid;
            S.chosen_cbefore = before;
        } else if (c1 && before + c0 < (uint64_t)c && before + c0 + c1 >= (uint64_t)c) {
            S.chosen = 2 * tid + 1;
            S.chosen_cbefore = before + c0;
        }
        __syncthreads();
        const uint32_t j = (uint32_t)S.chosen;
        c -= S.chosen_cbefore;
        n = res_filter(cr, n, shift, mask, j, false, true, ir, cnt, S);
    }
    // One token left (its index is fully determined): keep it.
    if (tid == 0 && n > 0 && c > 0) {
        const uint32_t pos = atomicAdd(cnt, 1u);
        ir[pos] = (int32_t)cr[0].y;
    }
}

// ---------------------------------------------------------------- p >= 1

__global__ __launch_bounds__(256) void sel_all_kernel(int N, int32_t *__restrict__ idx,
                                                      int32_t *__restrict__ count)
{
    const int64_t r = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < N) idx[r * (int64_t)N + i] = (int32_t)i;
    if (blockIdx.x == 0 && threadIdx.x == 0) count[r] = N;
}

hipError_t launch_topp_select(const float *scores, int64_t R, int N, float p,
                              int32_t *idx, int32_t *count, void *ws, hipStream_t stream)
{
    if (p >= 1.0f) {
        dim3 grid((unsigned)((N + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(sel_all_kernel, grid, dim3(256), 0, stream, N, idx, count);
        return hipGetLastError();
    }
    SelPtrs P = sel_ptrs(ws, R, N);
    dim3 grid((unsigned)P.nblk, (unsigned)R);
    hipLaunchKernelGGL(sel_max_kernel, grid, dim3(kSelThreads), 0, stream, scores, N, P, count);
    hipLaunchKernelGGL(sel_hist1_kernel, grid, dim3(kSelThreads), 0, stream, scores, N, P);
    hipLaunchKernelGGL(sel_pick1_kernel, dim3((unsigned)R), dim3(kSelThreads), 0, stream, P, p);
    hipLaunchKernelGGL(sel_emit1_kernel, grid, dim3(kSelThreads), 0, stream, scores, N, P, idx, count);
    hipLaunchKernelGGL(sel_resolve_kernel, dim3((unsigned)R), dim3(kResThreads), 0, stream, N, P, idx, count);
    return hipGetLastError();
}

}  // namespace rtp
