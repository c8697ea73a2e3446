// Sort-free top-p selection (gist.science summary of arXiv 2605.16928,
// method section 3: keep adding low-dim attention mass until it reaches p;
// method section 5: a histogram-based, sort-free threshold).
//
// The kept set is the shortest prefix, in descending score order with ties
// to the lower token index, whose mass sum(exp(s - M)) reaches p * Z.  It is
// found exactly, without sorting, as a mass-weighted radix select over the
// 64-bit composite key (order-preserving score key, then token index):
//
//   hist    one block per 8192-score chunk: the chunk max m_b and, per
//           level-1 bin (score key bits [31:20]), the count and the fp64
//           mass exp(s - ref) with ref = the bin's largest representable
//           score (or m_b in the chunk's top bin, so every term is <= 1);
//           written as a compact list of the chunk's non-empty bins
//   pick    one block per row: M = max m_b, the lists merged into one
//           histogram rescaled to exp(s - M), Z, the target p*Z, the
//           boundary bin j1 (the first bin, from the top, where the running
//           mass reaches the target) and the mass A above it
//   emit    tokens in bins above j1 are kept; tokens of bin j1 become
//           candidates (key, index)
//   resolve one block per row: the same step over key bits [19:10], then
//           [9:0] (the boundary is now one score value tau), then how many
//           tokens of score tau are needed and, if not all of them, the
//           lowest indices among them by a count-only radix select over the
//           index bits
//
// Masses are fp64 (exp in fp64, fp64 sums), so running sums agree with an
// fp64 reference to ~1e-16 relative; every rescaling factor is <= 1, so no
// finite input overflows.  HBM traffic: the scores are read twice (hist,
// emit); the lists and candidates are small except for near-flat rows.
#include <float.h>

#include "rtp_device.h"
#include "rtp_launch.h"

namespace rtp {

constexpr int kSelThreads = 256;
constexpr int kSelPerThread = 32;
constexpr int kSelChunk = kSelThreads * kSelPerThread;  // scores per block
constexpr int kBins1 = 4096;
constexpr int kPickThreads = 1024;
constexpr int kPickBatch = 2048;  // chunk lists merged per batch
constexpr int kResThreads = 1024;
constexpr int kResBins = 2048;
constexpr int kResCap = 8192;  // candidates resolved from LDS

struct SelRow {
    double Z;        // sum of exp(s - M) over the row
    double A;        // mass above the level-1 boundary bin
    double T;        // p * Z
    float M;         // row max
    uint32_t j1;     // level-1 boundary bin
    uint32_t n_cand; // candidates appended by emit
    uint32_t pad[7];
};

struct Hist2 {                 // level-2 histogram of the candidates,
    double mass[1024];         // key bits [19:10], mass exp(s - M)
    uint32_t cnt[1024];
};
static_assert(sizeof(SelRow) == 64, "SelRow is one 64-B record");

struct ChunkHdr {
    float m;       // chunk max
    uint32_t n;    // entries in the chunk's bin list
};

struct BinEntry {
    uint32_t bin;
    uint32_t cnt;
    double mass;   // sum of exp(s - ref) over the chunk's tokens in this bin
};

SelLayout sel_layout(int64_t R, int64_t N)
{
    SelLayout L;
    L.nblk = (N + kSelChunk - 1) / kSelChunk;
    size_t off = 0;
    L.rows = off;
    off += align_up((size_t)R * sizeof(SelRow), 256);
    L.hist2 = off;
    off += align_up((size_t)R * sizeof(Hist2), 256);
    L.hdr = off;
    off += align_up((size_t)R * L.nblk * sizeof(ChunkHdr), 256);
    L.lists = off;
    off += align_up((size_t)R * L.nblk * kBins1 * sizeof(BinEntry), 256);
    L.cand = off;
    off += align_up((size_t)R * N * sizeof(uint2), 256);
    L.total = off;
    return L;
}

struct SelPtrs {
    SelRow *rows;
    Hist2 *hist2;
    ChunkHdr *hdr;
    BinEntry *lists;
    uint2 *cand;
    int nblk;
};

static SelPtrs sel_ptrs(void *ws, int64_t R, int64_t N)
{
    SelLayout L = sel_layout(R, N);
    char *base = static_cast<char *>(ws);
    SelPtrs P;
    P.rows = reinterpret_cast<SelRow *>(base + L.rows);
    P.hist2 = reinterpret_cast<Hist2 *>(base + L.hist2);
    P.hdr = reinterpret_cast<ChunkHdr *>(base + L.hdr);
    P.lists = reinterpret_cast<BinEntry *>(base + L.lists);
    P.cand = reinterpret_cast<uint2 *>(base + L.cand);
    P.nblk = (int)L.nblk;
    return P;
}

// Largest finite score whose key lies in level-1 bin `bin` (bins that hold
// finite scores only).
__device__ __forceinline__ float bin_top(uint32_t bin) { return key_score((bin << 20) | 0xFFFFFu); }

// One chunk of a score row in registers.  Full chunks of 16-B aligned rows
// use 16-B loads (slot t of thread x: element c0 + ((t/4)*256 + x)*4 + t%4);
// otherwise slot t is element c0 + t*256 + x.  Missing elements are -inf.
struct ChunkView {
    bool vec;
    int64_t c0;
    __device__ int64_t index(int t) const
    {
        return vec ? c0 + ((int64_t)(t >> 2) * kSelThreads + threadIdx.x) * 4 + (t & 3)
                   : c0 + (int64_t)t * kSelThreads + threadIdx.x;
    }
};

__device__ __forceinline__ ChunkView load_chunk(const float *__restrict__ sr, int N, int64_t c0,
                                                float v[kSelPerThread])
{
    ChunkView cv;
    cv.c0 = c0;
    cv.vec = (c0 + kSelChunk <= N) && ((reinterpret_cast<uintptr_t>(sr + c0) & 15) == 0);
    if (cv.vec) {
        const float4 *p4 = reinterpret_cast<const float4 *>(sr + c0);
#pragma unroll
        for (int k = 0; k < kSelPerThread / 4; ++k) {
            const float4 x = p4[k * kSelThreads + threadIdx.x];
            v[4 * k] = x.x;
            v[4 * k + 1] = x.y;
            v[4 * k + 2] = x.z;
            v[4 * k + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int t = 0; t < kSelPerThread; ++t) {
            const int64_t i = c0 + (int64_t)t * kSelThreads + threadIdx.x;
            v[t] = i < N ? sr[i] : -INFINITY;
        }
    }
    return cv;
}

// --------------------------------------------------------------- hist

__global__ __launch_bounds__(kSelThreads) void sel_hist_kernel(const float *__restrict__ scores,
                                                               int N, SelPtrs P)
{
    __shared__ double hm[kBins1];
    __shared__ uint32_t hc[kBins1];
    __shared__ float red[kSelThreads / kWave];
    __shared__ uint32_t scan[kSelThreads / kWave + 1];
    const int64_t r = blockIdx.y;
    const int blk = blockIdx.x;
    const float *sr = scores + r * (int64_t)N;
    float v[kSelPerThread];
    const ChunkView cv = load_chunk(sr, N, (int64_t)blk * kSelChunk, v);

    for (int i = threadIdx.x; i < kBins1; i += kSelThreads) {
        hm[i] = 0.0;
        hc[i] = 0u;
    }
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < kSelPerThread; ++t) m = fmaxf(m, v[t]);
    m = wave_max(m);
    if (lane_id() == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    float mb = red[0];
    for (int i = 1; i < kSelThreads / kWave; ++i) mb = fmaxf(mb, red[i]);
    const uint32_t tb = score_key(mb) >> 20;
    const double mbd = (double)mb;
#pragma unroll 4
    for (int t = 0; t < kSelPerThread; ++t) {
        if (cv.index(t) < N) {
            const uint32_t bin = score_key(v[t]) >> 20;
            const double ref = bin == tb ? mbd : (double)bin_top(bin);
            atomicAdd(&hm[bin], exp((double)v[t] - ref));
            atomicAdd(&hc[bin], 1u);
        }
    }
    __syncthreads();
    // Compact the non-empty bins into this chunk's list.
    constexpr int kPer = kBins1 / kSelThreads;
    const int b0 = threadIdx.x * kPer;
    uint32_t nz = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) nz += hc[b0 + k] ? 1u : 0u;
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kSelThreads>(nz, scan, &total);
    BinEntry *out = P.lists + (r * P.nblk + blk) * (int64_t)kBins1;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint32_t c = hc[b0 + k];
        if (c) {
            BinEntry e;
            e.bin = (uint32_t)(b0 + k);
            e.cnt = c;
            e.mass = hm[b0 + k];
            out[pos++] = e;
        }
    }
    if (threadIdx.x == 0) {
        ChunkHdr h;
        h.m = mb;
        h.n = total;
        P.hdr[r * P.nblk + blk] = h;
    }
}

// --------------------------------------------------------------- pick

__global__ __launch_bounds__(kPickThreads) void sel_pick_kernel(SelPtrs P, float p,
                                                                int32_t *__restrict__ count)
{
    constexpr int kPer = kBins1 / kPickThreads;  // bins per thread
    constexpr int kNW = kPickThreads / kWave;
    __shared__ double hm[kBins1];
    __shared__ uint32_t hc[kBins1];
    __shared__ double scan[kNW + 1];
    __shared__ float red[kNW];
    __shared__ int chosen;  // highest bin where the running mass crosses T
    __shared__ int lowest;  // lowest non-empty bin
    __shared__ float bm[kPickBatch];
    __shared__ uint32_t bn[kPickBatch], boff[kPickBatch];
    __shared__ uint32_t uscan[kNW + 1];
    const int64_t r = blockIdx.x;
    const ChunkHdr *hr = P.hdr + r * P.nblk;
    const int tid = threadIdx.x;

    float m = -INFINITY;
    for (int k = tid; k < P.nblk; k += kPickThreads) m = fmaxf(m, hr[k].m);
    m = wave_max(m);
    if (lane_id() == 0) red[tid / kWave] = m;
    for (int i = tid; i < kBins1; i += kPickThreads) {
        hm[i] = 0.0;
        hc[i] = 0u;
    }
    for (int i = tid; i < 1024; i += kPickThreads) {
        P.hist2[r].mass[i] = 0.0;
        P.hist2[r].cnt[i] = 0u;
    }
    if (tid == 0) {
        chosen = -1;
        lowest = kBins1;
    }
    __syncthreads();
    float Mf = red[0];
    for (int i = 1; i < kNW; ++i) Mf = fmaxf(Mf, red[i]);
    const double M = (double)Mf;

    // Merge the chunk lists, kPickBatch chunks at a time: their entries are
    // laid end to end and spread evenly over the block.
    for (int k0 = 0; k0 < P.nblk; k0 += kPickBatch) {
        const int nk = min(kPickBatch, P.nblk - k0);
        uint32_t nloc = 0;
        for (int k = tid; k < nk; k += kPickThreads) {
            const ChunkHdr h = hr[k0 + k];
            bm[k] = h.m;
            bn[k] = h.n;
        }
        __syncthreads();
        // Exclusive prefix of list lengths (kPickBatch / kPickThreads per thread).
        constexpr int kPerB = kPickBatch / kPickThreads;
        const int kb = tid * kPerB;
        for (int q = 0; q < kPerB; ++q) nloc += (kb + q < nk) ? bn[kb + q] : 0u;
        uint32_t etot;
        uint32_t pre = block_exclusive_scan<kPickThreads>(nloc, uscan, &etot);
        for (int q = 0; q < kPerB; ++q) {
            if (kb + q < nk) {
                boff[kb + q] = pre;
                pre += bn[kb + q];
            }
        }
        __syncthreads();
        for (uint32_t e = tid; e < etot; e += kPickThreads) {
            int lo = 0, hi = nk - 1;  // last chunk with boff <= e
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (boff[mid] <= e) lo = mid; else hi = mid - 1;
            }
            const BinEntry be =
                P.lists[(r * P.nblk + k0 + lo) * (int64_t)kBins1 + (e - boff[lo])];
            const float mk = bm[lo];
            const uint32_t tb = score_key(mk) >> 20;
            const double ref = be.bin == tb ? (double)mk : (double)bin_top(be.bin);
            atomicAdd(&hm[be.bin], be.mass * exp(ref - M));
            atomicAdd(&hc[be.bin], be.cnt);
        }
        __syncthreads();
    }

    // Thread t owns bins top - t*kPer - [0, kPer): thread order is score order.
    const int top = kBins1 - 1 - tid * kPer;
    double wv[kPer];
    uint32_t c[kPer];
    double local = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        wv[k] = hm[top - k];
        c[k] = hc[top - k];
        local += wv[k];
    }
    double Z;
    const double before = block_exclusive_scan<kPickThreads>(local, scan, &Z);
    const double T = (double)p * Z;
    // Running sums restart from each thread's block prefix, so rounding may
    // show a crossing in two neighbouring threads; the highest bin wins.
    double cum = before;
    int my_cross = -1, my_lowest = -1;
    double cross_before = 0.0, lowest_before = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        if (c[k]) {
            if (my_cross < 0 && cum < T && cum + wv[k] >= T) {
                my_cross = top - k;
                cross_before = cum;
            }
            my_lowest = top - k;
            lowest_before = cum;
        }
        cum += wv[k];
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
        P.rows[r].M = Mf;
        P.rows[r].n_cand = 0u;
        count[r] = 0;
    }
}

// --------------------------------------------------------------- emit

__global__ __launch_bounds__(kSelThreads) void sel_emit_kernel(
    const float *__restrict__ scores, int N, SelPtrs P, int32_t *__restrict__ idx,
    int32_t *__restrict__ count)
{
    __shared__ uint32_t scan[kSelThreads / kWave + 1];
    __shared__ uint32_t base[2];
    const int64_t r = blockIdx.y;
    const uint32_t j1 = P.rows[r].j1;
    const double M = (double)P.rows[r].M;
    const float *sr = scores + r * (int64_t)N;
    int32_t *ir = idx + r * (int64_t)N;
    uint2 *cr = P.cand + r * (int64_t)N;
    Hist2 &h2 = P.hist2[r];
    float v[kSelPerThread];
    const ChunkView cv = load_chunk(sr, N, (int64_t)blockIdx.x * kSelChunk, v);
    // One slot reservation per block and list.
    uint32_t na = 0, nc = 0;
#pragma unroll
    for (int t = 0; t < kSelPerThread; ++t) {
        const uint32_t bin = score_key(v[t]) >> 20;  // missing elements: -inf, bin 7
        const bool valid = cv.index(t) < N;
        na += (valid && bin > j1) ? 1u : 0u;
        nc += (valid && bin == j1) ? 1u : 0u;
    }
    uint32_t ta, tc;
    uint32_t oa = block_exclusive_scan<kSelThreads>(na, scan, &ta);
    uint32_t oc = block_exclusive_scan<kSelThreads>(nc, scan, &tc);
    if (threadIdx.x == 0) {
        base[0] = ta ? atomicAdd(reinterpret_cast<uint32_t *>(count + r), ta) : 0u;
        base[1] = tc ? atomicAdd(&P.rows[r].n_cand, tc) : 0u;
    }
    __syncthreads();
    oa += base[0];
    oc += base[1];
#pragma unroll
    for (int t = 0; t < kSelPerThread; ++t) {
        const uint32_t key = score_key(v[t]);
        const uint32_t bin = key >> 20;
        const int64_t i = cv.index(t);
        if (i < N && bin > j1) ir[oa++] = (int32_t)i;
        if (i < N && bin == j1) {
            cr[oc++] = make_uint2(key, (uint32_t)i);
            const uint32_t d2 = (key >> 10) & 1023u;
            atomicAdd(&h2.mass[d2], exp((double)v[t] - M));
            atomicAdd(&h2.cnt[d2], 1u);
        }
    }
}

// ------------------------------------------------------------ resolve

struct ResShared {
    uint2 cand[kResCap];
    double hm[kResBins];
    uint32_t hc[kResBins];
    double dscan[kResThreads / kWave + 1];
    uint32_t uscan[kResThreads / kWave + 1];
    int chosen;
    double chosen_before;
    uint32_t chosen_cbefore;
    int lowest;
    uint32_t nsurv;
};

// Keeps candidates whose digit equals `keep_digit`, emits those on the kept
// side of it to idx, drops the rest; compacts survivors in place (cr is in
// LDS or global memory).  Returns the survivor count.  emit_above: digits
// above are emitted (score levels); otherwise digits below (index levels).
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

// Chooses the boundary digit of one score level from a histogram held by
// thread t as digit 1023 - t (descending score): the highest digit where
// the running mass crosses T, or, if rounding hides every crossing, the
// lowest non-empty one.  Returns the digit; *A gains the mass above it.
__device__ uint32_t res_choose(double w, uint32_t c, double *A, double T, ResShared &S)
{
    const int tid = threadIdx.x;
    const int dg = 1023 - tid;
    if (tid == 0) {
        S.chosen = -1;
        S.lowest = -1;
    }
    double tot;
    const double before = block_exclusive_scan<kResThreads>(w, S.dscan, &tot);
    const double x = *A + before;
    if (c && x < T && x + w >= T) atomicMax(&S.chosen, dg);
    if (c) atomicMax(&S.lowest, tid);
    __syncthreads();
    if (S.chosen < 0 && tid == S.lowest) S.chosen = dg;
    __syncthreads();
    if (dg == S.chosen) S.chosen_before = before;
    __syncthreads();
    const uint32_t j = (uint32_t)S.chosen;
    *A += S.chosen_before;
    __syncthreads();
    return j;
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
    const int64_t n1 = row.n_cand;
    uint2 *gc = P.cand + r * (int64_t)N;
    int32_t *ir = idx + r * (int64_t)N;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(count + r);
    const int tid = threadIdx.x;
    if (n1 == 0) return;

    // Level 2 (key bits [19:10]): the histogram was built by emit.
    const int d2 = 1023 - tid;
    const uint32_t j2 = res_choose(P.hist2[r].mass[d2], P.hist2[r].cnt[d2], &A, T, S);
    const int64_t n2 = P.hist2[r].cnt[j2];
    // One pass over the candidates: digits above j2 are kept, digit j2
    // survives (into LDS when it fits, else compacted in place).
    uint2 *cr;
    int64_t n;
    if (n2 <= kResCap) {
        if (tid == 0) S.nsurv = 0u;
        __syncthreads();
        for (int64_t c0 = 0; c0 < n1; c0 += kResThreads) {
            const int64_t k = c0 + tid;
            const bool valid = k < n1;
            const uint2 e = valid ? gc[k] : make_uint2(0, 0);
            const uint32_t dg = (e.x >> 10) & 1023u;
            const int64_t pa = wave_append(valid && dg > j2, cnt);
            if (pa >= 0) ir[pa] = (int32_t)e.y;
            const int64_t ps = wave_append(valid && dg == j2, &S.nsurv);
            if (ps >= 0) S.cand[ps] = e;
        }
        __syncthreads();
        cr = S.cand;
        n = S.nsurv;
    } else {
        cr = gc;
        n = res_filter(gc, n1, 10, 1023u, j2, true, false, ir, cnt, S);
    }

    // Level 3 (key bits [9:0]).
    if (n > 0) {
        for (int i = tid; i < 1024; i += kResThreads) {
            S.hm[i] = 0.0;
            S.hc[i] = 0u;
        }
        __syncthreads();
        for (int64_t k = tid; k < n; k += kResThreads) {
            const uint32_t key = cr[k].x;
            const uint32_t dg = key & 1023u;
            atomicAdd(&S.hm[dg], exp((double)key_score(key) - M));
            atomicAdd(&S.hc[dg], 1u);
        }
        __syncthreads();
        const uint32_t j3 = res_choose(S.hm[1023 - tid], S.hc[1023 - tid], &A, T, S);
        n = res_filter(cr, n, 0, 1023u, j3, true, false, ir, cnt, S);
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
        return launch(sel_all_kernel, grid, dim3(256), 0, stream, N, idx, count);
    }
    SelPtrs P = sel_ptrs(ws, R, N);
    dim3 grid((unsigned)P.nblk, (unsigned)R);
    RTP_TRY(launch(sel_hist_kernel, grid, dim3(kSelThreads), 0, stream, scores, N, P));
    RTP_TRY(launch(sel_pick_kernel, dim3((unsigned)R), dim3(kPickThreads), 0, stream, P, p,
                   count));
    RTP_TRY(launch(sel_emit_kernel, grid, dim3(kSelThreads), 0, stream, scores, N, P, idx,
                   count));
    return launch(sel_resolve_kernel, dim3((unsigned)R), dim3(kResThreads), 0, stream, N, P,
                  idx, count);
}

}  // namespace rtp
