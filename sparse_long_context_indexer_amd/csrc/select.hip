// Sort-free top-p selection (gist.science summary of arXiv 2605.16928,
// method section 3: keep adding low-dim attention mass until it reaches p;
// method section 5: a histogram-based, sort-free threshold).
//
// The kept set is the shortest prefix, in descending score order with ties
// to the lower token index, whose mass sum(exp(s - M)) reaches p * Z.  It is
// found exactly, without sorting, as a mass-weighted radix select over the
// 64-bit composite key (order-preserving score key, then token index):
//
//   hist    one block per 32768-score chunk: per level-1 bin (score key bits
//           [31:20], 4096 bins) the fp64 mass exp(s - top(bin)), top(bin)
//           being the bin's largest representable score, merged into the
//           row's histogram with global atomics; the chunk's own top bin is
//           kept apart, as mass exp(s - m_b) with m_b the chunk max, so every
//           term is <= 1 and nothing overflows for any finite input.  Block 0
//           of each row first clears the row's state.
//   emit    every block first derives its row's threshold from the finished
//           histogram (the pick): M = max m_b, the histogram rescaled to
//           exp(s - M), Z, the target p*Z, the boundary bin j1 (the highest
//           bin whose running mass from the top reaches the target) and the
//           mass A above it.  The same inputs and arithmetic give every block
//           of a row the same result, and the histogram loads overlap the
//           chunk's score loads.  Tokens in bins above j1 are kept; tokens of
//           bin j1 become candidates (key, index) and are counted by key bits
//           [19:10].  The row's last block to finish then resolves: the same
//           step over key bits [19:10]; when at most 64 candidates share the
//           boundary digit, one wave ranks them by (score, index) and keeps
//           the shortest rank prefix outright; otherwise the step runs again
//           over [9:0] (the boundary is now one score value tau), then
//           decides how many tokens of score tau are needed and, if not all
//           of them, takes the lowest indices among them by a count-only
//           radix select over the index bits
//
// Masses are fp64 (exp_tang, a table-driven fp64 exp within 1.3 ulp, and
// fp64 sums), so running sums agree with an fp64 reference to ~1e-15
// relative.  HBM traffic: the scores are read twice (hist, emit);
// candidates are few except for near-flat rows.
#include <float.h>

#include "rtp_device.h"
#include "rtp_exp.h"
#include "rtp_launch.h"

namespace rtp {

constexpr int kSelThreads = 1024;
constexpr int kSelPerThread = 32;
constexpr int kSelChunk = kSelThreads * kSelPerThread;  // scores per block
constexpr int kShift1 = 20;                  // level-1 bin = score key bits [31:20]
constexpr int kBins1 = 1 << (32 - kShift1);  // 4096 bins
constexpr int kShift2 = 10;                  // refinement digits: key bits [19:10], [9:0]
constexpr int kDig = 1 << kShift2;           // 1024 digits per refinement level
constexpr int kResThreads = 1024;
constexpr int kResBins = 2048;
constexpr int kResCap = 8192;  // candidates resolved from LDS (two buffers)

struct SelRow {
    uint64_t slots;      // emit's slot counters: kept (high 32 bits), candidates (low)
    uint32_t hist_done;  // hist blocks finished
    uint32_t emit_done;  // emit blocks finished
    unsigned long long ready;  // tagged: the row's state below was cleared
    uint32_t kept1;      // tokens kept by the emit blocks (published for attention blocks)
    uint32_t pad[9];
};
static_assert(sizeof(SelRow) == 64, "SelRow is one 64-B record");

struct Hist1 {                 // level-1 histogram of one row; masses are
    double mass[kBins1];       // relative to each bin's top score
};

struct Hist2 {                 // the boundary bin's candidates by key bits
    double mass[kDig];         // [19:10]: mass exp(s - M) and count, built
    uint32_t cnt[kDig];        // by the emit blocks
};

struct ChunkTop {              // a chunk's top bin, kept out of Hist1
    float m;                   // chunk max
    uint32_t pad;
    double mass;               // sum of exp(s - m) over its tokens in that bin
};

SelLayout sel_layout(int64_t R, int64_t N)
{
    SelLayout L;
    L.nblk = (N + kSelChunk - 1) / kSelChunk;
    size_t off = 0;
    L.rows = off;
    off += align_up((size_t)R * sizeof(SelRow), 256);
    L.hist1 = off;
    off += align_up((size_t)R * sizeof(Hist1), 256);
    L.hist2 = off;
    off += align_up((size_t)R * sizeof(Hist2), 256);
    L.tops = off;
    off += align_up((size_t)R * L.nblk * sizeof(ChunkTop), 256);
    L.cand = off;
    off += align_up((size_t)R * N * sizeof(uint2), 256);
    L.total = off;
    return L;
}

struct SelPtrs {
    SelRow *rows;
    Hist1 *hist1;
    Hist2 *hist2;
    ChunkTop *tops;
    uint2 *cand;
    int nblk;
    WaitCtl wc;  // poll limit of the waits on earlier blocks, and where a give-up is reported
};

static SelPtrs sel_ptrs(void *ws, int64_t R, int64_t N)
{
    SelLayout L = sel_layout(R, N);
    char *base = static_cast<char *>(ws);
    SelPtrs P;
    P.rows = reinterpret_cast<SelRow *>(base + L.rows);
    P.hist1 = reinterpret_cast<Hist1 *>(base + L.hist1);
    P.hist2 = reinterpret_cast<Hist2 *>(base + L.hist2);
    P.tops = reinterpret_cast<ChunkTop *>(base + L.tops);
    P.cand = reinterpret_cast<uint2 *>(base + L.cand);
    P.nblk = (int)L.nblk;
    return P;
}

// Candidates (key, index) cross from the emit blocks to the row's resolving
// block through agent-scope 8-byte accesses.
__device__ __forceinline__ uint2 ld_cand(const uint2 *p)
{
    const unsigned long long v = ld_agent(reinterpret_cast<const unsigned long long *>(p));
    return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
__device__ __forceinline__ void st_cand(uint2 *p, uint2 e)
{
    st_agent(reinterpret_cast<unsigned long long *>(p),
             (unsigned long long)e.x | ((unsigned long long)e.y << 32));
}

// Largest finite score whose key lies in level-1 bin `bin` (bins that hold
// finite scores only).
__device__ __forceinline__ float bin_top(uint32_t bin)
{
    return key_score((bin << kShift1) | ((1u << kShift1) - 1u));
}

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
    // The same in 32 bits (token indices are below N <= INT32_MAX).
    __device__ uint32_t index32(int t) const
    {
        const uint32_t c = (uint32_t)c0;
        return vec ? c + ((uint32_t)(t >> 2) * kSelThreads + threadIdx.x) * 4u + (uint32_t)(t & 3)
                   : c + (uint32_t)t * kSelThreads + threadIdx.x;
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

// ----------------------------------------------------- row state
//
// Block 0 of each row's hist grid clears the row's state (histograms,
// counters) at the start of a call and then counts itself on the row's
// tagged `ready` counter; the row's other blocks wait for it before their
// first global add, which comes after their whole LDS pass, so the wait is
// almost always already over.  Block 0 is dispatched before the row's other
// blocks (it has the lowest index), so the wait always ends.  The row's
// last hist block resets `ready` for the next call.

__device__ __forceinline__ void clear_row(SelPtrs P, int64_t r)
{
    Hist1 &g = P.hist1[r];
    Hist2 &h2 = P.hist2[r];
    for (int i = threadIdx.x; i < kBins1; i += kSelThreads) st_agent(&g.mass[i], 0.0);
    for (int i = threadIdx.x; i < kDig; i += kSelThreads) {
        st_agent(&h2.mass[i], 0.0);
        st_agent(&h2.cnt[i], 0u);
    }
    if (threadIdx.x == 0) {
        st_agent(reinterpret_cast<unsigned long long *>(&P.rows[r].slots), 0ull);
        st_agent(&P.rows[r].hist_done, 0u);
        st_agent(&P.rows[r].emit_done, 0u);
    }
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) ctr_add(&P.rows[r].ready, 1u);
}

// Every block waited for below was dispatched before the waiting one (block
// 0 of the row; in the one-launch selection, the row's histogram blocks);
// waits are bounded by wc.limit polls, and a give-up is reported in the
// library's status word.

// Waits until the row's tagged `ready` counter holds at least `level`: 1
// once block 0 has cleared the row, 2 once the row's Hist1 is complete
// (one-launch selection only).
__device__ __forceinline__ void wait_row_ready(const SelRow &row, uint32_t level, const WaitCtl &wc)
{
    for (uint32_t it = 0;; ++it) {
        const unsigned long long v = ld_agent(&row.ready);
        if ((uint32_t)v == kCtrTag && (uint32_t)(v >> 32) >= level) return;
        if (it >= wc.limit) {
            report_timeout(wc);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// --------------------------------------------------------------- hist

// 2^(j/64) for exp_tang; each kernel copies it to LDS.
__constant__ double kExp2Tbl[kExpTable] = RTP_EXP2_TABLE;

// A token's weight in the running sums: its mass exp(x) (x = its score
// minus a reference) for top-p; 1 for top-k, whose prefixes count tokens.
template <bool kCount>
__device__ __forceinline__ double weight(double x, const double *etbl)
{
    if constexpr (kCount)
        return 1.0;
    else
        return exp_tang(x, etbl);
}

struct HistShared {
    double hm[kBins1];
    double etbl[kExpTable];
    float red[kSelThreads / kWave];
};

// The level-1 histogram of one chunk (scores in v): accumulated in LDS (hm,
// kBins1 doubles; etbl receives the exp table; red kSelThreads/kWave
// floats), then added to the row's Hist1 once block 0 has cleared it, and
// the chunk's top-bin record stored.  Leaves the block's arrival to the
// caller.
template <bool kCount>
__device__ __forceinline__ void hist_body(const float (&v)[kSelPerThread], const ChunkView &cv, int N, int64_t r,
                          int blk, SelPtrs P, double *hm, double *etbl, float *red)
{
    for (int i = threadIdx.x; i < kBins1; i += kSelThreads) hm[i] = 0.0;
    if (threadIdx.x < kExpTable) etbl[threadIdx.x] = kExp2Tbl[threadIdx.x];
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < kSelPerThread; ++t) m = fmaxf(m, v[t]);
    m = wave_max(m);
    if (lane_id() == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    float mb = red[0];
    for (int i = 1; i < kSelThreads / kWave; ++i) mb = fmaxf(mb, red[i]);
    const uint32_t tb = score_key(mb) >> kShift1;
    // s - ref is exact in fp32: a bin's scores and its reference share one
    // sign and binade.  A slot past the end of the row (-inf) has a NaN
    // reference, and exp_tang gives NaN +0.
    // A bin's top score shares the sign and the bits above kShift1 with
    // every score of the bin: the low bits all set for a positive score,
    // all clear for a negative one.
    // Block 0 of the row has usually cleared the row by mid-way through this
    // loop: thread 0 reads `ready` there, so that the wait after the loop
    // normally costs no round trip.
    unsigned long long rdy = 0;
#pragma unroll
    for (int t = 0; t < kSelPerThread; ++t) {
        if (t == kSelPerThread / 2 && blk != 0 && threadIdx.x == 0)
            rdy = ld_agent(&P.rows[r].ready);
        const uint32_t u = __float_as_uint(v[t] + 0.0f);  // -0 folded into +0
        const uint32_t sm = (uint32_t)((int32_t)u >> 31);
        const uint32_t bin = (u ^ (sm | 0x80000000u)) >> kShift1;  // score_key(v) >> kShift1
        constexpr uint32_t kLow = (1u << kShift1) - 1u;
        const uint32_t top = (u | (kLow & ~sm)) & ~(kLow & sm);      // bin_top(bin)
        const float ref = bin == tb ? mb : __uint_as_float(top);
        if constexpr (kCount)
            atomicAdd(&hm[bin], cv.vec || cv.index32(t) < (uint32_t)N ? 1.0 : 0.0);
        else
            atomicAdd(&hm[bin], exp_tang((double)(v[t] - ref), etbl));
    }
    if (blk != 0 && threadIdx.x == 0 && !((uint32_t)rdy == kCtrTag && (rdy >> 32) >= 1))
        wait_row_ready(P.rows[r], 1u, P.wc);
    __syncthreads();
    Hist1 &g = P.hist1[r];
    for (int i = threadIdx.x; i < kBins1; i += kSelThreads) {
        const double w = hm[i];
        if (w > 0.0 && (uint32_t)i != tb) atomicAdd(&g.mass[i], w);
    }
    if (threadIdx.x == 0) {
        ChunkTop &t = P.tops[r * P.nblk + blk];
        st_agent(&t.m, mb);
        st_agent(&t.mass, hm[tb]);
    }
}

template <bool kCount>
__global__ __launch_bounds__(kSelThreads) void sel_hist_kernel(const float *__restrict__ scores,
                                                               int N, SelPtrs P)
{
    __shared__ HistShared S;
    const int64_t r = blockIdx.y;
    const int blk = blockIdx.x;
    float v[kSelPerThread];
    const ChunkView cv =
        load_chunk(scores + r * (int64_t)N, N, (int64_t)blk * kSelChunk, v);  // missing: -inf
    if (blk == 0) clear_row(P, r);
    hist_body<kCount>(v, cv, N, r, blk, P, S.hm, S.etbl, S.red);
    // Every block of the row has passed its wait once all have counted
    // themselves here, so the last one resets `ready` for the next call.
    if (threadIdx.x == 0 &&
        atomicAdd(&P.rows[r].hist_done, 1u) == (uint32_t)(P.nblk - 1))
        ctr_reset(&P.rows[r].ready);
}

// --------------------------------------------------------------- emit

struct ResShared;
template <bool kCount, bool kVis = false>
__device__ __forceinline__ void resolve_row(int N, SelPtrs P, int64_t r, int32_t *idx, int32_t *count,
                            uint32_t *kbr, ResShared &S);

// ------------------------------------------------------------ resolve
//
// One block per row.  Kept tokens are appended to idx behind the ones emit
// wrote, through a block-local slot counter, and the row's count is written
// once at the end.  Each level: a histogram of the surviving candidates in
// LDS, the boundary digit chosen by a single wave (a wave-wide scan, no
// block barrier), then one pass that emits the digits on the kept side and
// moves the boundary digit's candidates to the other LDS buffer (order is
// free: the kept set is a set).  Rows with more candidates than fit in LDS
// use global memory with ordered in-place compaction instead.  A boundary
// digit of at most one wave of candidates is finished by that wave alone,
// with no further block barrier.

constexpr int kResNW = kResThreads / kWave;

struct ResShared {
    // The pick's level-1 histogram (aliased), then emit's candidate stage,
    // then the resolve's candidate buffers.
    uint2 buf[2][kResCap];
    double etbl[kExpTable];
    double hm[kResBins];
    uint32_t hc[kResBins];
    uint32_t uscan[kResNW + 1];
    double dscan[kResNW + 1];
    float red[kResNW];
    // pick: per wave, its first crossing bin and its last bin with mass
    int wcross[kResNW], wlow[kResNW];
    double wcross_before[kResNW], wlow_before[kResNW];
    // The row's threshold (the same in every block of the row)
    float M;      // row max
    uint32_t j1;  // level-1 boundary bin
    double A;     // mass above bin j1
    double T;     // p * Z
    // Two counters in one word, so a wave reserves both with one atomic:
    // tokens kept by this block so far (low half) and candidates moved to
    // the other buffer (high half).
    unsigned long long nn;
    uint32_t j;      // chosen digit
    uint32_t cbefore;
    double abefore;  // A plus the mass above the chosen digit
    // emit's own use of the block's LDS
    unsigned long long wbase[kSelThreads / kWave];
    unsigned long long bcount, gbase;
    int last;
};
static_assert(sizeof(double) * kBins1 <= sizeof(uint2) * kResCap, "pick histogram fits in buf");

// --------------------------------------------------------------- pick
//
// The row's threshold from its finished level-1 histogram (g) and chunk
// tops; gmv holds this thread's bins tid + k*kSelThreads, tm0/tmass0 the
// top of chunk tid (when tid < nblk).  Leaves M, T, j1 and A in S.
constexpr int kPickPer = kBins1 / kSelThreads;  // bins per thread

template <bool kCount>
__device__ __forceinline__ void pick_block(const ChunkTop *tops, int nblk, double target,
                           const double (&gmv)[kPickPer], float tm0, double tmass0, ResShared &S)
{
    double *hm = reinterpret_cast<double *>(&S.buf[0][0]);
    const int tid = threadIdx.x;
    float m = tm0;
    for (int k = tid + kSelThreads; k < nblk; k += kSelThreads) m = fmaxf(m, tops[k].m);
    m = wave_max(m);
    if (lane_id() == 0) S.red[tid / kWave] = m;
    __syncthreads();
    float Mf = S.red[0];
    for (int i = 1; i < kResNW; ++i) Mf = fmaxf(Mf, S.red[i]);
    const double M = (double)Mf;
    // A bin counted in Hist1 lies below some chunk's top bin, so its top
    // score is below M: every factor is <= 1.
#pragma unroll
    for (int k = 0; k < kPickPer; ++k) {
        const int i = tid + k * kSelThreads;
        hm[i] = gmv[k] > 0.0 ? gmv[k] * weight<kCount>((double)bin_top(i) - M, S.etbl) : 0.0;
    }
    __syncthreads();
    if (tid < nblk)
        atomicAdd(&hm[score_key(tm0) >> kShift1], tmass0 * weight<kCount>((double)tm0 - M, S.etbl));
    for (int k = tid + kSelThreads; k < nblk; k += kSelThreads) {
        const float tm = tops[k].m;
        atomicAdd(&hm[score_key(tm) >> kShift1],
                  tops[k].mass * weight<kCount>((double)tm - M, S.etbl));
    }
    __syncthreads();

    // Thread t owns bins top - t*kPickPer - [0, kPickPer): thread order is
    // score order.
    const int top = kBins1 - 1 - tid * kPickPer;
    double wv[kPickPer];
    double local = 0.0;
#pragma unroll
    for (int k = 0; k < kPickPer; ++k) {
        wv[k] = hm[top - k];
        local += wv[k];
    }
    double Z;
    const double before = block_exclusive_scan<kSelThreads, double, false>(local, S.dscan, &Z);
    // top-p: p * Z; top-k: k (Z is then the row's token count).
    const double T = kCount ? target : target * Z;
    // The boundary is the highest bin with mass whose running sum (every bin
    // down to and including it) reaches T; each thread tests its own bins,
    // so no rounding of the block prefix can skip it.  If the total stays
    // below T, the lowest bin with mass.  Bins whose mass underflows to 0
    // hold nothing a prefix can need.
    double cum = before;
    int my_cross = -1, my_lowest = -1;
    double cross_before = 0.0, lowest_before = 0.0;
#pragma unroll
    for (int k = 0; k < kPickPer; ++k) {
        if (wv[k] > 0.0) {
            if (my_cross < 0 && cum + wv[k] >= T) {
                my_cross = top - k;
                cross_before = cum;
            }
            my_lowest = top - k;
            lowest_before = cum;
        }
        cum += wv[k];
    }
    // Thread order is score order: the highest crossing bin belongs to the
    // first thread with a crossing, the lowest bin with mass to the last
    // thread with mass.  Each wave reports its own first / last such lane.
    const int lane = lane_id(), w = tid / kWave;
    const uint64_t cm = __ballot(my_cross >= 0);
    const uint64_t lm = __ballot(my_lowest >= 0);
    if (lane == 0) {
        S.wcross[w] = -1;
        S.wlow[w] = -1;
    }
    if (cm && lane == __ffsll((unsigned long long)cm) - 1) {
        S.wcross[w] = my_cross;
        S.wcross_before[w] = cross_before;
    }
    if (lm && lane == 63 - __clzll((unsigned long long)lm)) {
        S.wlow[w] = my_lowest;
        S.wlow_before[w] = lowest_before;
    }
    __syncthreads();
    if (w == 0) {
        // Lane i looks at wave i's reports; the first wave with a crossing,
        // else the last wave with mass.
        const bool hc = lane < kResNW && S.wcross[lane] >= 0;
        const bool hl = lane < kResNW && S.wlow[lane] >= 0;
        const uint64_t cb = __ballot(hc), lb = __ballot(hl);
        if (lane == 0) {
            if (cb) {
                const int wc = __ffsll((unsigned long long)cb) - 1;
                S.j1 = (uint32_t)S.wcross[wc];
                S.A = S.wcross_before[wc];
            } else if (lb) {
                const int wl = 63 - __clzll((unsigned long long)lb);
                S.j1 = (uint32_t)S.wlow[wl];
                S.A = S.wlow_before[wl];
            } else {
                S.j1 = 0u;
                S.A = 0.0;
            }
            S.T = T;
            S.M = Mf;
        }
    }
    __syncthreads();
}

// Wave 0 chooses the boundary digit of a score level from S.hm/S.hc over
// digits 0..kDig-1: the highest non-empty digit whose running mass (A plus
// every digit down to and including it) reaches T -- a test no rounding of
// the parallel prefix can skip -- or, if the total stays below T, the
// lowest non-empty digit.  Lane l owns digits kDig - 1 - 16l - [0, 16); it
// reads them into registers once and decides with selects.
__device__ __forceinline__ void res_choose_mass(double A, double T, ResShared &S)
{
    const int lane = lane_id();
    constexpr int kPerLane = kDig / kWave;
    const int top = kDig - 1 - kPerLane * lane;
    double wv[kPerLane];
    uint32_t cv[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        wv[k] = S.hm[top - k];
        cv[k] = S.hc[top - k];
    }
    double local = 0.0;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) local += wv[k];
    const double inc = wave_inclusive_scan(local);
    double cum = A + (inc - local);
    int cross = -1, low = -1;
    double cross_b = 0.0, low_b = 0.0;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const bool ne = cv[k] != 0u;
        const bool hit = ne && cross < 0 && cum + wv[k] >= T;
        cross = hit ? top - k : cross;
        cross_b = hit ? cum : cross_b;
        low = ne ? top - k : low;
        low_b = ne ? cum : low_b;
        cum += wv[k];
    }
    // Highest crossing digit = lowest lane with a crossing; else the lowest
    // non-empty digit = highest lane with one.
    const uint64_t cm = __ballot(cross >= 0);
    if (cm) {
        const int src = __ffsll((unsigned long long)cm) - 1;
        if (lane == src) {
            S.j = (uint32_t)cross;
            S.abefore = cross_b;
        }
    } else {
        const uint64_t lm = __ballot(low >= 0);
        const int src = 63 - __clzll((unsigned long long)lm);
        if (lane == src) {
            S.j = (uint32_t)low;
            S.abefore = low_b;
        }
    }
}

// Wave 0 chooses the index digit holding the c-th lowest index over nb
// digits (ascending); lane l owns digits [l*per, (l+1)*per).
__device__ __forceinline__ void res_choose_count(uint32_t c, int nb, ResShared &S)
{
    const int lane = lane_id();
    const int per = nb / kWave;
    const int d0 = lane * per;
    uint32_t local = 0;
    for (int k = 0; k < per; ++k) local += S.hc[d0 + k];
    const uint32_t inc = wave_inclusive_scan(local);
    uint32_t cum = inc - local;
    for (int k = 0; k < per; ++k) {
        const uint32_t w = S.hc[d0 + k];
        if (w && cum < c && cum + w >= c) {
            S.j = (uint32_t)(d0 + k);
            S.cbefore = cum;
        }
        cum += w;
    }
}

// Appends token i to the row's kept list at slot pa (with kVis an
// agent-scope store: other blocks of the same launch read it) and, when the
// row has a keep bitmap, sets its bit (the emit blocks wrote the bitmap's
// words with agent-scope stores before the resolve started).
template <bool kVis>
__device__ __forceinline__ void keep_token(int32_t *ir, int64_t pa, uint32_t i, uint32_t *kbr)
{
    if constexpr (kVis)
        st_agent(reinterpret_cast<uint32_t *>(ir + pa), i);
    else
        ir[pa] = (int32_t)i;
    if (kbr) atomicOr(kbr + (i >> 5), 1u << (i & 31u));
}

// The kept-token counter (the low half of S.nn).
__device__ __forceinline__ uint32_t *nout_ptr(ResShared &S) { return reinterpret_cast<uint32_t *>(&S.nn); }

// Ordered in-place filter for candidates in global memory (see the header
// comment); survivors keep their relative order.
template <bool kVis>
__device__ __forceinline__ int64_t res_filter_global(uint2 *cr, int64_t n, int shift, uint32_t mask,
                                     uint32_t keep_digit, bool emit_above, bool by_index,
                                     int32_t *ir, uint32_t *kbr, ResShared &S)
{
    int64_t kept_total = 0;
    for (int64_t c0 = 0; c0 < n; c0 += kResThreads) {
        const int64_t k = c0 + threadIdx.x;
        const bool valid = k < n;
        uint2 e = valid ? ld_cand(cr + k) : make_uint2(0, 0);
        const uint32_t field = by_index ? e.y : e.x;
        const uint32_t dg = (field >> shift) & mask;
        const bool out = valid && (emit_above ? dg > keep_digit : dg < keep_digit);
        const bool keep = valid && dg == keep_digit;
        const int64_t pa = wave_append(out, nout_ptr(S));
        if (pa >= 0) keep_token<kVis>(ir, pa, e.y, kbr);
        uint32_t tot;
        const uint32_t pos = block_exclusive_scan<kResThreads>((uint32_t)keep, S.uscan, &tot);
        // All reads of this chunk are done (the scan synchronised the block),
        // and survivors land at or below their read position.
        if (keep) st_cand(cr + kept_total + pos, e);
        kept_total += tot;
        __syncthreads();
    }
    return kept_total;
}

// One pass over n candidates in src (LDS, or global memory when kGlobal):
// emits the kept side of digit j, moves digit j's candidates to dst (LDS,
// which must hold them).  Returns the number moved.  Each thread takes kB
// candidates at a time; a wave reserves the slots of all of them with one
// LDS atomic (both counts packed in 16-bit halves, which never carry: a
// wave holds at most 64 * kB of each).
// With acc_next, the moved candidates' histogram over key bits [9:0]
// (mass exp(s - M) and count) is built in S.hm / S.hc on the way, for the
// next score level.
template <bool kGlobal, bool kCount, bool kVis = false>
__device__ __forceinline__ uint32_t res_filter_lds(const uint2 *src, int64_t n, uint2 *dst, int shift,
                                   uint32_t mask, uint32_t j, bool emit_above, bool by_index,
                                   int32_t *ir, uint32_t *kbr, ResShared &S,
                                   bool acc_next = false, double M = 0.0)
{
    // From global memory, kB loads per thread are in flight before any is used.
    constexpr int kB = kGlobal ? 10 : 4;
    static_assert(kWave * kB < 65536, "per-wave counts fit in 16 bits");
    static_assert(kResThreads == kDig, "one digit per thread");
    if (threadIdx.x == 0) S.nn &= 0xFFFFFFFFull;  // no candidates moved yet
    __syncthreads();  // every thread has read what it needed of S.hm / S.hc
    if (acc_next) {
        S.hm[threadIdx.x] = 0.0;
        S.hc[threadIdx.x] = 0u;
        __syncthreads();
    }
    for (int64_t c0 = 0; c0 < n; c0 += (int64_t)kResThreads * kB) {
        uint2 e[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int64_t k = c0 + (int64_t)u * kResThreads + threadIdx.x;
            e[u] = k < n ? (kGlobal ? ld_cand(src + k) : src[k]) : make_uint2(0, 0);
        }
        uint32_t outm = 0, keepm = 0;  // bit u: candidate u is emitted / moved
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const bool valid = c0 + (int64_t)u * kResThreads + threadIdx.x < n;
            const uint32_t dg = ((by_index ? e[u].y : e[u].x) >> shift) & mask;
            outm |= (valid && (emit_above ? dg > j : dg < j)) ? (1u << u) : 0u;
            keepm |= (valid && dg == j) ? (1u << u) : 0u;
        }
        const uint32_t mine = (uint32_t)__popc(outm) | ((uint32_t)__popc(keepm) << 16);
        const uint32_t inc = wave_inclusive_scan(mine);
        const uint32_t wtot = read_lane(inc, kWave - 1);
        unsigned long long base = 0;
        if (wtot && lane_id() == 0)
            base = atomicAdd(&S.nn, (unsigned long long)(wtot & 0xFFFFu) |
                                        ((unsigned long long)(wtot >> 16) << 32));
        base = read_lane(base, 0);
        const uint32_t ex = inc - mine;
        uint32_t pa = (uint32_t)base + (ex & 0xFFFFu);
        uint32_t pk = (uint32_t)(base >> 32) + (ex >> 16);
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (outm & (1u << u)) keep_token<kVis>(ir, pa++, e[u].y, kbr);
            if (keepm & (1u << u)) {
                dst[pk++] = e[u];
                if (acc_next) {
                    const uint32_t d1 = e[u].x & (uint32_t)(kDig - 1);
                    atomicAdd(&S.hm[d1], weight<kCount>((double)key_score(e[u].x) - M, S.etbl));
                    atomicAdd(&S.hc[d1], 1u);
                }
            }
        }
    }
    __syncthreads();
    return (uint32_t)(S.nn >> 32);
}

// Wave 0 finishes a row whose last n <= kWave candidates sit in LDS: lane l
// ranks candidate l against the others (score descending, then index
// ascending: the order of the sorted definition), the masses exp(s - M) are
// laid out in rank order and prefix-summed from A, and the wave keeps the
// shortest rank prefix whose running mass reaches T (all n if none does).
template <bool kCount, bool kVis = false>
__device__ __forceinline__ void resolve_few(const uint2 *cr, int n, double A, double T, double M, int32_t *ir,
                            uint32_t *kbr, ResShared &S)
{
    const int l = lane_id();
    const bool v = l < n;
    const uint2 e = v ? cr[l] : make_uint2(0u, 0u);
    int rank = 0;
    for (int k = 0; k < n; ++k) {
        const uint32_t kk = read_lane(e.x, k), ki = read_lane(e.y, k);
        rank += (kk > e.x || (kk == e.x && ki < e.y)) ? 1 : 0;
    }
    // Only this wave uses S.hm until the block's next barrier; its LDS
    // accesses complete in program order.
    if (v) S.hm[rank] = weight<kCount>((double)key_score(e.x) - M, S.etbl);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const double w = v ? S.hm[l] : 0.0;
    const double cum = A + wave_inclusive_scan(w);
    const uint64_t hit = __ballot(v && cum >= T);
    const int last = hit ? __ffsll((unsigned long long)hit) - 1 : n - 1;
    const int64_t pa = wave_append(v && rank <= last, nout_ptr(S));
    if (pa >= 0) keep_token<kVis>(ir, pa, e.y, kbr);
}

template <bool kCount, bool kVis>
__device__ __forceinline__ void resolve_row(int N, SelPtrs P, int64_t r, int32_t *idx, int32_t *count,
                            uint32_t *kbr, ResShared &S)
{
    __syncthreads();  // emit is done with the shared words it used
    const SelRow &row = P.rows[r];
    const int tid = threadIdx.x;
    uint2 *gc = P.cand + r * (int64_t)N;
    // The emit totals and the level-2 histogram are requested together.
    const unsigned long long slots =
        ld_agent(reinterpret_cast<const unsigned long long *>(&row.slots));
    const double h2m = ld_agent(&P.hist2[r].mass[tid]);
    const uint32_t h2c = ld_agent(&P.hist2[r].cnt[tid]);
    const double M = (double)S.M;
    const double T = S.T;
    double A = S.A;
    int64_t n = (uint32_t)slots;
    const uint32_t emitted = (uint32_t)(slots >> 32);  // kept by emit
    int32_t *ir = idx + r * (int64_t)N + emitted;
    bool in_lds = false;  // candidates start in global memory
    int cur = 0;          // LDS buffer holding them once they fit
    if (tid == 0) S.nn = 0ull;
    const uint2 *cr = gc;
    // Candidate k from LDS, or from global memory.
    auto cand = [&](int64_t k) { return in_lds ? cr[k] : ld_cand(cr + k); };

    // Score levels: key bits [19:10] (histogram built by the emit blocks),
    // then [9:0] (histogram of the survivors).
    static_assert(kResThreads == kDig, "one digit per thread");
    bool next_built = false;  // level 1's histogram was built by level 0's filter
    bool few = false;         // at most a wave of candidates left, in LDS
    for (int level = 0; level < 2 && n > 0 && !few; ++level) {
        const int shift = level == 0 ? kShift2 : 0;
        if (level == 0) {
            S.hm[tid] = h2m;
            S.hc[tid] = h2c;
            __syncthreads();
        } else if (!next_built) {
            S.hm[tid] = 0.0;
            S.hc[tid] = 0u;
            __syncthreads();
            for (int64_t k = tid; k < n; k += kResThreads) {
                const uint32_t key = cand(k).x;
                const uint32_t dg = (key >> shift) & (uint32_t)(kDig - 1);
                atomicAdd(&S.hm[dg], weight<kCount>((double)key_score(key) - M, S.etbl));
                atomicAdd(&S.hc[dg], 1u);
            }
            __syncthreads();
        }
        if (tid < kWave) res_choose_mass(A, T, S);
        __syncthreads();
        const uint32_t j = S.j;
        A = S.abefore;  // A plus the mass of the digits above j
        if (in_lds) {
            n = res_filter_lds<false, kCount, kVis>(S.buf[cur], n, S.buf[cur ^ 1], shift, kDig - 1, j, true,
                                      false, ir, kbr, S);
            cur ^= 1;
            cr = S.buf[cur];
        } else if (S.hc[j] <= (uint32_t)kResCap) {
            // The boundary digit's candidates fit in LDS: continue there,
            // building the next level's histogram on the way unless one
            // wave can finish them.
            few = S.hc[j] <= (uint32_t)kWave;
            next_built = level == 0 && !few;
            n = res_filter_lds<true, kCount, kVis>(gc, n, S.buf[0], shift, kDig - 1, j, true, false, ir, kbr, S,
                                     next_built, M);
            few = few && n <= kWave;
            in_lds = true;
            cur = 0;
            cr = S.buf[0];
        } else {
            n = res_filter_global<kVis>(gc, n, shift, kDig - 1, j, true, false, ir, kbr, S);
        }
    }

    if (few) {
        if (tid < kWave) resolve_few<kCount, kVis>(cr, (int)n, A, T, M, ir, kbr, S);
    } else if (n > 0) {
        // Every survivor now has the same score tau.  Keep the first c of
        // them in index order: the smallest c with A + c * e_tau >= T.
        const uint32_t tau_key = cand(0).x;
        const double e_tau = weight<kCount>((double)key_score(tau_key) - M, S.etbl);
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
                const uint32_t ix = valid ? cand(k).y : 0u;
                const int64_t pa = wave_append(valid, nout_ptr(S));
                if (pa >= 0) keep_token<kVis>(ir, pa, ix, kbr);
            }
        } else {
            // Count-only radix select of the c lowest indices: bits [30:20],
            // [19:10], [9:0].  Indices are distinct, so the last level leaves
            // one token.
            for (int level = 0; level < 3 && n > 0 && c > 0; ++level) {
                // (computed, not table-driven: a small local table indexed by
                // the loop counter would live in scratch memory)
                const int shift = level == 0 ? 20 : (level == 1 ? 10 : 0);
                const uint32_t mask = level == 0 ? 2047u : 1023u;
                const int nb = (int)mask + 1;
                for (int i = tid; i < nb; i += kResThreads) S.hc[i] = 0u;
                __syncthreads();
                for (int64_t k = tid; k < n; k += kResThreads)
                    atomicAdd(&S.hc[(cand(k).y >> shift) & mask], 1u);
                __syncthreads();
                if (tid < kWave) res_choose_count((uint32_t)c, nb, S);
                __syncthreads();
                const uint32_t j = S.j;
                c -= S.cbefore;
                if (in_lds) {
                    n = res_filter_lds<false, kCount, kVis>(S.buf[cur], n, S.buf[cur ^ 1], shift, mask, j,
                                              false, true, ir, kbr, S);
                    cur ^= 1;
                    cr = S.buf[cur];
                } else if (S.hc[j] <= (uint32_t)kResCap) {
                    n = res_filter_lds<true, kCount, kVis>(gc, n, S.buf[0], shift, mask, j, false, true, ir,
                                             kbr, S);
                    in_lds = true;
                    cur = 0;
                    cr = S.buf[0];
                } else {
                    n = res_filter_global<kVis>(gc, n, shift, mask, j, false, true, ir, kbr, S);
                }
            }
            // One token left (its index is fully determined): keep it.
            if (tid == 0 && n > 0 && c > 0) keep_token<kVis>(ir, (uint32_t)S.nn++, cand(0).y, kbr);
        }
    }
    __syncthreads();
    if (tid == 0) {
        if constexpr (kVis)
            st_agent(reinterpret_cast<uint32_t *>(count + r), emitted + (uint32_t)S.nn);
        else
            count[r] = (int32_t)(emitted + (uint32_t)S.nn);
    }
}

// What the pick reads of the row: this thread's Hist1 bins and the top
// record of chunk tid, with agent-scope loads (in the one-launch selection
// the histogram blocks of the same launch wrote them).
struct PickIn {
    double gmv[kPickPer];
    float tm0;
    double tmass0;
};

__device__ __forceinline__ void pick_inputs(SelPtrs P, int64_t r, PickIn &pi)
{
    const Hist1 &g = P.hist1[r];
#pragma unroll
    for (int k = 0; k < kPickPer; ++k) pi.gmv[k] = ld_agent(&g.mass[threadIdx.x + k * kSelThreads]);
    pi.tm0 = -INFINITY;
    pi.tmass0 = 0.0;
    if ((int)threadIdx.x < P.nblk) {
        const ChunkTop &t = P.tops[r * P.nblk + threadIdx.x];
        pi.tm0 = ld_agent(&t.m);
        pi.tmass0 = ld_agent(&t.mass);
    }
}

// One chunk's share of the emit pass (scores in v, the pick's inputs in
// pi): the row's threshold, the chunk's kept tokens and boundary-bin
// candidates, its share of Hist2; the last chunk of the row to finish
// resolves the boundary bin.
struct SelAttArgs;
// The emit block's part in the selection-and-attention launch (defined with
// that launch below).
__device__ __forceinline__ void emit_attend(const SelAttArgs &A, const SelPtrs &P, int64_t r, int N,
                            int32_t *__restrict__ idx, int32_t *__restrict__ count,
                            uint32_t above, uint32_t ex, const ChunkView &cv, ResShared &S);

template <bool kCount, bool kAtt = false>
__device__ __forceinline__ void emit_body(const float (&v)[kSelPerThread], const ChunkView &cv, int N,
                          SelPtrs P, int64_t r, double target, const PickIn &pi,
                          int32_t *__restrict__ idx, int32_t *__restrict__ count,
                          uint32_t *__restrict__ keep_bits, ResShared &S,
                          const SelAttArgs *att = nullptr)
{
    static_assert(kSelThreads == kResThreads, "the last emit block runs the resolve");
    unsigned long long *wbase = S.wbase;
    int32_t *ir = idx + r * (int64_t)N;
    uint2 *cr = P.cand + r * (int64_t)N;
    if (threadIdx.x < kExpTable) S.etbl[threadIdx.x] = kExp2Tbl[threadIdx.x];
    pick_block<kCount>(P.tops + r * P.nblk, P.nblk, target, pi.gmv, pi.tm0, pi.tmass0, S);
    const uint32_t j1 = S.j1;
    if (threadIdx.x == 0) S.bcount = 0ull;
    S.hm[threadIdx.x] = 0.0;  // this block's share of the row's Hist2
    S.hc[threadIdx.x] = 0u;
    // Per lane: bit t of `above` / `atb` marks slot t as kept / candidate;
    // `mine` packs their counts (kept in the high half).
    static_assert(kSelPerThread == 32, "one mask bit per slot");
    // Keys above hi lie in bins above j1; keys in [lo, hi] in bin j1.
    const uint32_t lo = j1 << kShift1, hi = lo | ((1u << kShift1) - 1u);
    uint32_t above = 0, atb = 0;
    if (cv.vec) {
#pragma unroll
        for (int t = 0; t < kSelPerThread; ++t) {
            const uint32_t key = score_key(v[t]);
            above |= key > hi ? (1u << t) : 0u;
            atb |= (key >= lo && key <= hi) ? (1u << t) : 0u;
        }
    } else {
#pragma unroll
        for (int t = 0; t < kSelPerThread; ++t) {
            const uint32_t key = score_key(v[t]);
            const bool valid = cv.index32(t) < (uint32_t)N;
            above |= (valid && key > hi) ? (1u << t) : 0u;
            atb |= (valid && key >= lo && key <= hi) ? (1u << t) : 0u;
        }
    }
    const uint32_t mine = ((uint32_t)__popc(above) << 16) | (uint32_t)__popc(atb);
    // Keep bitmap: this chunk's words, with the bits of the tokens kept here
    // (the resolve adds the boundary bin's kept tokens).  Agent-scope
    // stores, so the resolve's atomics land on the written words.
    uint32_t *kbr = keep_bits ? keep_bits + r * (int64_t)((N + 31) / 32) : nullptr;
    if (kbr) {
        const int lane = lane_id();
        uint32_t *kw = kbr + (uint32_t)(cv.c0 >> 5);
        if (cv.vec) {
            // Slots 4g..4g+3 of thread x are tokens g*4096 + 4x + 0..3: a
            // nibble of word g*128 + x/8; eight lanes fill one word.
#pragma unroll
            for (int g = 0; g < kSelPerThread / 4; ++g) {
                uint32_t wv = ((above >> (4 * g)) & 0xFu) << (4 * (lane & 7));
                wv |= dpp<kDppQuadXor1>(wv, wv);
                wv |= dpp<kDppQuadXor2>(wv, wv);
                wv |= dpp<kDppRowHalfMirror>(wv, wv);
                if ((lane & 7) == 0) st_agent(kw + g * 128 + (threadIdx.x >> 3), wv);
            }
        } else {
            // Slot t of thread x is token t*1024 + x: a wave's ballot is two
            // words; words past the end of the row are not written.
            const uint32_t n_words = (uint32_t)(((int64_t)N - cv.c0 + 31) >> 5);
#pragma unroll
            for (int t = 0; t < kSelPerThread; ++t) {
                const unsigned long long bal = __ballot((above >> t) & 1u);
                const uint32_t wi = (uint32_t)t * 32u + (threadIdx.x >> 5);
                if ((lane & 31) == 0 && wi < n_words)
                    st_agent(kw + wi, (uint32_t)(lane == 0 ? bal : bal >> 32));
            }
        }
    }
    // Wave prefix (a wave holds at most 2048 of each, so halves never
    // carry), then one LDS atomic per wave for its block offset and one
    // global atomic per block for its row offset.
    const uint32_t inc = wave_inclusive_scan(mine);
    const uint32_t wtot = read_lane(inc, kWave - 1);
    __syncthreads();
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0)
        wbase[w] = atomicAdd(&S.bcount, ((unsigned long long)(wtot >> 16) << 32) | (wtot & 0xFFFFu));
    __syncthreads();
    // The row offsets come back from a global atomic; until they are needed
    // the block stages its candidates in LDS and builds its share of the
    // row's Hist2 (candidates by key bits [19:10], mass exp(s - M)) there.
    const uint32_t bc = (uint32_t)S.bcount;  // this block's candidates
    unsigned long long gb = 0;
    if (threadIdx.x == 0 && S.bcount)
        gb = atomicAdd(reinterpret_cast<unsigned long long *>(&P.rows[r].slots), S.bcount);
    uint2 *stage = &S.buf[0][0];
    const bool staged = bc <= (uint32_t)(2 * kResCap);
    const uint32_t ex = inc - mine;
    const double M = (double)S.M;
    if (staged) {
        uint32_t oc = (uint32_t)wbase[w] + (ex & 0xFFFFu);
#pragma unroll
        for (int t = 0; t < kSelPerThread; ++t)
            if (atb & (1u << t)) stage[oc++] = make_uint2(score_key(v[t]), cv.index32(t));
        __syncthreads();
        for (uint32_t k = threadIdx.x; k < bc; k += kSelThreads) {
            const uint2 e = stage[k];
            const uint32_t dg = (e.x >> kShift2) & (uint32_t)(kDig - 1);
            atomicAdd(&S.hm[dg], weight<kCount>((double)key_score(e.x) - M, S.etbl));
            atomicAdd(&S.hc[dg], 1u);
        }
    }
    if (threadIdx.x == 0) S.gbase = gb;
    __syncthreads();
    const unsigned long long base = S.gbase + wbase[w];
    uint32_t oa = (uint32_t)(base >> 32) + (ex >> 16);
    for (uint32_t m = above; m; m &= m - 1) ir[oa++] = (int32_t)cv.index32(__ffs(m) - 1);
    uint2 *gcb = cr + (uint32_t)S.gbase;  // this block's candidates' place in the row
    if (staged) {
        // Written out coalesced, in block order.
        for (uint32_t k = threadIdx.x; k < bc; k += kSelThreads) st_cand(gcb + k, stage[k]);
    } else {
        // More candidates than the stage holds: written directly, then read
        // back for the histogram.
        uint32_t oc = (uint32_t)wbase[w] + (ex & 0xFFFFu);
#pragma unroll
        for (int t = 0; t < kSelPerThread; ++t)
            if (atb & (1u << t)) st_cand(gcb + oc++, make_uint2(score_key(v[t]), cv.index32(t)));
        wait_vmem();
        __syncthreads();
        for (uint32_t k = threadIdx.x; k < bc; k += kSelThreads) {
            const uint2 e = ld_cand(gcb + k);
            const uint32_t dg = (e.x >> kShift2) & (uint32_t)(kDig - 1);
            atomicAdd(&S.hm[dg], weight<kCount>((double)key_score(e.x) - M, S.etbl));
            atomicAdd(&S.hc[dg], 1u);
        }
    }
    __syncthreads();
    if (S.hc[threadIdx.x]) {
        Hist2 &h2 = P.hist2[r];
        atomicAdd(&h2.mass[threadIdx.x], S.hm[threadIdx.x]);
        atomicAdd(&h2.cnt[threadIdx.x], S.hc[threadIdx.x]);
    }
    // The last chunk of the row to finish resolves the boundary bin, once
    // every block's candidate stores have completed.
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0)
        S.last = atomicAdd(&P.rows[r].emit_done, 1u) == (uint32_t)(P.nblk - 1);
    __syncthreads();
    if constexpr (kAtt) {
        emit_attend(*att, P, r, N, idx, count, above, ex, cv, S);
        return;
    }
    if (!S.last) return;
    resolve_row<kCount>(N, P, r, idx, count, kbr, S);
    // Every block of the row has passed its waits: `ready` is reset for the
    // next call (in the two-launch selection it already is).
    if (threadIdx.x == 0) ctr_reset(&P.rows[r].ready);
}

template <bool kCount>
__global__ __launch_bounds__(kSelThreads) void sel_emit_kernel(
    const float *__restrict__ scores, int N, SelPtrs P, double target, int32_t *__restrict__ idx,
    int32_t *__restrict__ count, uint32_t *__restrict__ keep_bits)
{
    __shared__ ResShared S;
    const int64_t r = blockIdx.y;
    // The row's histogram and chunk tops (finished by the hist kernel) are
    // requested together with the chunk's scores.
    PickIn pi;
    pick_inputs(P, r, pi);
    float v[kSelPerThread];
    const ChunkView cv =
        load_chunk(scores + r * (int64_t)N, N, (int64_t)blockIdx.x * kSelChunk, v);
    emit_body<kCount>(v, cv, N, P, r, target, pi, idx, count, keep_bits, S);
}

// Both passes in one launch.  Block rows [0, R) are the histogram blocks,
// rows [R, 2R) the emit blocks, so every histogram block is dispatched
// before any emit block.  An emit block loads its chunk, then waits until
// its row's Hist1 is complete (the last histogram block of the row raises
// `ready` to 2); it never waits for a later block, and no histogram block
// waits for an emit block, so the launch needs no co-residency.
template <bool kCount>
__global__ __launch_bounds__(kSelThreads) void sel_fused_kernel(
    const float *__restrict__ scores, int N, SelPtrs P, double target, int32_t *__restrict__ idx,
    int32_t *__restrict__ count, uint32_t *__restrict__ keep_bits)
{
    __shared__ ResShared S;
    const int R = (int)gridDim.y / 2;
    const int blk = blockIdx.x;
    if ((int)blockIdx.y < R) {
        const int64_t r = blockIdx.y;
        float v[kSelPerThread];
        const ChunkView cv = load_chunk(scores + r * (int64_t)N, N, (int64_t)blk * kSelChunk, v);
        if (blk == 0) clear_row(P, r);
        static_assert(sizeof(double) * kBins1 <= sizeof(S.buf), "the histogram fits in buf");
        hist_body<kCount>(v, cv, N, r, blk, P, reinterpret_cast<double *>(&S.buf[0][0]), S.etbl,
                          S.red);
        wait_vmem();  // this block's Hist1 adds and top record are done
        __syncthreads();
        if (threadIdx.x == 0 &&
            atomicAdd(&P.rows[r].hist_done, 1u) == (uint32_t)(P.nblk - 1))
            ctr_add(&P.rows[r].ready, 1u);  // 2: the row's Hist1 is complete
        return;
    }
    const int64_t r = blockIdx.y - R;
    float v[kSelPerThread];
    const ChunkView cv = load_chunk(scores + r * (int64_t)N, N, (int64_t)blk * kSelChunk, v);
    if (threadIdx.x == 0) wait_row_ready(P.rows[r], 2u, P.wc);
    __syncthreads();
    PickIn pi;
    pick_inputs(P, r, pi);
    emit_body<kCount>(v, cv, N, P, r, target, pi, idx, count, keep_bits, S);
}

// ---------------------------------------------------------------- p >= 1

__global__ __launch_bounds__(256) void sel_all_kernel(int N, int32_t *__restrict__ idx,
                                                      int32_t *__restrict__ count,
                                                      uint32_t *__restrict__ keep_bits)
{
    const int64_t r = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < N) idx[r * (int64_t)N + i] = (int32_t)i;
    if (blockIdx.x == 0 && threadIdx.x == 0) count[r] = N;
    const int64_t n_words = ((int64_t)N + 31) / 32;
    if (keep_bits && i < n_words) {
        const int64_t left = (int64_t)N - i * 32;  // tokens in this word
        keep_bits[r * n_words + i] = left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
    }
}

// ------------------------------------------------- sinks + window bits
//
// Adds the local rows [0, min(n_sink, w0)) and [w0, N), w0 = max(0, N -
// window), to every keep bitmap row: thread w owns word w of its row, so no
// two threads touch one word.

__global__ __launch_bounds__(256) void keep_local_kernel(uint32_t *__restrict__ keep_bits, int N,
                                                         int n_words, int64_t sink_end,
                                                         int64_t w0)
{
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= n_words) return;
    const int64_t lo = w * 32, hi = lo + 32;
    // Bits of [a, b) within this word.
    auto span = [&](int64_t a, int64_t b) -> uint32_t {
        a = a > lo ? a : lo;
        b = b < hi ? b : hi;
        if (a >= b) return 0u;
        const uint32_t n = (uint32_t)(b - a), s = (uint32_t)(a - lo);
        return (n == 32u ? 0xFFFFFFFFu : ((1u << n) - 1u)) << s;
    };
    const uint32_t m = span(0, sink_end) | span(w0, N);
    if (m) keep_bits[(int64_t)blockIdx.y * n_words + w] |= m;
}

hipError_t launch_keep_local(uint32_t *keep_bits, int64_t R, int N, int n_sink, int window,
                             hipStream_t stream)
{
    const int n_words = (N + 31) / 32;
    const int64_t w0 = N > window ? (int64_t)N - window : 0;
    const int64_t sink_end = n_sink < w0 ? n_sink : w0;
    dim3 grid((unsigned)((n_words + 255) / 256), (unsigned)R);
    return launch(keep_local_kernel, grid, dim3(256), 0, stream, keep_bits, N, n_words, sink_end,
                  w0);
}

constexpr int64_t kMaxFusedRows = 65535;  // grid rows of one launch

hipError_t launch_topp_hist(const float *scores, int64_t R, int N, void *ws, hipStream_t stream)
{
    SelPtrs P = sel_ptrs(ws, R, N);
    RTP_TRY(wait_ctl(&P.wc));
    return launch(sel_hist_kernel<false>, dim3((unsigned)P.nblk, (unsigned)R), dim3(kSelThreads),
                  0, stream, scores, N, P);
}

static hipError_t launch_keep_all(int64_t R, int N, int32_t *idx, int32_t *count,
                                  uint32_t *keep_bits, hipStream_t stream)
{
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)R);
    return launch(sel_all_kernel, grid, dim3(256), 0, stream, N, idx, count, keep_bits);
}

// target: p for top-p (kCount false), k for top-k (kCount true).
template <bool kCount>
static hipError_t launch_select(const float *scores, int64_t R, int N, double target,
                                int32_t *idx, int32_t *count, uint32_t *keep_bits, void *ws,
                                hipStream_t stream)
{
    SelPtrs P = sel_ptrs(ws, R, N);
    RTP_TRY(wait_ctl(&P.wc));
    if (2 * R <= kMaxFusedRows)
        return launch(sel_fused_kernel<kCount>, dim3((unsigned)P.nblk, (unsigned)(2 * R)),
                      dim3(kSelThreads), 0, stream, scores, N, P, target, idx, count, keep_bits);
    dim3 grid((unsigned)P.nblk, (unsigned)R);
    RTP_TRY(launch(sel_hist_kernel<kCount>, grid, dim3(kSelThreads), 0, stream, scores, N, P));
    return launch(sel_emit_kernel<kCount>, grid, dim3(kSelThreads), 0, stream, scores, N, P, target,
                  idx, count, keep_bits);
}

hipError_t launch_topp_select(const float *scores, int64_t R, int N, float p, int32_t *idx,
                              int32_t *count, uint32_t *keep_bits, void *ws, hipStream_t stream)
{
    if (p >= 1.0f) return launch_keep_all(R, N, idx, count, keep_bits, stream);
    return launch_select<false>(scores, R, N, (double)p, idx, count, keep_bits, ws, stream);
}

hipError_t launch_topk_select(const float *scores, int64_t R, int N, int k, int32_t *idx,
                              int32_t *count, uint32_t *keep_bits, void *ws, hipStream_t stream)
{
    if (k >= N) return launch_keep_all(R, N, idx, count, keep_bits, stream);
    return launch_select<true>(scores, R, N, (double)k, idx, count, keep_bits, ws, stream);
}

// ---------------------------------- selection and attention in one launch
//
// The top-p set of each score row and exact attention over it (gist.science
// summary, method sections 3 and 5), with the local heads over sinks +
// window (section 1), in the selection's own launch.  The histogram blocks
// are those above.  Each emit block, once it has counted itself done:
//   - if it is the row's last, resolves the boundary bin first (the kept
//     tokens and the count with agent-scope stores) and raises `ready` to 3;
//   - attends the tokens it emitted itself, from an LDS copy of its own
//     list (no memory round trip), while the row's resolve runs;
//   - waits for the row's resolve and attends its share (1/nblk) of the
//     tokens the resolve added;
//   - takes local tiles from a shared queue until none is left: 64
//     sink/window rows of one local KV head for all its query heads, merged
//     by the tile of the (batch row, KV head) that arrives last.
// Every emit block thus leaves two partials (m, l, o) per row; they merge in
// groups of 16 (the group's last arriver), then per row (the last group
// merger writes the output and resets the row's `ready`).  Every wait is on
// the row's last emit block, which is already running when it is waited
// on.  Logits are in log2 units (scale * log2(e) folded into q).

namespace {

constexpr int kAW = kSelThreads / kWave;  // waves per block
constexpr int kAPF = 132;                 // floats per partial: m, l, pad, pad, o[128]
constexpr int kARU = 8;                   // rows in flight per 16-lane group
constexpr int kAGS = 16;                  // partials per group merge
constexpr int kALT = 64;                  // local rows per tile
constexpr int kAMH = 8;                   // query heads per KV head, at most
constexpr int kALU = kALT / kAW;          // local rows per wave and tile

// Per-wave partial slots in LDS for nh heads: m[w * nh + h], l likewise,
// o[(w * nh + h) * 128 + d].
struct SlotView {
    float *m, *l, *o;
    int nh;
};

// Slots for one head in the resolve's digit histogram (free by then).
__device__ __forceinline__ SlotView slots_one(ResShared &S)
{
    static_assert(sizeof(S.hm) >= sizeof(float) * kAW * (2 + 128), "one head's slots fit");
    float *f = reinterpret_cast<float *>(&S.hm[0]);
    return SlotView{f, f + kAW, f + 2 * kAW, 1};
}

// Slots for kAMH heads in the candidate buffers (free by then).
__device__ __forceinline__ SlotView slots_heads(ResShared &S)
{
    static_assert(sizeof(S.buf) >= sizeof(float) * kAW * kAMH * (2 + 128), "the slots fit");
    float *f = reinterpret_cast<float *>(&S.buf[0][0]);
    return SlotView{f, f + kAW * kAMH, f + 2 * kAW * kAMH, kAMH};
}

struct AttState {
    float m, l, o[8];
};

__device__ __forceinline__ float att_rescale(float m_old, float m_new)
{
    return m_old == -INFINITY ? 0.0f : exp2f(m_old - m_new);
}

// Sum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ float att_sum16(float v)
{
    v += dpp<kDppQuadXor1>(v, v);
    v += dpp<kDppQuadXor2>(v, v);
    v += dpp<kDppRowHalfMirror>(v, v);
    v += dpp<kDppRowMirror>(v, v);
    return v;
}

__device__ __forceinline__ void att_reset(AttState &a)
{
    a.m = -INFINITY;
    a.l = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) a.o[c] = 0.0f;
}

// This lane's 8 dimensions of a query row, times scale * log2(e).
__device__ __forceinline__ void att_q8(const uint16_t *p, float qscale, float (&qf)[8])
{
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    bf16x8_to_f32(w, qf);
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] *= qscale;
}

// One online-softmax step of this lane's 16-lane group over rows tok[u] (a
// negative token is no row); Kb/Vb point at the KV head's row 0 plus this
// lane's 8 dimensions.
__device__ __forceinline__ void att_rows(const uint16_t *__restrict__ Kb,
                                         const uint16_t *__restrict__ Vb, const float (&qf)[8],
                                         const int (&tok)[kARU], AttState &a)
{
    uint4 kw[kARU], vw[kARU];
#pragma unroll
    for (int u = 0; u < kARU; ++u) {
        const int64_t off = tok[u] >= 0 ? (int64_t)tok[u] * 128 : 0;
        kw[u] = ld_nt16(Kb + off);
        vw[u] = ld_nt16(Vb + off);
    }
    float lg[kARU];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kARU; ++u) {
        float kf[8];
        bf16x8_to_f32(kw[u], kf);
        float d = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) d = fmaf(qf[c], kf[c], d);
        d = att_sum16(d);
        lg[u] = tok[u] >= 0 ? d : -INFINITY;
        mx = fmaxf(mx, lg[u]);
    }
    const float mn = fmaxf(a.m, mx);
    if (mn == -INFINITY) return;
    const float corr = att_rescale(a.m, mn);
    a.l *= corr;
#pragma unroll
    for (int c = 0; c < 8; ++c) a.o[c] *= corr;
#pragma unroll
    for (int u = 0; u < kARU; ++u) {
        const float pw = tok[u] >= 0 ? exp2f(lg[u] - mn) : 0.0f;
        float vf[8];
        bf16x8_to_f32(vw[u], vf);
        a.l += pw;
#pragma unroll
        for (int c = 0; c < 8; ++c) a.o[c] = fmaf(pw, vf[c], a.o[c]);
    }
    a.m = mn;
}

// Merges the four 16-lane groups of the wave into the wave's slot for head
// h.  Every lane of the wave calls it.
__device__ __forceinline__ void att_flush(AttState &a, int w, int h, const SlotView &v)
{
    const int lane = lane_id(), sub = lane & 15;
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
        const float mo = __shfl_xor(a.m, off);
        const float lo = __shfl_xor(a.l, off);
        const float mn = fmaxf(a.m, mo);
        const float fa = att_rescale(a.m, mn), fb = att_rescale(mo, mn);
        a.l = a.l * fa + lo * fb;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float oo = __shfl_xor(a.o[c], off);
            a.o[c] = a.o[c] * fa + oo * fb;
        }
        a.m = mn;
    }
    const int s = w * v.nh + h;
    if (lane < 16) {
#pragma unroll
        for (int c = 0; c < 8; ++c) v.o[s * 128 + sub * 8 + c] = a.o[c];
        if (lane == 0) {
            v.l[s] = a.l;
            v.m[s] = a.m;
        }
    }
}

// Merges the waves' slots of heads hh < nh into one partial each at dst +
// hh * hstride (agent-scope stores).  Thread t takes head t / 128 and output
// dimension t % 128.
__device__ __forceinline__ void att_slots_to_partial(int nh, const SlotView &v, float *dst,
                                                     int64_t hstride)
{
    const int hh = threadIdx.x >> 7, d = threadIdx.x & 127;
    if (hh >= nh) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAW; ++w) M = fmaxf(M, v.m[w * v.nh + hh]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kAW; ++w) {
            const float mw = v.m[w * v.nh + hh];
            if (mw != -INFINITY) {
                const float f = exp2f(mw - M);
                L = fmaf(v.l[w * v.nh + hh], f, L);
                O = fmaf(v.o[(w * v.nh + hh) * 128 + d], f, O);
            }
        }
    }
    float *pp = dst + hh * hstride;
    st_agent(pp + 4 + d, O);
    if (d == 0) {
        st_agent(pp, M);
        st_agent(pp + 1, L);
    }
}

// Merges n partials of each head hh < nh: partial (k, hh) at base + k *
// kstride + hh * kAPF (agent-scope loads).  Writes the merged partial at
// dst + hh * kAPF (agent-scope stores) or, with dst NULL, the normalised
// output row at outp + hh * 128.
__device__ __forceinline__ void att_merge(const float *base, int64_t kstride, int n, int nh,
                                          float *dst, float *outp)
{
    const int hh = threadIdx.x >> 7, d = threadIdx.x & 127;
    if (hh >= nh) return;
    constexpr int kB = 8;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int k0 = 0; k0 < n; k0 += kB) {
        float pm[kB], pl[kB], po[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const bool ok = k0 + u < n;
            const float *pk = base + (int64_t)(ok ? k0 + u : k0) * kstride + hh * kAPF;
            pm[u] = ok ? ld_agent(pk) : -INFINITY;
            pl[u] = ld_agent(pk + 1);
            po[u] = ld_agent(pk + 4 + d);
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < kB; ++u) mb = fmaxf(mb, pm[u]);
        if (mb == -INFINITY) continue;
        const float cr = att_rescale(M, mb);
        L *= cr;
        O *= cr;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const float f = att_rescale(pm[u], mb);
            L = f > 0.0f ? fmaf(pl[u], f, L) : L;
            O = f > 0.0f ? fmaf(po[u], f, O) : O;
        }
        M = mb;
    }
    if (dst) {
        float *pp = dst + hh * kAPF;
        st_agent(pp + 4 + d, O);
        if (d == 0) {
            st_agent(pp, M);
            st_agent(pp + 1, L);
        }
    } else {
        outp[hh * 128 + d] = L > 0.0f ? O / L : 0.0f;
    }
}

// After this block's agent-scope stores: counts the block on ctr and tells
// every thread whether it was the last of `expected` (the last one resets
// the counter for the next call).  `flag` is an LDS word.
__device__ __forceinline__ bool att_arrive_last(unsigned long long *ctr, uint32_t expected,
                                                int &flag)
{
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        const bool last = ctr_arrive(ctr) == expected - 1u;
        if (last) ctr_reset(ctr);
        flag = last ? 1 : 0;
    }
    __syncthreads();
    return flag != 0;
}

}  // namespace

struct SelAttArgs {
    const uint16_t *q, *K, *V;  // bf16: q [B][Hq][128]; K, V [B][Hkv][kv_cap][128]
    float *out;                 // f32 [B][Hq][128]
    int Hq, Hkv, H_r, G;        // score row b * H_r + h: query head h of batch row b
    int64_t kv_cap;
    float qscale;               // scale * log2(e)
    int ng;                     // group merges per row: ceil(2 nblk / kAGS)
    int nE;                     // emit blocks: R * nblk
    int n_lkv;                  // local KV heads, after the H_r / G retrieval ones
    int nl_rows, sink_end, w0;  // local rows: [0, sink_end), then [w0, N)
    int nlt;                    // local tiles per (batch row, local KV head)
    int n_items;                // local tiles in all
    float *part;                // [R][2 nblk] block partials
    float *gpart;               // [R][ng] group merges
    unsigned long long *gctr;   // [R][ng] tagged counters
    unsigned long long *rctr;   // [R]
    float *lpart;               // [n_items][kAMH] local partials
    unsigned long long *lctr;   // [B * n_lkv]
    unsigned long long *lq;     // the local tiles' queue
};

namespace {

// Local tile `item`: rows [tile*kALT, +kALT) of the sink + window list of
// local KV head gl of batch row bl, for its G query heads.  Lane group lg of
// a wave takes query heads 2lg and 2lg + 1, so all four groups read the same
// row.
__device__ __forceinline__ void att_local_tile(const SelAttArgs &A, int item, const SlotView &v, int &flag)
{
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int lg = lane >> 4, sub = lane & 15;
    const int tile = item % A.nlt, rest = item / A.nlt;
    const int gl = rest % A.n_lkv, bl = rest / A.n_lkv;
    const int gk = A.H_r / A.G + gl;
    const int p0 = tile * kALT, p1 = min(A.nl_rows, p0 + kALT);
    const int ha = 2 * lg, hb = 2 * lg + 1;
    const bool ua = ha < A.G, ub = hb < A.G;
    float qa[8], qb[8];
    const uint16_t *qrow = A.q + ((int64_t)bl * A.Hq + (int64_t)gk * A.G) * 128 + sub * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) qa[c] = qb[c] = 0.0f;
    if (ua) att_q8(qrow + ha * 128, A.qscale, qa);
    if (ub) att_q8(qrow + hb * 128, A.qscale, qb);
    const int64_t kvb = ((int64_t)bl * A.Hkv + gk) * A.kv_cap * 128 + sub * 8;
    uint4 kw[kALU], vw[kALU];
    bool ok[kALU];
#pragma unroll
    for (int u = 0; u < kALU; ++u) {
        const int pos = p0 + w * kALU + u;
        ok[u] = pos < p1;
        const int tok = pos < A.sink_end ? pos : A.w0 + (pos - A.sink_end);
        const int64_t off = ok[u] ? (int64_t)tok * 128 : 0;
        kw[u] = ld_nt16(A.K + kvb + off);
        vw[u] = ld_nt16(A.V + kvb + off);
    }
    AttState sa, sb;
    att_reset(sa);
    att_reset(sb);
    float la[kALU], lb[kALU];
    float ma = -INFINITY, mbx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kALU; ++u) {
        float kf[8];
        bf16x8_to_f32(kw[u], kf);
        float da = 0.0f, db = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            da = fmaf(qa[c], kf[c], da);
            db = fmaf(qb[c], kf[c], db);
        }
        da = att_sum16(da);
        db = att_sum16(db);
        la[u] = ok[u] ? da : -INFINITY;
        lb[u] = ok[u] ? db : -INFINITY;
        ma = fmaxf(ma, la[u]);
        mbx = fmaxf(mbx, lb[u]);
    }
    sa.m = ma;
    sb.m = mbx;
#pragma unroll
    for (int u = 0; u < kALU; ++u) {
        const float pa = ok[u] && ma != -INFINITY ? exp2f(la[u] - ma) : 0.0f;
        const float pb = ok[u] && mbx != -INFINITY ? exp2f(lb[u] - mbx) : 0.0f;
        float vf[8];
        bf16x8_to_f32(vw[u], vf);
        sa.l += pa;
        sb.l += pb;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            sa.o[c] = fmaf(pa, vf[c], sa.o[c]);
            sb.o[c] = fmaf(pb, vf[c], sb.o[c]);
        }
    }
    if (ua) {
        const int s = w * v.nh + ha;
#pragma unroll
        for (int c = 0; c < 8; ++c) v.o[s * 128 + sub * 8 + c] = sa.o[c];
        if (sub == 0) {
            v.m[s] = sa.m;
            v.l[s] = sa.l;
        }
    }
    if (ub) {
        const int s = w * v.nh + hb;
#pragma unroll
        for (int c = 0; c < 8; ++c) v.o[s * 128 + sub * 8 + c] = sb.o[c];
        if (sub == 0) {
            v.m[s] = sb.m;
            v.l[s] = sb.l;
        }
    }
    __syncthreads();
    att_slots_to_partial(A.G, v, A.lpart + (int64_t)item * kAMH * kAPF, kAPF);
    if (att_arrive_last(A.lctr + rest, (uint32_t)A.nlt, flag)) {
        float *outp = A.out + ((int64_t)bl * A.Hq + (int64_t)gk * A.G) * 128;
        att_merge(A.lpart + (int64_t)rest * A.nlt * kAMH * kAPF, (int64_t)kAMH * kAPF, A.nlt, A.G,
                  nullptr, outp);
    }
    __syncthreads();
}

// Publishes the block's one-head slots as partial pi of row r and runs the
// merges it is last for: the group of 16 partials, then the row (the output,
// and the reset of the row's `ready`).
__device__ __forceinline__ void att_publish(const SelAttArgs &A, const SelPtrs &P, int64_t r, int pi, int nparts,
                            const SlotView &v, int &flag)
{
    __syncthreads();
    att_slots_to_partial(1, v, A.part + ((int64_t)r * nparts + pi) * kAPF, kAPF);
    const int gi = pi / kAGS, gn = min(kAGS, nparts - gi * kAGS);
    if (att_arrive_last(A.gctr + (int64_t)r * A.ng + gi, (uint32_t)gn, flag)) {
        att_merge(A.part + ((int64_t)r * nparts + gi * kAGS) * kAPF, kAPF, gn, 1,
                  A.gpart + ((int64_t)r * A.ng + gi) * kAPF, nullptr);
        if (att_arrive_last(A.rctr + r, (uint32_t)A.ng, flag)) {
            const int b = (int)(r / A.H_r), h = (int)(r % A.H_r);
            att_merge(A.gpart + (int64_t)r * A.ng * kAPF, kAPF, A.ng, 1, nullptr,
                      A.out + ((int64_t)b * A.Hq + h) * 128);
            // Every block of the row has passed its wait.
            if (threadIdx.x == 0) ctr_reset(&P.rows[r].ready);
        }
    }
    __syncthreads();
}

// Local tiles from the launch's queue until none is left; every emit block
// calls it once, so the block whose grab is the last of all resets it.
__device__ __forceinline__ void att_local_queue(const SelAttArgs &A, ResShared &S)
{
    if (A.n_items <= 0) return;
    const SlotView heads = slots_heads(S);
    for (;;) {
        if (threadIdx.x == 0) {
            const uint32_t it = ctr_add(A.lq, 1u);
            if (it >= (uint32_t)A.n_items && it == (uint32_t)(A.n_items + A.nE - 1))
                ctr_reset(A.lq);
            S.j = it;
        }
        __syncthreads();
        const uint32_t it = S.j;
        __syncthreads();
        if (it >= (uint32_t)A.n_items) break;
        att_local_tile(A, (int)it, heads, S.last);
    }
}

}  // namespace

__device__ __forceinline__ void emit_attend(const SelAttArgs &A, const SelPtrs &P, int64_t r, int N,
                            int32_t *__restrict__ idx, int32_t *__restrict__ count,
                            uint32_t above, uint32_t ex, const ChunkView &cv, ResShared &S)
{
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int lg = lane >> 4, sub = lane & 15;
    const int e = blockIdx.x, nblk = P.nblk, nparts = 2 * nblk;
    const bool last = S.last != 0;
    // This wave's first slot in the block's list of emitted tokens, and
    // the block's count (the resolve reuses the LDS words they sit in).
    const uint32_t wkb = (uint32_t)(S.wbase[w] >> 32);
    const uint32_t nk = (uint32_t)(S.bcount >> 32);
    __syncthreads();
    if (last) {
        if (tid == 0) {
            const unsigned long long sl =
                ld_agent(reinterpret_cast<const unsigned long long *>(&P.rows[r].slots));
            st_agent(&P.rows[r].kept1, (uint32_t)(sl >> 32));
        }
        resolve_row<false, true>(N, P, r, idx, count, nullptr, S);
        wait_vmem();
        __syncthreads();
        if (tid == 0) ctr_add(&P.rows[r].ready, 1u);  // 3: the row's set is complete
    }
    const int b = (int)(r / A.H_r), h = (int)(r % A.H_r), g = h / A.G;
    float qf[8];
    att_q8(A.q + ((int64_t)b * A.Hq + h) * 128 + sub * 8, A.qscale, qf);
    const int64_t kvb = ((int64_t)b * A.Hkv + g) * A.kv_cap * 128 + sub * 8;
    const SlotView one = slots_one(S);

    // 1. The tokens this block emitted, from an LDS copy of its list.
    uint32_t *list = reinterpret_cast<uint32_t *>(&S.buf[0][0]);
    {
        uint32_t o = wkb + (ex >> 16);
        for (uint32_t m = above; m; m &= m - 1) list[o++] = cv.index32(__ffs(m) - 1);
    }
    if (tid < kAW) {
        one.m[tid] = -INFINITY;
        one.l[tid] = 0.0f;
    }
    __syncthreads();
    {
        AttState st;
        att_reset(st);
        const uint32_t gi = (uint32_t)(w * 4 + lg);  // rows gi + 64 j of the list
        for (uint32_t k0 = gi; k0 < nk; k0 += 64u * kARU) {
            int tok[kARU];
#pragma unroll
            for (int u = 0; u < kARU; ++u) {
                const uint32_t k = k0 + 64u * (uint32_t)u;
                tok[u] = k < nk ? (int)list[k] : -1;
            }
            att_rows(A.K + kvb, A.V + kvb, qf, tok, st);
        }
        att_flush(st, w, 0, one);
    }
    att_publish(A, P, r, e, nparts, one, S.last);

    // 2. This block's share of the tokens the row's resolve added.
    if (tid == 0) {
        wait_row_ready(P.rows[r], 3u, P.wc);
        const uint32_t k1 = min(ld_agent(&P.rows[r].kept1), (uint32_t)N);
        uint32_t c = min(ld_agent(reinterpret_cast<const uint32_t *>(count + r)), (uint32_t)N);
        c = max(c, k1);
        const uint64_t len = c - k1;
        S.j = k1 + (uint32_t)(len * (uint64_t)e / (uint64_t)nblk);
        S.cbefore = k1 + (uint32_t)(len * (uint64_t)(e + 1) / (uint64_t)nblk);
    }
    if (tid < kAW) {
        one.m[tid] = -INFINITY;
        one.l[tid] = 0.0f;
    }
    __syncthreads();
    {
        const uint32_t lo = S.j, hi = S.cbefore;
        const uint32_t *ir = reinterpret_cast<const uint32_t *>(idx + r * (int64_t)N);
        AttState st;
        att_reset(st);
        const uint32_t gi = (uint32_t)(w * 4 + lg);
        for (uint32_t k0 = lo + gi; k0 < hi; k0 += 64u * kARU) {
            int tok[kARU];
#pragma unroll
            for (int u = 0; u < kARU; ++u) {
                const uint32_t k = k0 + 64u * (uint32_t)u;
                const uint32_t t = k < hi ? ld_agent(ir + k) : 0xFFFFFFFFu;
                tok[u] = t < (uint32_t)N ? (int)t : -1;
            }
            att_rows(A.K + kvb, A.V + kvb, qf, tok, st);
        }
        att_flush(st, w, 0, one);
    }
    att_publish(A, P, r, nblk + e, nparts, one, S.last);
    // 3. Local tiles from the queue.
    att_local_queue(A, S);
}

// The selection with attention (block rows [0, R) histogram blocks, [R, 2R)
// emit blocks, as in sel_fused_kernel).
__global__ __launch_bounds__(kSelThreads) void sel_attend_kernel(
    const float *__restrict__ scores, int N, SelPtrs P, double target,
    int32_t *__restrict__ idx, int32_t *__restrict__ count, SelAttArgs A)
{
    __shared__ ResShared S;
    const int R = (int)gridDim.y / 2;
    const int blk = blockIdx.x;
    if ((int)blockIdx.y < R) {
        const int64_t r = blockIdx.y;
        float v[kSelPerThread];
        const ChunkView cv = load_chunk(scores + r * (int64_t)N, N, (int64_t)blk * kSelChunk, v);
        if (blk == 0) clear_row(P, r);
        hist_body<false>(v, cv, N, r, blk, P, reinterpret_cast<double *>(&S.buf[0][0]), S.etbl,
                         S.red);
        wait_vmem();
        __syncthreads();
        if (threadIdx.x == 0 &&
            atomicAdd(&P.rows[r].hist_done, 1u) == (uint32_t)(P.nblk - 1))
            ctr_add(&P.rows[r].ready, 1u);  // 2: the row's Hist1 is complete
        return;
    }
    const int64_t r = blockIdx.y - R;
    float v[kSelPerThread];
    const ChunkView cv = load_chunk(scores + r * (int64_t)N, N, (int64_t)blk * kSelChunk, v);
    if (threadIdx.x == 0) wait_row_ready(P.rows[r], 2u, P.wc);
    __syncthreads();
    PickIn pi;
    pick_inputs(P, r, pi);
    emit_body<false, true>(v, cv, N, P, r, target, pi, idx, count, nullptr, S, &A);
}

struct SelAttGeom {
    int64_t R;
    int nblk, ng, G, n_lkv, nl_rows, sink_end, w0, nlt, n_items;
    size_t part, gpart, gctr, rctr, lpart, lctr, lq, total;
};

static SelAttGeom sel_att_geom(int B, int Hq, int Hkv, int N, int H_r, int n_sink, int window)
{
    SelAttGeom g;
    g.R = (int64_t)B * H_r;
    const SelLayout L = sel_layout(g.R, N);
    g.nblk = (int)L.nblk;
    g.ng = (2 * g.nblk + kAGS - 1) / kAGS;
    g.G = Hq / Hkv;
    g.n_lkv = Hkv - H_r / g.G;
    const int w0 = N > window ? N - window : 0;
    g.w0 = w0;
    g.sink_end = n_sink < w0 ? n_sink : w0;
    g.nl_rows = g.sink_end + (N - w0);
    g.nlt = (g.nl_rows + kALT - 1) / kALT;
    g.n_items = B * g.n_lkv * g.nlt;
    size_t off = align_up(L.total, 256);
    g.part = off;
    off += align_up((size_t)g.R * 2 * g.nblk * kAPF * sizeof(float), 256);
    g.gpart = off;
    off += align_up((size_t)g.R * g.ng * kAPF * sizeof(float), 256);
    g.gctr = off;
    off += align_up((size_t)g.R * g.ng * 8, 256);
    g.rctr = off;
    off += align_up((size_t)g.R * 8, 256);
    g.lpart = off;
    off += align_up((size_t)g.n_items * kAMH * kAPF * sizeof(float), 256);
    g.lctr = off;
    off += align_up((size_t)B * g.n_lkv * 8, 256);
    g.lq = off;
    off += 256;
    g.total = off;
    return g;
}

size_t topp_attend_ws_bytes(int cus, int B, int Hq, int Hkv, int N, int H_r, int n_sink,
                            int window)
{
    (void)cus;
    const SelAttGeom g = sel_att_geom(B, Hq, Hkv, N, H_r, n_sink, window);
    const size_t att = attend_ws_bytes(B, H_r, Hq - H_r, N);  // the p >= 1 path
    return g.total > att ? g.total : att;
}

bool topp_attend_fits(int cus, int B, int Hq, int Hkv, int N, int H_r, int n_sink, int window)
{
    (void)cus;
    const SelAttGeom g = sel_att_geom(B, Hq, Hkv, N, H_r, n_sink, window);
    return g.G <= kAMH && H_r % g.G == 0 && 2 * g.R <= kMaxFusedRows;
}

hipError_t launch_topp_attend(const float *scores, const uint16_t *q, const uint16_t *K,
                              const uint16_t *V, int B, int Hq, int Hkv, int N, int64_t kv_cap,
                              int H_r, int n_sink, int window, float p, float scale, float *out,
                              int32_t *idx, int32_t *count, void *ws, hipStream_t stream)
{
    if (p >= 1.0f) {
        // Every token is kept: the listing, then the attention launch.
        RTP_TRY(launch_keep_all((int64_t)B * H_r, N, idx, count, nullptr, stream));
        return launch_decode_attend(q, K, V, idx, count, B, Hq, Hkv, N, kv_cap, 0, H_r, H_r,
                                    Hq - H_r, n_sink, window, scale, out, ws, stream);
    }
    const SelAttGeom g = sel_att_geom(B, Hq, Hkv, N, H_r, n_sink, window);
    SelPtrs P = sel_ptrs(ws, g.R, N);
    RTP_TRY(wait_ctl(&P.wc));
    char *base = static_cast<char *>(ws);
    SelAttArgs A;
    A.q = q;
    A.K = K;
    A.V = V;
    A.out = out;
    A.Hq = Hq;
    A.Hkv = Hkv;
    A.H_r = H_r;
    A.G = g.G;
    A.kv_cap = kv_cap;
    A.qscale = scale * 1.4426950408889634f;
    A.ng = g.ng;
    A.nE = (int)(g.R * g.nblk);
    A.n_lkv = g.n_lkv;
    A.nl_rows = g.nl_rows;
    A.sink_end = g.sink_end;
    A.w0 = g.w0;
    A.nlt = g.nlt;
    A.n_items = g.n_items;
    A.part = reinterpret_cast<float *>(base + g.part);
    A.gpart = reinterpret_cast<float *>(base + g.gpart);
    A.gctr = reinterpret_cast<unsigned long long *>(base + g.gctr);
    A.rctr = reinterpret_cast<unsigned long long *>(base + g.rctr);
    A.lpart = reinterpret_cast<float *>(base + g.lpart);
    A.lctr = reinterpret_cast<unsigned long long *>(base + g.lctr);
    A.lq = reinterpret_cast<unsigned long long *>(base + g.lq);
    return launch(sel_attend_kernel, dim3((unsigned)g.nblk, (unsigned)(2 * g.R)),
                  dim3(kSelThreads), 0, stream, scores, N, P, (double)p, idx, count, A);
}

}  // namespace rtp
