// One decode step of one attention layer in a single launch: the indexer
// scan, the top-p selection and exact sparse attention for the retrieval
// heads, and sinks + window attention for the local heads (gist.science
// summary of arXiv 2605.16928: method section 1, the two head roles;
// section 2, the 16-dim indexer taken before RoPE; section 3, keep adding
// low-dim attention mass until it reaches p; section 5, a sort-free
// histogram threshold and bandwidth-optimised sparse decode).
//
// The results are those of rtp_index_scores, rtp_topp_select,
// rtp_sparse_decode and rtp_local_decode run in sequence; what changes is
// where the intermediate data lives.  The launch is persistent: one block
// of 1024 threads per compute unit, each owning a chunk of up to 32768
// scores of one (batch row, retrieval KV head) for its whole life.
//
//   scan     each block streams its chunk of the indexer key cache once,
//            scores it against the G query heads of the KV head (the same
//            fp32 fma chain as rtp_index_scores), and keeps the scores in
//            registers.  Nothing of them goes to memory unless the caller
//            asks for the scores.
//   level 1  per head, a block histogram of fp64 mass exp(s - m_b) (m_b the
//            block's max) over bins of width 1/4 on the logit axis,
//            floor(4 s), counted down from the block's top bin; the last
//            bin collects everything further down.  One block per head (of
//            the row's last blocks) waits for every record of its row,
//            realigns them to the row's top bin, rescales them to the row
//            max, and picks the head's boundary bin J* and the mass A above
//            it.
//   local    meanwhile the other blocks run the local heads: 64-row tiles
//            of the sink + window rows, every K/V row read once for the G
//            query heads of its KV head.  When the rows leave compute units
//            free, extra blocks there take the local tiles instead.
//   classify every block waits for its row's thresholds (a wait on blocks
//            that may come later: it relies on the launch's blocks being
//            resident together, which the host ensures by launching at most
//            one block per compute unit), then lists its tokens above bin J*
//            as kept (the row's idx list and an LDS list), and rescores the
//            tokens of bin J*: exact score key and index go to the row's
//            candidate list.  Once every block has classified, each head's
//            reducer builds the head's level-2 histogram from that list in
//            LDS (1024 digits of width 1/4096 inside bin J*) and picks the
//            boundary digit.
//   gather   every other block attends its own level-1 rows while the
//            boundary digits are picked, then its candidates above those
//            digits; one partial per head is merged by last arrivers in two
//            levels.
//   resolve  each head's reducer then resolves the head's boundary digit: a
//            mass-weighted radix select over its candidates' score keys,
//            ties to the lower index, then the kept boundary rows'
//            attention, whose partial joins the head's final merge; then it
//            attends its own rows.
//
// Every wait is bounded (a host-set limit) and reports a give-up in the
// library's status word; every data-dependent index is range-checked, so a
// give-up yields wrong numbers but no stray access.
#include <float.h>
#include <math.h>

#include "rtp_device.h"
#include "rtp_exp.h"
#include "rtp_launch.h"

namespace rtp {

namespace {

constexpr int kT = 1024;                // threads per block
constexpr int kNW = kT / kWave;         // waves per block
constexpr int kTPT = 4;                 // tokens per thread
constexpr int kChunk = kTPT * 1024;     // tokens per block, at most
constexpr int kMH = 8;                  // query heads per KV head, at most
constexpr int kNB = 128;                // level-1 bins per head (the last: everything lower)
constexpr float kBPU = 4.0f;            // bins per unit of logit
constexpr int kGS = 16;                 // records merged per last-arriver step
constexpr int kTile = 64;               // local rows per item
constexpr int kPF = 132;                // floats per attention partial: m, l, pad, pad, o[128]
constexpr int kRU = 8;                  // rows in flight per 16-lane group (sparse rows)
constexpr int kBatch = 4 * kRU;         // rows per wave batch
constexpr int kLU = 4;                  // rows in flight per wave (local rows)
constexpr int kLocIters = kTile / (kNW * kLU);  // local row batches per wave
constexpr int kFine = 1024;             // level-2 digits of the boundary bin
constexpr int kResCap = 1536;           // resolve candidates per LDS buffer
constexpr int kBkCap = 2048;            // kept boundary tokens listed in LDS
constexpr int kListCap = kMH * kChunk;  // kept-token offsets per block (all heads)
constexpr float kLog2eF = 1.4426950408889634f;

static_assert(kNB * kMH == kT, "one thread per (head, bin)");
static_assert(128 * kMH == kT, "one thread per (head, output dimension)");
static_assert(kTile == kNW * kLocIters * kLU, "each wave takes kLocIters * kLU local rows");
static_assert(kFine == kT, "one thread per level-2 digit");

static __constant__ double kLayerExpTbl[kExpTable] = RTP_EXP2_TABLE;

// -------------------------------------------------------------- records

struct HistRec {            // level-1 histogram of the G heads of one block or group
    double mass[kMH][kNB];  // relative to m[h]
    float m[kMH];           // max score
    int32_t T[kMH];         // bin of m: bin j holds scores with floor(4 s) = T - j
};

struct PickRec {            // a head's threshold
    float M;                // row max
    int32_t T;              // bin of M
    int32_t jstar;          // boundary bin: J < jstar kept, J == jstar candidates
    int32_t pad;
    double A;               // mass of the bins above jstar, relative to M
    double Pt;              // p * Z
};

struct Pick2Rec {           // a head's level-2 threshold inside the boundary bin
    int32_t j2;             // boundary digit (mode 0)
    int32_t mode;           // 0: digits above j2 kept, j2 resolved; 1: every candidate kept;
                            // 2: every candidate resolved
    uint32_t ka;            // tokens kept above the boundary bin
    uint32_t k2;            // candidates kept above the boundary digit
    uint32_t cstar;         // candidates in the boundary digit (mode 0) or all (mode 2)
    uint32_t nc;            // candidates
    double A2;              // mass above the boundary digit, relative to M
};

struct RgCtl {  // tagged counters of one (batch row, retrieval KV head)
    unsigned long long hist_row, pick_ready, classified, pick2_ready, p2_done, fin_done, pad0,
        pad1;
    unsigned long long kept[kMH], cand[kMH], kept2[kMH], att_row[kMH];
};
static_assert(sizeof(RgCtl) == 320, "RgCtl is 320 B");

struct LayerWs {
    HistRec *h1;                   // [NB] one per block
    PickRec *pick;                 // [RG][kMH]
    Pick2Rec *pick2;               // [RG][kMH]
    RgCtl *ctl;                    // [RG]
    unsigned long long *att_grp;   // [RG][ngrp]
    unsigned long long *loc_ctr;   // [B][n_lkv]
    float *att1;                   // [NB][kMH][kPF]
    float *att2;                   // [RG][ngrp + 1][kMH][kPF]; entry ngrp: the boundary rows
    float *loc;                    // [NI][kMH][kPF]
    uint2 *cand;                   // [RG][G][N]
    uint2 *pdesc;                  // [RG][kMH][kMH] a reducer's level-1 lists: (idx slot, count)
};

struct LayerParams {
    const float *q_r;
    const float *k_r;
    const uint16_t *q;
    const uint16_t *K;
    const uint16_t *V;
    float *out;
    int32_t *idx;
    int32_t *count;
    float *scores;  // optional
    int64_t kr_cap, kv_cap;
    int B, Hq, Hkv, N, Hq_r, Hkv_r;
    int bpr, C, ngrp;
    int n_lkv, nlt, NI, nl_rows, sink_end, w0;
    int NBr, NX;  // row blocks (the grid's first), then blocks for local items only
    int keep_all;
    double pd;
    float qscale;
    uint32_t spin_limit;
    uint32_t *status;
    LayerWs ws;
};

struct Cand {
    uint32_t key, idx;
    double e;  // exp(s - M)
};

struct HistLds {
    double hist[kMH][kNB];   // the block's histogram
    double wrow[kNW][kNB];   // a head's records merged per wave (row reducer)
    double acc[kNB];         // a head's merged histogram (row reducer)
    double rf[256];          // per block record: exp(m_b - M)
    double ru[kNW];
    float rm[256];           // per block record: max and top bin
    int32_t rT[256];
    int32_t ro[256];         // T - T_b
    float wm[kNW];
    int32_t wt[kNW];
    float M;
    int32_t T;
};

struct FineLds {  // a head's level-2 histogram
    double m[kFine];
    uint32_t c[kFine];
    double dscan[kNW];
    uint32_t uscan[kNW], first[kNW];
};

struct SlotLds {  // per-wave attention partials
    float m[kNW][kMH], l[kNW][kMH];
    float o[kNW][kMH][128];
};

struct ResLds {
    Cand buf[2][kResCap];
    double hm[256];
    uint32_t hc[2048];
    double tmp[kWave];
    uint32_t uscan[kNW];
    double dscan[kNW];
};

struct LayerLds {
    union {
        HistLds h;
        SlotLds s;
        ResLds r;
        FineLds f;
    } a;
    union {
        uint32_t gsw[kMH * kTPT / 2][kT];  // scan to classify: this thread's score bins, 2 per word
        uint16_t list[kListCap];  // kept-token offsets in the chunk, head h at h * kChunk
    } b;
    int32_t bk[kBkCap];           // a resolved head's kept boundary tokens
    double etbl[kExpTable];
    alignas(16) float qr[kMH][16];
    PickRec pick[kMH];
    float mb[kMH];
    int32_t Tb[kMH];
    float red[kMH][kNW];
    uint32_t wcnt[kMH][kNW];
    uint32_t kc[kMH], cc[kMH];
    uint32_t kgb[kMH], cgb[kMH];
    Pick2Rec pick2[kMH];
    uint32_t n2[kMH], k2b[kMH];  // level-2 kept rows of the block per head, their slot base
    uint32_t fka, fnc;           // a head's kept and candidate totals (its reducer)
    uint32_t kt[kMH];            // both lists of a head
    uint2 pd[kMH][kMH];          // the reducers' level-1 lists: [reducer][head] (idx slot, count)
    int bpre[kMH + 1];
    int hlast[kMH];
    int flag;
    uint32_t nkeep, nmove, j, cbefore, kmin, kmax;
    double abefore;
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float rescale2(float m_old, float m_new)
{
    return m_old == -INFINITY ? 0.0f : exp2f(m_old - m_new);
}

__device__ __forceinline__ float sum16(float v)
{
    v += dpp<kDppQuadXor1>(v, v);
    v += dpp<kDppQuadXor2>(v, v);
    v += dpp<kDppRowHalfMirror>(v, v);
    v += dpp<kDppRowMirror>(v, v);
    return v;
}

// Level-1 bin coordinate of a score: floor(4 s), clamped to 16 bits.  4 s is
// exact (a power-of-two scale), the clamp keeps it finite, and the map is
// monotone, so "bin above" means "score above".
__device__ __forceinline__ int score_bin(float s)
{
    return (int)floorf(fminf(fmaxf(s * kBPU, -32768.0f), 32767.0f));
}

__device__ __forceinline__ void st_agent_i(int32_t *p, int32_t v)
{
    st_agent(reinterpret_cast<uint32_t *>(p), (uint32_t)v);
}
__device__ __forceinline__ int32_t ld_agent_i(const int32_t *p)
{
    return (int32_t)ld_agent(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ uint2 ld_cand2(const uint2 *p)
{
    const unsigned long long v = ld_agent(reinterpret_cast<const unsigned long long *>(p));
    return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
__device__ __forceinline__ void st_cand2(uint2 *p, uint2 e)
{
    st_agent(reinterpret_cast<unsigned long long *>(p),
             (unsigned long long)e.x | ((unsigned long long)e.y << 32));
}

// Thread 0 polls a tagged counter until it holds at least `level`; after
// `limit` polls it gives up and sets the timeout bit of the status word.
__device__ __forceinline__ void wait_level(const unsigned long long *ctr, uint32_t level, uint32_t limit,
                           uint32_t *status)
{
    for (uint32_t it = 0;; ++it) {
        const unsigned long long v = ld_agent(ctr);
        if ((uint32_t)v == kCtrTag && (uint32_t)(v >> 32) >= level) return;
        if (it >= limit) {
            if (status) atomicOr(status, kStatusWaitTimeout);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// After this block's agent-scope stores: counts the block on ctr and tells
// every thread whether it was the last of `expected` (the last one resets
// the counter for the next call).
__device__ __forceinline__ bool arrive_last_blk(unsigned long long *ctr, uint32_t expected, LayerLds &S)
{
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        const bool last = ctr_arrive(ctr) == expected - 1u;
        if (last) ctr_reset(ctr);
        S.flag = last ? 1 : 0;
    }
    __syncthreads();
    return S.flag != 0;
}

// ------------------------------------------------------------ attention

struct AttState {
    float m, l, o[8];
};

__device__ __forceinline__ void att_reset(AttState &a)
{
    a.m = -INFINITY;
    a.l = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) a.o[c] = 0.0f;
}

__device__ __forceinline__ void load_q8(const uint16_t *p, float scale, float (&qf)[8])
{
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    bf16x8_to_f32(w, qf);
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] *= scale;
}

// One online-softmax step of this lane's 16-lane group over rows tok[u]
// (a negative or out-of-range token is no row) of one KV head; Kb/Vb point
// at the head's row 0 plus this lane's 8 dimensions.
__device__ __forceinline__ void att_rows(const uint16_t *__restrict__ Kb,
                                         const uint16_t *__restrict__ Vb, const float (&qf)[8],
                                         const int (&tok)[kRU], int N, AttState &a)
{
    uint4 kw[kRU], vw[kRU];
    bool ok[kRU];
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
        ok[u] = (unsigned)tok[u] < (unsigned)N;
        const int64_t off = ok[u] ? (int64_t)tok[u] * 128 : 0;
        kw[u] = ld_nt16(Kb + off);
        vw[u] = ld_nt16(Vb + off);
    }
    float lg[kRU];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
        float kf[8];
        bf16x8_to_f32(kw[u], kf);
        float d = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) d = fmaf(qf[c], kf[c], d);
        d = sum16(d);
        lg[u] = ok[u] ? d : -INFINITY;
        mx = fmaxf(mx, lg[u]);
    }
    const float mn = fmaxf(a.m, mx);
    if (mn == -INFINITY) return;
    const float corr = rescale2(a.m, mn);
    a.l *= corr;
#pragma unroll
    for (int c = 0; c < 8; ++c) a.o[c] *= corr;
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
        const float pw = ok[u] ? exp2f(lg[u] - mn) : 0.0f;
        float vf[8];
        bf16x8_to_f32(vw[u], vf);
        a.l += pw;
#pragma unroll
        for (int c = 0; c < 8; ++c) a.o[c] = fmaf(pw, vf[c], a.o[c]);
    }
    a.m = mn;
}

// Merges the four 16-lane groups of the wave, then into the wave's slot for
// head h (an empty slot has m = -inf).  Every lane of the wave must call it.
__device__ __forceinline__ void att_flush(AttState &a, int w, int h, LayerLds &S)
{
    const int lane = lane_id(), sub = lane & 15;
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
        const float mo = __shfl_xor(a.m, off);
        const float lo = __shfl_xor(a.l, off);
        const float mn = fmaxf(a.m, mo);
        const float fa = rescale2(a.m, mn), fb = rescale2(mo, mn);
        a.l = a.l * fa + lo * fb;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float oo = __shfl_xor(a.o[c], off);
            a.o[c] = a.o[c] * fa + oo * fb;
        }
        a.m = mn;
    }
    if (lane < 16) {
        const float ms = S.a.s.m[w][h];
        const float mn = fmaxf(a.m, ms);
        if (mn == -INFINITY) return;
        const float fa = rescale2(a.m, mn), fb = rescale2(ms, mn);
        const bool had = ms != -INFINITY;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float prev = had ? S.a.s.o[w][h][sub * 8 + c] * fb : 0.0f;
            S.a.s.o[w][h][sub * 8 + c] = fmaf(a.o[c], fa, prev);
        }
        if (lane == 0) {
            S.a.s.l[w][h] = fmaf(a.l, fa, had ? S.a.s.l[w][h] * fb : 0.0f);
            S.a.s.m[w][h] = mn;
        }
    }
}

__device__ __forceinline__ void slots_clear(LayerLds &S)
{
    if ((int)threadIdx.x < kNW * kMH) {
        S.a.s.m[threadIdx.x / kMH][threadIdx.x % kMH] = -INFINITY;
        S.a.s.l[threadIdx.x / kMH][threadIdx.x % kMH] = 0.0f;
    }
}

// Merges the waves' slots of heads hh < nh into one partial per head at
// dst + hh * hstride (agent-scope stores).  Thread t takes head t / 128 and
// output dimension t % 128.
__device__ __forceinline__ void slots_to_partial(int nh, float *dst, int64_t hstride, LayerLds &S)
{
    const int hh = threadIdx.x >> 7, d = threadIdx.x & 127;
    if (hh >= nh) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, S.a.s.m[w][hh]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
            const float mw = S.a.s.m[w][hh];
            if (mw != -INFINITY) {
                const float f = exp2f(mw - M);
                L = fmaf(S.a.s.l[w][hh], f, L);
                O = fmaf(S.a.s.o[w][hh][d], f, O);
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

// Merges n partial records for each head hh < nh whose bit is set in hmask:
// record (k, hh) at base + k * kstride + hh * kPF (published by other blocks:
// agent-scope loads).  Writes a merged record at dst + hh * kPF (agent-scope
// stores) or, with dst NULL, the normalised output row at outp + hh * 128.
__device__ __forceinline__ void merge_records(const float *base, int64_t kstride, int n, int nh, uint32_t hmask,
                              float *dst, float *outp)
{
    const int hh = threadIdx.x >> 7, d = threadIdx.x & 127;
    if (hh >= nh || !((hmask >> hh) & 1u)) return;
    constexpr int kB = 8;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int k0 = 0; k0 < n; k0 += kB) {
        float pm[kB], pl[kB], po[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const bool ok = k0 + u < n;
            const float *pk = base + (int64_t)(ok ? k0 + u : k0) * kstride + hh * kPF;
            pm[u] = ok ? ld_agent(pk) : -INFINITY;
            pl[u] = ld_agent(pk + 1);
            po[u] = ld_agent(pk + 4 + d);
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < kB; ++u) mb = fmaxf(mb, pm[u]);
        if (mb == -INFINITY) continue;
        const float cr = rescale2(M, mb);
        L *= cr;
        O *= cr;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const float f = rescale2(pm[u], mb);
            L = f > 0.0f ? fmaf(pl[u], f, L) : L;
            O = f > 0.0f ? fmaf(po[u], f, O) : O;
        }
        M = mb;
    }
    if (dst) {
        float *pp = dst + hh * kPF;
        st_agent(pp + 4 + d, O);
        if (d == 0) {
            st_agent(pp, M);
            st_agent(pp + 1, L);
        }
    } else {
        outp[hh * 128 + d] = L > 0.0f ? O / L : 0.0f;
    }
}

// ------------------------------------------------------------------ scan

// This thread's key rows c0 + t*kT + tid (t < kTPT) of KV head g of row b,
// all loads issued at once (zeros at or past the chunk's end).
__device__ __forceinline__ void scan_load(const LayerParams &P, int b, int g, int64_t c0, int cn,
                                          float4 (&kv)[kTPT][4])
{
    const int tid = threadIdx.x;
    const float4 *kr =
        reinterpret_cast<const float4 *>(P.k_r + ((int64_t)b * P.Hkv_r + g) * P.kr_cap * 16);
#pragma unroll
    for (int t = 0; t < kTPT; ++t) {
        const int o = t * kT + tid;
        if (o < cn) {
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[t][j] = kr[(c0 + o) * 4 + j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[t][j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// Scores of the loaded rows t < NT for the G query heads (q_r from LDS):
// one sequential fma chain per score over dimensions 0..15 from +0
// (bit-identical to rtp_index_scores; a chain from +0 never ends at -0, so
// no sign fix-up is needed).  The NT chains of a head advance together,
// dimension by dimension, so consecutive fmas are independent.  Tokens at
// or past the chunk's end score -inf.
template <int G, int NT>
__device__ __forceinline__ void scan_scores(const float4 (&kv)[kTPT][4], int cn, const LayerLds &S,
                                            float (&sc)[kTPT][G])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        // (a compiler barrier: one head's chains in flight at a time)
        asm volatile("" ::: "memory");
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            const float4 q = reinterpret_cast<const float4 *>(S.qr[h])[j4];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(q.x, kv[t][j4].x, acc[t]);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(q.y, kv[t][j4].y, acc[t]);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(q.z, kv[t][j4].z, acc[t]);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(q.w, kv[t][j4].w, acc[t]);
        }
#pragma unroll
        for (int t = 0; t < kTPT; ++t) sc[t][h] = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t) sc[t][h] = t * kT + tid < cn ? acc[t] : -INFINITY;
    }
}

// The block's scores (token slots t < NT hold its tokens: NT = the chunk's
// length over kT, rounded up), the optional score output, the block's max
// and top bin per head, then its level-1 histogram (mass exp(s - m_b) in
// fp64, bins counted down from the top bin) and every score's bin in LDS
// (two 16-bit bins per word) for the classify.  The histogram has no
// per-token branch: a token past the chunk's end adds +0 to the last bin,
// so a head's exponentials run interleaved.
template <int G, int NT>
__device__ __forceinline__ void block_scan_hist(const LayerParams &P, int b, int g, int64_t c0,
                                                int cn, const float4 (&kv)[kTPT][4], LayerLds &S)
{
    const int tid = threadIdx.x, w = tid / kWave;
    float sc[kTPT][G];
    scan_scores<G, NT>(kv, cn, S, sc);
    if (P.scores) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float *sr = P.scores + ((int64_t)b * P.Hq_r + (int64_t)g * G + h) * P.N + c0;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t * kT + tid < cn) sr[t * kT + tid] = sc[t][h];
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t) m = fmaxf(m, sc[t][h]);
        m = wave_max(m);
        if (lane_id() == 0) S.red[h][w] = m;
    }
    __syncthreads();
    if (tid < G) {
        float m = S.red[tid][0];
        for (int i = 1; i < kNW; ++i) m = fmaxf(m, S.red[tid][i]);
        S.mb[tid] = m;
        S.Tb[tid] = score_bin(m);
    }
    __syncthreads();
    uint32_t gw[G * kTPT / 2];
#pragma unroll
    for (int e = 0; e < G * kTPT / 2; ++e) gw[e] = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        asm volatile("" ::: "memory");
        const double mbd = (double)S.mb[h];
        const int Tb = S.Tb[h];
        double ev[NT];
        int jv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float s = sc[t][h];
            const int gs = score_bin(s);
            jv[t] = min(Tb - gs, kNB - 1);
            ev[t] = exp_tang((double)s - mbd, S.etbl);
            const int e = t * G + h;
            gw[e >> 1] |= ((uint32_t)gs & 0xFFFFu) << (16 * (e & 1));
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
            atomicAdd(&S.a.h.hist[h][jv[t]], t * kT + tid < cn ? ev[t] : 0.0);
    }
#pragma unroll
    for (int e = 0; e < G * kTPT / 2; ++e) S.b.gsw[e][tid] = gw[e];
    __syncthreads();
}

// --------------------------------------------------------- level 1 merge

// The row's reducer for head h: merges the n block records of head h (all
// published) into the row's histogram and publishes the head's threshold.
// One round of loads: every record's max, top bin and bins together.  Each
// record's bins are shifted down by the distance of its top bin from the
// row's top and scaled by exp(m_b - M); bins that fall out of the window
// join the last bin.  Then: Z = sum of every bin; the boundary bin is the
// first bin from the top whose running mass (every bin above it plus its
// own) reaches p Z, tested bin by bin so no rounding of the parallel prefix
// can skip it; when the total falls short of p Z through rounding, the
// lowest bin with mass.
template <int G>
__device__ __forceinline__ void reduce_head(const LayerParams &P, int rg, int h, LayerLds &S)
{
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int n = P.bpr;  // <= 256
    HistLds &H = S.a.h;
    const HistRec *in = P.ws.h1 + (int64_t)rg * P.bpr;
    // Wave w takes records w, w + 16, ...; lane l their bins l and l + 64.
    constexpr int kPer = 256 / kNW;  // records per wave
    double v0[kPer], v1[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int b = w + k * kNW;
        v0[k] = b < n ? ld_agent(&in[b].mass[h][lane]) : 0.0;
        v1[k] = b < n ? ld_agent(&in[b].mass[h][lane + kWave]) : 0.0;
    }
    float m = -INFINITY;
    int T = -32768;
    if (tid < n) {
        m = ld_agent(&in[tid].m[h]);
        T = ld_agent_i(&in[tid].T[h]);
        H.rm[tid] = m;
        H.rT[tid] = T;
    }
    H.wrow[w][lane] = 0.0;
    H.wrow[w][lane + kWave] = 0.0;
    m = wave_max(m);
    const float tw = wave_max((float)T);
    if (lane == 0) {
        H.wm[w] = m;
        H.wt[w] = (int32_t)tw;
    }
    __syncthreads();
    if (tid == 0) {
        float M = H.wm[0];
        int32_t TT = H.wt[0];
        for (int i = 1; i < kNW; ++i) {
            M = fmaxf(M, H.wm[i]);
            TT = max(TT, H.wt[i]);
        }
        H.M = M;
        H.T = TT;
    }
    __syncthreads();
    if (tid < n) {
        H.ro[tid] = H.T - H.rT[tid];
        H.rf[tid] = exp_tang((double)H.rm[tid] - (double)H.M, S.etbl);
    }
    __syncthreads();
    // Each wave adds its records into a row of its own, record by record:
    // the lanes shift by the same distance, so no two touch one bin, and
    // the wave's LDS operations run in order (no atomics).
    double u = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int b = w + k * kNW;
        if (b < n) {
            const int o = H.ro[b];
            const double f = H.rf[b];
            const double a0 = v0[k] * f, a1 = v1[k] * f;
            const int d0 = lane + o, d1 = lane + kWave + o;
            if (o >= 0 && d0 < kNB - 1)
                H.wrow[w][d0] += a0;
            else
                u += a0;
            if (lane + kWave < kNB - 1 && o >= 0 && d1 < kNB - 1)
                H.wrow[w][d1] += a1;
            else
                u += a1;
        }
    }
    const double ws = wave_sum(u);
    if (lane == 0) H.ru[w] = ws;
    __syncthreads();
    if (tid < kNB) {
        double a = 0.0;
#pragma unroll
        for (int q = 0; q < kNW; ++q) a += H.wrow[q][tid];
        H.acc[tid] = a;
    }
    __syncthreads();
    if (tid == 0) {
        double U = 0.0;
        for (int i = 0; i < kNW; ++i) U += H.ru[i];
        H.acc[kNB - 1] += U;
    }
    __syncthreads();
    if (w != 0) return;
    const double w0 = H.acc[2 * lane], w1 = H.acc[2 * lane + 1];
    const double inc = wave_inclusive_scan(w0 + w1);
    const double Z = read_lane(inc, kWave - 1);
    const double Pt = P.pd * Z;
    double cum = wave_shift_up(inc);
    int cross = -1, low = -1;
    double cross_b = 0.0, low_b = 0.0;
    if (w0 > 0.0) {
        if (cum + w0 >= Pt) {
            cross = 2 * lane;
            cross_b = cum;
        }
        low = 2 * lane;
        low_b = cum;
    }
    cum += w0;
    if (w1 > 0.0) {
        if (cross < 0 && cum + w1 >= Pt) {
            cross = 2 * lane + 1;
            cross_b = cum;
        }
        low = 2 * lane + 1;
        low_b = cum;
    }
    const uint64_t cm = __ballot(cross >= 0);
    const uint64_t lm = __ballot(low >= 0);
    int js;
    double A;
    if (cm) {
        const int src = __ffsll((unsigned long long)cm) - 1;
        js = read_lane(cross, src);
        A = read_lane(cross_b, src);
    } else if (lm) {
        const int src = 63 - __clzll((unsigned long long)lm);
        js = read_lane(low, src);
        A = read_lane(low_b, src);
    } else {
        js = 0;
        A = 0.0;
    }
    if (P.keep_all) {
        js = kNB;  // every bin kept, no candidates
        A = Z;
    }
    if (lane == 0) {
        PickRec *pr = P.ws.pick + (int64_t)rg * kMH + h;
        st_agent(&pr->M, H.M);
        st_agent_i(&pr->T, H.T);
        st_agent_i(&pr->jstar, js);
        st_agent(&pr->A, A);
        st_agent(&pr->Pt, Pt);
    }
}

// Level-2 digit of a score inside its level-1 bin: floor(4096 s) counted from
// the bin's low edge, 1024 digits of width 1/4096 (clamped, so scores beyond
// the 16-bit bin range land in the end digits).  Monotone in s within a bin.
__device__ __forceinline__ int fine_digit(float s)
{
    const double t = floor((double)s * 4096.0) - (double)score_bin(s) * 1024.0;
    return (int)fmin(fmax(t, 0.0), (double)(kFine - 1));
}

// Head h's level-2 threshold, by the head's reducer block once every block
// of the row has classified.  The head's candidates (the row's candidate
// list) make a histogram in LDS over 1024 digits of width 1/4096 inside the
// boundary bin: fp64 mass exp(s - M) and count per digit.  The boundary
// digit is the first from the top whose running mass from A (the mass above
// the boundary bin) reaches p Z; the digits above it are kept, the digit
// itself is resolved.  Also reads the head's kept and candidate totals and
// resets those counters (every block has added to them).
template <int G>
__device__ __forceinline__ void fine_head(const LayerParams &P, int rg, int h, LayerLds &S)
{
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    RgCtl &ctl = P.ws.ctl[rg];
    FineLds &F = S.a.f;
    F.m[tid] = 0.0;
    F.c[tid] = 0u;
    if (tid == 0) {
        S.fka = (uint32_t)(ld_agent(&ctl.kept[h]) >> 32);
        S.fnc = (uint32_t)(ld_agent(&ctl.cand[h]) >> 32);
        ctr_reset(&ctl.kept[h]);
        ctr_reset(&ctl.cand[h]);
    }
    __syncthreads();
    const PickRec pk = S.pick[h];
    const uint32_t ka = S.fka, nc = min(S.fnc, (uint32_t)P.N);
    const bool digits = pk.jstar < kNB - 1 && nc > 0u;
    if (digits) {
        const uint2 *gc = P.ws.cand + ((int64_t)rg * G + h) * P.N;
        const double M = (double)pk.M;
        constexpr int kU = 8;  // candidates in flight per thread
        for (uint32_t k0 = 0; k0 < nc; k0 += kU * kT) {
            uint2 e[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const uint32_t k = k0 + (uint32_t)(u * kT + tid);
                e[u] = k < nc ? ld_cand2(gc + k) : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (k0 + (uint32_t)(u * kT + tid) < nc) {
                    const float sv = key_score(e[u].x);
                    const int d = fine_digit(sv);
                    atomicAdd(&F.m[d], exp_tang((double)sv - M, S.etbl));
                    atomicAdd(&F.c[d], 1u);
                }
            }
        }
    }
    __syncthreads();
    // Thread t takes digit 1023 - t: exclusive prefixes from the top.
    const double fm = F.m[kFine - 1 - tid];
    const uint32_t fc = F.c[kFine - 1 - tid];
    double tot;
    const double before = block_exclusive_scan<kT, double>(fm, F.dscan, &tot);
    uint32_t ctot;
    const uint32_t cb = block_exclusive_scan<kT, uint32_t>(fc, F.uscan, &ctot);
    const bool hit = digits && fc != 0u && pk.A + before + fm >= pk.Pt;
    const uint64_t hm = __ballot(hit);
    if (lane == 0) F.first[w] = hm ? (uint32_t)(__ffsll((unsigned long long)hm) - 1) : 64u;
    __syncthreads();
    int ft = -1;
    for (int i = 0; i < kNW; ++i)
        if (F.first[i] < 64u) {
            ft = i * kWave + (int)F.first[i];
            break;
        }
    Pick2Rec r;
    r.ka = ka;
    r.nc = nc;
    bool writer = tid == 0;
    if (!digits) {
        // No candidates, or the boundary bin is the last (no digits): every
        // candidate goes to the resolve.
        r.mode = 2;
        r.j2 = 0;
        r.k2 = 0u;
        r.cstar = nc;
        r.A2 = pk.A;
    } else if (ft < 0) {
        // The bin's mass falls short of the target through rounding: every
        // candidate is kept.
        r.mode = 1;
        r.j2 = -1;
        r.k2 = nc;
        r.cstar = 0u;
        r.A2 = pk.A;
    } else {
        writer = tid == ft;
        r.mode = 0;
        r.j2 = kFine - 1 - ft;
        r.k2 = cb;
        r.cstar = fc;
        r.A2 = pk.A + before;
    }
    if (writer) {
        S.pick2[h] = r;
        Pick2Rec *pr = P.ws.pick2 + (int64_t)rg * kMH + h;
        st_agent_i(&pr->j2, r.j2);
        st_agent_i(&pr->mode, r.mode);
        st_agent(&pr->ka, r.ka);
        st_agent(&pr->k2, r.k2);
        st_agent(&pr->cstar, r.cstar);
        st_agent(&pr->nc, r.nc);
        st_agent(&pr->A2, r.A2);
    }
}

// ----------------------------------------------------------- local heads

// One local item: rows [tile*kTile, +kTile) of the sink + window list of
// local KV head gl of batch row bl, for its G query heads.  Lane group lg of
// a wave takes query heads 2lg and 2lg + 1, so every lane group reads the
// same row (one memory request per row and wave).
template <int G>
__device__ __forceinline__ void local_item(const LayerParams &P, int item, LayerLds &S)
{
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int lg = lane >> 4, sub = lane & 15;
    const int tile = item % P.nlt;
    const int rest = item / P.nlt;
    const int gl = rest % P.n_lkv, bl = rest / P.n_lkv;
    const int gk = P.Hkv_r + gl;
    const int p0 = tile * kTile, p1 = min(P.nl_rows, p0 + kTile);
    const int ha = 2 * lg, hb = 2 * lg + 1;
    const bool ua = ha < G, ub = hb < G;
    float qa[8], qb[8];
    const uint16_t *qrow = P.q + ((int64_t)bl * P.Hq + (int64_t)gk * G) * 128 + sub * 8;
    if (ua) {
        load_q8(qrow + ha * 128, P.qscale, qa);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) qa[c] = 0.0f;
    }
    if (ub) {
        load_q8(qrow + hb * 128, P.qscale, qb);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) qb[c] = 0.0f;
    }
    const int64_t kvb = ((int64_t)bl * P.Hkv + gk) * P.kv_cap * 128 + sub * 8;
    const uint16_t *Kb = P.K + kvb;
    const uint16_t *Vb = P.V + kvb;
    AttState sa, sb;
    att_reset(sa);
    att_reset(sb);
    for (int it = 0; it < kLocIters; ++it) {
        uint4 kw[kLU], vw[kLU];
        bool ok[kLU];
#pragma unroll
        for (int u = 0; u < kLU; ++u) {
            const int pos = p0 + w * (kLocIters * kLU) + it * kLU + u;
            ok[u] = pos < p1;
            const int tok = pos < P.sink_end ? pos : P.w0 + (pos - P.sink_end);
            const int64_t off = ok[u] ? (int64_t)tok * 128 : 0;
            kw[u] = ld_nt16(Kb + off);
            vw[u] = ld_nt16(Vb + off);
        }
        float la[kLU], lb[kLU];
        float ma = -INFINITY, mbx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kLU; ++u) {
            float kf[8];
            bf16x8_to_f32(kw[u], kf);
            float da = 0.0f, db = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                da = fmaf(qa[c], kf[c], da);
                db = fmaf(qb[c], kf[c], db);
            }
            da = sum16(da);
            db = sum16(db);
            la[u] = ok[u] ? da : -INFINITY;
            lb[u] = ok[u] ? db : -INFINITY;
            ma = fmaxf(ma, la[u]);
            mbx = fmaxf(mbx, lb[u]);
        }
        const float na = fmaxf(sa.m, ma), nb = fmaxf(sb.m, mbx);
        const float ca = rescale2(sa.m, na), cb = rescale2(sb.m, nb);
        sa.l *= ca;
        sb.l *= cb;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            sa.o[c] *= ca;
            sb.o[c] *= cb;
        }
#pragma unroll
        for (int u = 0; u < kLU; ++u) {
            const float pa = ok[u] && na != -INFINITY ? exp2f(la[u] - na) : 0.0f;
            const float pb = ok[u] && nb != -INFINITY ? exp2f(lb[u] - nb) : 0.0f;
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
        sa.m = na;
        sb.m = nb;
    }
    if (ua) {
#pragma unroll
        for (int c = 0; c < 8; ++c) S.a.s.o[w][ha][sub * 8 + c] = sa.o[c];
        if (sub == 0) {
            S.a.s.m[w][ha] = sa.m;
            S.a.s.l[w][ha] = sa.l;
        }
    }
    if (ub) {
#pragma unroll
        for (int c = 0; c < 8; ++c) S.a.s.o[w][hb][sub * 8 + c] = sb.o[c];
        if (sub == 0) {
            S.a.s.m[w][hb] = sb.m;
            S.a.s.l[w][hb] = sb.l;
        }
    }
    __syncthreads();
    slots_to_partial(G, P.ws.loc + (int64_t)item * kMH * kPF, kPF, S);
    if (arrive_last_blk(P.ws.loc_ctr + (int64_t)bl * P.n_lkv + gl, (uint32_t)P.nlt, S)) {
        float *outp = P.out + ((int64_t)bl * P.Hq + (int64_t)gk * G) * 128;
        merge_records(P.ws.loc + (int64_t)rest * P.nlt * kMH * kPF, (int64_t)kMH * kPF, P.nlt, G,
                      0xFFu, nullptr, outp);
    }
    __syncthreads();
}

// -------------------------------------------------------------- classify

// Marks this block's tokens against the row's threshold.  Kept tokens go to
// the head's LDS list (one global slot reservation per head and block; the
// idx entries are written later, by level1_idx); tokens of the boundary bin
// are rescored and written as candidates (score key, index).
template <int G>
__device__ __forceinline__ void classify(const LayerParams &P, int rg, int b, int g, int64_t c0,
                                         int cn, LayerLds &S)
{
    constexpr int TPT = kTPT;
    constexpr int cmax = kChunk;
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    RgCtl &ctl = P.ws.ctl[rg];
    // This thread's score bins (read before the block overwrites them with
    // its lists: the barriers below come first).
    uint32_t gsp[G * kTPT / 2];
#pragma unroll
    for (int e = 0; e < G * kTPT / 2; ++e) gsp[e] = S.b.gsw[e][tid];
    uint32_t km[G], cm[G], ex[G];
    uint32_t anyc = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int T = S.pick[h].T, js = S.pick[h].jstar;
        uint32_t k = 0, c = 0;
#pragma unroll
        for (int t = 0; t < TPT; ++t) {
            const int e = t * G + h;
            const int gs = (int)(int16_t)(gsp[e >> 1] >> (16 * (e & 1)));
            const int J = min(max(T - gs, 0), kNB - 1);
            const bool v = t * kT + tid < cn;
            k |= (v && J < js) ? (1u << t) : 0u;
            c |= (v && J == js) ? (1u << t) : 0u;
        }
        km[h] = k;
        cm[h] = c;
        anyc |= c;
        const uint32_t mine = (uint32_t)__popc(k) | ((uint32_t)__popc(c) << 16);
        const uint32_t inc = wave_inclusive_scan(mine);
        ex[h] = inc - mine;
        if (lane == kWave - 1) S.wcnt[h][w] = inc;
    }
    __syncthreads();
    if (tid < G) {
        uint32_t run = 0;
        for (int w2 = 0; w2 < kNW; ++w2) {
            const uint32_t v = S.wcnt[tid][w2];
            S.wcnt[tid][w2] = run;
            run += v;
        }
        S.kc[tid] = run & 0xFFFFu;
        S.cc[tid] = run >> 16;
    }
    __syncthreads();
    if (tid < G) S.kgb[tid] = ctr_add(&ctl.kept[tid], S.kc[tid]);
    if (tid >= 64 && tid < 64 + G) S.cgb[tid - 64] = ctr_add(&ctl.cand[tid - 64], S.cc[tid - 64]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        uint32_t pos = (S.wcnt[h][w] & 0xFFFFu) + (ex[h] & 0xFFFFu);
        for (uint32_t m = km[h]; m; m &= m - 1) {
            const int t = __ffs(m) - 1;
            S.b.list[h * cmax + pos++] = (uint16_t)(t * kT + tid);
        }
    }
    __syncthreads();
    // Candidates: the exact score again (the same chain as the scan, from the
    // key rows of this thread's candidate tokens, all loaded first), its key
    // to the row's candidate list.
    const float4 *krow =
        reinterpret_cast<const float4 *>(P.k_r + ((int64_t)b * P.Hkv_r + g) * P.kr_cap * 16);
    float4 kv[kTPT][4];
#pragma unroll
    for (int t = 0; t < kTPT; ++t) {
        if ((anyc >> t) & 1u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[t][j] = krow[(c0 + t * kT + tid) * 4 + j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[t][j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (!cm[h]) continue;
        uint2 *cr = P.ws.cand + ((int64_t)rg * G + h) * P.N;
        uint32_t cpos = S.cgb[h] + (S.wcnt[h][w] >> 16) + (ex[h] >> 16);
#pragma unroll
        for (int t = 0; t < kTPT; ++t) {
            if (!((cm[h] >> t) & 1u)) continue;
            const float k[16] = {kv[t][0].x, kv[t][0].y, kv[t][0].z, kv[t][0].w,
                                 kv[t][1].x, kv[t][1].y, kv[t][1].z, kv[t][1].w,
                                 kv[t][2].x, kv[t][2].y, kv[t][2].z, kv[t][2].w,
                                 kv[t][3].x, kv[t][3].y, kv[t][3].z, kv[t][3].w};
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) acc = __builtin_fmaf(S.qr[h][j], k[j], acc);
            const float sv = (acc == 0.0f) ? 0.0f : acc;
            const uint32_t i = (uint32_t)(c0 + t * kT + tid);
            const uint32_t slot = cpos++;
            if (slot < (uint32_t)P.N) st_cand2(cr + slot, make_uint2(score_key(sv), i));
        }
    }
    wait_vmem();
    __syncthreads();
}

// The idx entries of the block's level-1 kept tokens, from its LDS lists
// (coalesced, agent-scope: the blocks that attend a reducer's rows read
// them).
template <int G>
__device__ __forceinline__ void level1_idx(const LayerParams &P, int b, int g, int64_t c0,
                                           LayerLds &S)
{
    constexpr int cmax = kChunk;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        int32_t *ir = P.idx + ((int64_t)b * P.Hq_r + (int64_t)g * G + h) * P.N;
        const uint32_t kb = S.kgb[h], kc = S.kc[h];
        for (uint32_t e = threadIdx.x; e < kc; e += kT) {
            const uint32_t slot = kb + e;
            if (slot < (uint32_t)P.N) st_agent_i(ir + slot, (int32_t)(c0 + S.b.list[h * cmax + e]));
        }
    }
}

// -------------------------------------------------------- own kept rows

// Attends the block's listed rows of each head (head h: cnt[h] offsets in
// the chunk from S.b.list[h * kChunk + off[h]], off NULL for 0), kBatch
// rows per wave batch, merged into the waves' slots.
template <int G>
__device__ __forceinline__ void gather_lists(const LayerParams &P, int b, int g, int64_t c0,
                                             const uint32_t *off, const uint32_t *cnt, LayerLds &S)
{
    constexpr int cmax = kChunk;
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int lg = lane >> 4, sub = lane & 15;
    if (tid == 0) {
        int acc = 0;
        for (int h = 0; h < G; ++h) {
            S.bpre[h] = acc;
            acc += ((int)cnt[h] + kBatch - 1) / kBatch;
        }
        S.bpre[G] = acc;
    }
    __syncthreads();
    const int nbat = S.bpre[G];
    const int64_t kvb = ((int64_t)b * P.Hkv + g) * P.kv_cap * 128 + sub * 8;
    const uint16_t *Kb = P.K + kvb;
    const uint16_t *Vb = P.V + kvb;
    int cur = -1;
    AttState a;
    att_reset(a);
    float qf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = 0.0f;
    for (int bi = w; bi < nbat; bi += kNW) {
        int h = 0;
        while (h + 1 < G && S.bpre[h + 1] <= bi) ++h;
        if (h != cur) {
            if (cur >= 0) att_flush(a, w, cur, S);
            cur = h;
            att_reset(a);
            load_q8(P.q + ((int64_t)b * P.Hq + (int64_t)g * G + h) * 128 + sub * 8, P.qscale, qf);
        }
        const int base = (bi - S.bpre[h]) * kBatch;
        const int kc = (int)cnt[h];
        const int lo = h * cmax + (off ? (int)off[h] : 0);
        int tok[kRU];
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
            const int e = base + lg + 4 * u;
            tok[u] = e < kc ? (int)(c0 + S.b.list[lo + e]) : -1;
        }
        att_rows(Kb, Vb, qf, tok, P.N, a);
    }
    if (cur >= 0) att_flush(a, w, cur, S);
    __syncthreads();
}

// The row's reducer blocks leave their level-1 rows to the others: block c
// (c < r0, the blocks that reduce nothing) attends, for each head, its share
// [c R / r0, (c + 1) R / r0) of the reducers' level-1 lists (R rows in all,
// tokens read from idx).  Work items (head, batch of kBatch rows) go to the
// waves in turn, so the heads' short shares run side by side.
template <int G>
__device__ __forceinline__ void gather_reducer_rows(const LayerParams &P, int b, int g, int c,
                                                    int r0, int nr, LayerLds &S)
{
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int lg = lane >> 4, sub = lane & 15;
    if (tid < G) {
        uint32_t R = 0;
        for (int q = 0; q < nr; ++q) R += S.pd[q][tid].y;
        const uint32_t lo = (uint32_t)(((uint64_t)R * (uint32_t)c) / (uint32_t)r0);
        const uint32_t hi = (uint32_t)(((uint64_t)R * (uint32_t)(c + 1)) / (uint32_t)r0);
        S.kgb[tid] = lo;  // (the block's own slots are written: reused)
        S.kt[tid] = hi - lo;
    }
    __syncthreads();
    int nbat = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) nbat = max(nbat, ((int)S.kt[h] + kBatch - 1) / kBatch);
    const int64_t kvb = ((int64_t)b * P.Hkv + g) * P.kv_cap * 128 + sub * 8;
    for (int it = w; it < nbat * G; it += kNW) {
        const int h = it % G, bi = it / G;
        const int n = (int)S.kt[h];
        if (bi * kBatch >= n) continue;
        const int32_t *ir = P.idx + ((int64_t)b * P.Hq_r + (int64_t)g * G + h) * P.N;
        float qf[8];
        load_q8(P.q + ((int64_t)b * P.Hq + (int64_t)g * G + h) * 128 + sub * 8, P.qscale, qf);
        int tok[kRU];
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
            const int e = bi * kBatch + lg + 4 * u;
            tok[u] = -1;
            if (e < n) {
                uint32_t pos = S.kgb[h] + (uint32_t)e;
                for (int q = 0; q < nr; ++q) {
                    const uint2 d = S.pd[q][h];
                    if (pos < d.y) {
                        const uint32_t slot = d.x + pos;
                        if (slot < (uint32_t)P.N) tok[u] = ld_agent_i(ir + slot);
                        break;
                    }
                    pos -= d.y;
                }
            }
        }
        AttState a;
        att_reset(a);
        att_rows(P.K + kvb, P.V + kvb, qf, tok, P.N, a);
        att_flush(a, w, h, S);
    }
    __syncthreads();
}

// The block's candidates that the level-2 threshold keeps: those above the
// boundary digit (mode 0) or all of them (mode 1).  They are listed in LDS
// after the head's level-1 list (offsets in the chunk from
// S.b.list[h * kChunk + S.kc[h]], S.n2[h] of them; both lists hold distinct
// tokens of the chunk, so they fit) and written to the head's idx list after
// the ka tokens of level 1 (one slot reservation per head and block).  Then
// the block counts itself on p2_done: it reads no candidate of the row
// after this.
template <int G>
__device__ __forceinline__ void level2_lists(const LayerParams &P, int rg, int b, int g, int64_t c0, LayerLds &S)
{
    constexpr int cmax = kChunk;
    const int tid = threadIdx.x;
    RgCtl &ctl = P.ws.ctl[rg];
    if (tid < G) S.n2[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int mode = S.pick2[h].mode;
        if (mode == 2) continue;
        const int j2 = S.pick2[h].j2;
        const uint32_t cb = S.cgb[h];
        const uint32_t n = min(S.cc[h], (uint32_t)P.N - min(cb, (uint32_t)P.N));
        const uint2 *cr = P.ws.cand + ((int64_t)rg * G + h) * P.N + cb;
        for (uint32_t e0 = 0; e0 < n; e0 += kT) {
            const uint32_t e = e0 + (uint32_t)tid;
            bool keep = false;
            uint32_t off = 0u;
            if (e < n) {
                const uint2 c = ld_cand2(cr + e);
                keep = mode == 1 || fine_digit(key_score(c.x)) > j2;
                off = c.y - (uint32_t)c0;
            }
            const int64_t pos = wave_append(keep, &S.n2[h]) + (int64_t)S.kc[h];
            if (keep && pos < cmax) S.b.list[h * cmax + pos] = (uint16_t)off;
        }
    }
    __syncthreads();
    if (tid < G) {
        S.n2[tid] = min(S.n2[tid], (uint32_t)cmax - S.kc[tid]);
        S.k2b[tid] = S.n2[tid] ? ctr_add(&ctl.kept2[tid], S.n2[tid]) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
        int32_t *ir = P.idx + ((int64_t)b * P.Hq_r + (int64_t)g * G + h) * P.N;
        const uint32_t base = S.pick2[h].ka + S.k2b[h];
        const int lo = h * cmax + (int)S.kc[h];
        for (uint32_t e = tid; e < S.n2[h]; e += kT) {
            const uint32_t slot = base + e;
            if (slot < (uint32_t)P.N) ir[slot] = (int32_t)(c0 + S.b.list[lo + e]);
        }
    }
    if (tid == 0) ctr_arrive(&ctl.p2_done);
}

// One of the row's bpr + G finishers (every block after its level-2 lists,
// every resolver after its resolve).  The last resets the counters that
// outlive the waits on them.
template <int G>
__device__ __forceinline__ void fin_arrive(const LayerParams &P, RgCtl &ctl)
{
    if (ctr_arrive(&ctl.fin_done) != (uint32_t)(P.bpr + G - 1)) return;
    ctr_reset(&ctl.hist_row);
    ctr_reset(&ctl.pick_ready);
    ctr_reset(&ctl.classified);
    ctr_reset(&ctl.pick2_ready);
    ctr_reset(&ctl.p2_done);
#pragma unroll
    for (int h = 0; h < G; ++h) ctr_reset(&ctl.kept2[h]);
    ctr_reset(&ctl.fin_done);
}

// --------------------------------------------------------------- resolve

// Appends kept boundary tokens (one LDS slot reservation per wave): to the
// head's idx list after the rows kept by the blocks, and to the LDS list
// of rows the resolving block attends.  Every lane of the wave must call it.
__device__ __forceinline__ void keep_tok(bool pred, uint32_t tok, int32_t *ir, uint32_t cap,
                                         LayerLds &S)
{
    const uint64_t mask = __ballot(pred);
    if (!mask) return;
    const int leader = __ffsll((unsigned long long)mask) - 1;
    const int lane = lane_id();
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(&S.nkeep, (uint32_t)__popcll(mask));
    base = read_lane(base, leader);
    if (!pred) return;
    const uint64_t below = lane == 0 ? 0ull : (mask & (~0ull >> (64 - lane)));
    const uint32_t pos = base + (uint32_t)__popcll(below);
    if (pos < cap) ir[pos] = (int32_t)tok;
    if (pos < (uint32_t)kBkCap) S.bk[pos] = (int32_t)tok;
}

// Reserves LDS slots in dst for survivors (one LDS atomic per wave).
__device__ __forceinline__ void move_cand(bool pred, const Cand &c, Cand *dst, LayerLds &S)
{
    const uint64_t mask = __ballot(pred);
    if (!mask) return;
    const int leader = __ffsll((unsigned long long)mask) - 1;
    const int lane = lane_id();
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(&S.nmove, (uint32_t)__popcll(mask));
    base = read_lane(base, leader);
    if (!pred) return;
    const uint64_t below = lane == 0 ? 0ull : (mask & (~0ull >> (64 - lane)));
    const uint32_t pos = base + (uint32_t)__popcll(below);
    if (pos < (uint32_t)kResCap) dst[pos] = c;
}

// Candidate k of the current set: from LDS (with its mass) or from memory.
struct CandSet {
    const Cand *lds;
    const uint2 *gc;
    __device__ Cand get(int64_t k, double M, const double *etbl) const
    {
        if (lds) return lds[k];
        const uint2 e = ld_cand2(gc + k);
        Cand c;
        c.key = e.x;
        c.idx = e.y;
        c.e = exp_tang((double)key_score(e.x) - M, etbl);
        return c;
    }
};

// One pass over the current set of n candidates: cls(c) = 0 drop, 1 keep,
// 2 survive.  Survivors go to the LDS buffer dst when to_lds, otherwise are
// compacted in place in memory (in order: positions only move down).
// Returns the number of survivors.
template <class Cls>
__device__ __forceinline__ int64_t filter_pass(const CandSet &cs, int64_t n, Cls cls, bool to_lds, Cand *dst,
                               uint2 *gc, double M, int32_t *ir, uint32_t cap, LayerLds &S)
{
    const int tid = threadIdx.x;
    if (tid == 0) S.nmove = 0;
    __syncthreads();
    int64_t kept_total = 0;
    for (int64_t k0 = 0; k0 < n; k0 += kT) {
        const int64_t k = k0 + tid;
        const bool valid = k < n;
        Cand c;
        c.key = 0;
        c.idx = 0;
        c.e = 0.0;
        if (valid) c = cs.get(k, M, S.etbl);
        const int cl = valid ? cls(c) : 0;
        keep_tok(cl == 1, c.idx, ir, cap, S);
        if (to_lds) {
            move_cand(cl == 2, c, dst, S);
        } else {
            uint32_t tot;
            const uint32_t pos =
                block_exclusive_scan<kT>((uint32_t)(cl == 2), S.a.r.uscan, &tot);
            if (cl == 2) st_cand2(gc + kept_total + pos, make_uint2(c.key, c.idx));
            kept_total += tot;
            wait_vmem();
            __syncthreads();
        }
    }
    __syncthreads();
    return to_lds ? (int64_t)min(S.nmove, (uint32_t)kResCap) : kept_total;
}

// Wave 0 finishes a set of n <= 64 candidates in LDS: ranks them by (score
// key descending, index ascending), lays their masses out in rank order,
// and keeps the shortest rank prefix whose running mass from A reaches Pt
// (all n when none does).
__device__ __forceinline__ void finish_few(const Cand *c, int n, double A, double Pt, int32_t *ir, uint32_t cap,
                           LayerLds &S)
{
    const int l = lane_id();
    const bool v = l < n;
    Cand e;
    e.key = 0;
    e.idx = 0;
    e.e = 0.0;
    if (v) e = c[l];
    int rank = 0;
    for (int k = 0; k < n; ++k) {
        const uint32_t kk = read_lane(e.key, k), ki = read_lane(e.idx, k);
        rank += (kk > e.key || (kk == e.key && ki < e.idx)) ? 1 : 0;
    }
    if (v) S.a.r.tmp[rank] = e.e;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const double wv = v ? S.a.r.tmp[l] : 0.0;
    const double cum = A + wave_inclusive_scan(wv);
    const uint64_t hit = __ballot(v && cum >= Pt);
    const int last = hit ? __ffsll((unsigned long long)hit) - 1 : n - 1;
    keep_tok(v && rank <= last, e.idx, ir, cap, S);
}

// Resolves head h's final candidate set: the candidates of the boundary
// digit (level-2 mode 0) or every candidate (mode 2).  Appends the kept ones
// at ir (room for cap) and leaves their count in S.nkeep.  A set too large
// for LDS is compacted in place in the candidate list, which waits until
// no block reads the list any more.
template <int G>
__device__ __forceinline__ void resolve_set(const LayerParams &P, int rg, int h, int32_t *ir, uint32_t cap,
                            LayerLds &S)
{
    const int tid = threadIdx.x;
    const int N = P.N;
    const Pick2Rec q = S.pick2[h];
    if (q.mode == 1) return;
    const PickRec pk = S.pick[h];
    const double M = (double)pk.M, Pt = pk.Pt;
    double A = q.A2;
    uint2 *gc = P.ws.cand + ((int64_t)rg * G + h) * N;
    CandSet cs{nullptr, gc};
    int cur = 0;
    int64_t n = (int64_t)min(q.nc, (uint32_t)N);
    if (q.mode == 0) {
        const int j2 = q.j2;
        if (q.cstar <= (uint32_t)kResCap) {
            // The boundary digit's candidates into LDS, kU loads in flight
            // per thread; masses for those only.
            if (tid == 0) S.nmove = 0;
            __syncthreads();
            constexpr int kU = 8;
            for (int64_t k0 = 0; k0 < n; k0 += (int64_t)kU * kT) {
                uint2 e[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int64_t k = k0 + u * kT + tid;
                    e[u] = k < n ? ld_cand2(gc + k) : make_uint2(0u, 0u);
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int64_t k = k0 + u * kT + tid;
                    const float sv = key_score(e[u].x);
                    const bool ok = k < n && fine_digit(sv) == j2;
                    Cand c;
                    c.key = e[u].x;
                    c.idx = e[u].y;
                    c.e = ok ? exp_tang((double)sv - M, S.etbl) : 0.0;
                    move_cand(ok, c, S.a.r.buf[0], S);
                }
            }
            __syncthreads();
            n = (int64_t)min(S.nmove, (uint32_t)kResCap);
            cs.lds = S.a.r.buf[0];
        } else {
            // In place in the candidate list, once no block reads it.
            if (tid == 0)
                wait_level(&P.ws.ctl[rg].p2_done, (uint32_t)P.bpr, P.spin_limit, P.status);
            __syncthreads();
            n = filter_pass(
                cs, n, [=](const Cand &x) { return fine_digit(key_score(x.key)) == j2 ? 2 : 0; },
                false, nullptr, gc, M, ir, cap, S);
        }
    }
    n = min(n, (int64_t)cap);
    for (int level = 0; level < 8 && n > 0; ++level) {
        if (!cs.lds && n <= kResCap) {
            for (int64_t k = tid; k < n; k += kT) S.a.r.buf[0][k] = cs.get(k, M, S.etbl);
            __syncthreads();
            cs.lds = S.a.r.buf[0];
            cur = 0;
        }
        if (cs.lds && n <= kWave) {
            if (tid < kWave) finish_few(cs.lds, (int)n, A, Pt, ir, cap, S);
            __syncthreads();
            return;
        }
        // The set's key range: its keys share the bits above the highest
        // bit where the smallest and largest differ.
        if (tid == 0) {
            S.kmin = 0xFFFFFFFFu;
            S.kmax = 0u;
        }
        __syncthreads();
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
        for (int64_t k = tid; k < n; k += kT) {
            const uint32_t key = cs.lds ? cs.lds[k].key : ld_cand2(gc + k).x;
            lo = min(lo, key);
            hi = max(hi, key);
        }
        atomicMin(&S.kmin, lo);
        atomicMax(&S.kmax, hi);
        __syncthreads();
        const uint32_t kmin = S.kmin, kmax = S.kmax;
        if (kmin == kmax) {
            // Every candidate has the same score: keep the c lowest indices,
            // c the smallest count whose mass from A reaches Pt.
            const Cand c0 = cs.get(0, M, S.etbl);
            const double e = c0.e;
            int64_t c = n;
            if (A + (double)n * e >= Pt && e > 0.0) {
                const double need = (Pt - A) / e;
                c = need < 1.0 ? 1 : (int64_t)ceil(need);
                if (c > n) c = n;
                while (c > 1 && A + (double)(c - 1) * e >= Pt) --c;
                while (c < n && A + (double)c * e < Pt) ++c;
            }
            if (c >= n) {
                filter_pass(cs, n, [](const Cand &) { return 1; }, true, nullptr, gc, M, ir, cap,
                            S);
                return;
            }
            // Count-only radix select of the c lowest indices: bits [30:20],
            // [19:10], [9:0].
            int64_t need = c;
            for (int lv = 0; lv < 3 && n > 0 && need > 0; ++lv) {
                const int shift = lv == 0 ? 20 : (lv == 1 ? 10 : 0);
                const uint32_t mask = lv == 0 ? 2047u : 1023u;
                const int nb = (int)mask + 1;
                for (int i = tid; i < nb; i += kT) S.a.r.hc[i] = 0u;
                __syncthreads();
                for (int64_t k = tid; k < n; k += kT) {
                    const uint32_t ix = cs.lds ? cs.lds[k].idx : ld_cand2(gc + k).y;
                    atomicAdd(&S.a.r.hc[(ix >> shift) & mask], 1u);
                }
                __syncthreads();
                if (tid < kWave) {
                    const int per = nb / kWave;
                    const int d0 = tid * per;
                    uint32_t local = 0;
                    for (int q = 0; q < per; ++q) local += S.a.r.hc[d0 + q];
                    const uint32_t incl = wave_inclusive_scan(local);
                    uint32_t run = incl - local;
                    for (int q = 0; q < per; ++q) {
                        const uint32_t cnt = S.a.r.hc[d0 + q];
                        if (cnt && (int64_t)run < need && (int64_t)(run + cnt) >= need) {
                            S.j = (uint32_t)(d0 + q);
                            S.cbefore = run;
                        }
                        run += cnt;
                    }
                }
                __syncthreads();
                const uint32_t D = S.j;
                const int64_t ns = S.a.r.hc[D];
                need -= (int64_t)S.cbefore;
                const bool take_all = need >= ns;
                auto cls = [=](const Cand &x) {
                    const uint32_t d = (x.idx >> shift) & mask;
                    return d < D ? 1 : (d == D ? (take_all ? 1 : 2) : 0);
                };
                const bool to_lds = cs.lds || ns <= kResCap;
                Cand *dst = cs.lds ? S.a.r.buf[cur ^ 1] : S.a.r.buf[0];
                n = filter_pass(cs, n, cls, to_lds, dst, gc, M, ir, cap, S);
                if (take_all) return;
                if (to_lds) {
                    cur = cs.lds ? (cur ^ 1) : 0;
                    cs.lds = S.a.r.buf[cur];
                }
            }
            // Indices are distinct: one token remains, and it is needed.
            if (n > 0 && need > 0) {
                const Cand x = cs.get(0, M, S.etbl);
                if (tid < kWave) keep_tok(tid == 0, x.idx, ir, cap, S);
                __syncthreads();
            }
            return;
        }
        // One 8-bit digit below the shared bits: mass and count per digit.
        const int hb = 31 - __clz(kmin ^ kmax);
        const int shift = hb >= 7 ? hb - 7 : 0;
        if (tid < 256) {
            S.a.r.hm[tid] = 0.0;
            S.a.r.hc[tid] = 0u;
        }
        __syncthreads();
        for (int64_t k = tid; k < n; k += kT) {
            const Cand x = cs.get(k, M, S.etbl);
            const uint32_t d = (x.key >> shift) & 255u;
            atomicAdd(&S.a.r.hm[d], x.e);
            atomicAdd(&S.a.r.hc[d], 1u);
        }
        __syncthreads();
        // Wave 0: the first digit from the top whose running mass from A
        // reaches Pt (lane l owns digits 255 - 4l - [0, 4)); none: keep all.
        if (tid < kWave) {
            const int top = 255 - 4 * tid;
            double wv[4];
            uint32_t cv[4];
            double loc = 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wv[q] = S.a.r.hm[top - q];
                cv[q] = S.a.r.hc[top - q];
                loc += wv[q];
            }
            const double incl = wave_inclusive_scan(loc);
            double cum = A + wave_shift_up(incl);
            int cross = -1;
            double cb = 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cross < 0 && cv[q] != 0u && cum + wv[q] >= Pt) {
                    cross = top - q;
                    cb = cum;
                }
                cum += wv[q];
            }
            const uint64_t cm = __ballot(cross >= 0);
            if (tid == 0) S.flag = cm ? 1 : 0;
            if (cm) {
                const int src = __ffsll((unsigned long long)cm) - 1;
                if (tid == src) {
                    S.j = (uint32_t)cross;
                    S.abefore = cb;
                }
            }
        }
        __syncthreads();
        if (!S.flag) {
            filter_pass(cs, n, [](const Cand &) { return 1; }, true, nullptr, gc, M, ir, cap, S);
            return;
        }
        const uint32_t D = S.j;
        A = S.abefore;
        const int64_t ns = S.a.r.hc[D];
        auto cls = [=](const Cand &x) {
            const uint32_t d = (x.key >> shift) & 255u;
            return d > D ? 1 : (d == D ? 2 : 0);
        };
        const bool to_lds = cs.lds || ns <= kResCap;
        Cand *dst = cs.lds ? S.a.r.buf[cur ^ 1] : S.a.r.buf[0];
        n = filter_pass(cs, n, cls, to_lds, dst, gc, M, ir, cap, S);
        if (to_lds) {
            cur = cs.lds ? (cur ^ 1) : 0;
            cs.lds = S.a.r.buf[cur];
        }
    }
}

// Claimed head h: resolve its final candidate set, write the head's count,
// attend the kept boundary rows and join the head's final merge.
template <int G>
__device__ __forceinline__ void resolve_head(const LayerParams &P, int rg, int b, int g, int h, LayerLds &S)
{
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int lg = lane >> 4, sub = lane & 15;
    RgCtl &ctl = P.ws.ctl[rg];
    const Pick2Rec q = S.pick2[h];
    const uint32_t base = min(q.ka + q.k2, (uint32_t)P.N);
    const uint32_t cap = (uint32_t)P.N - base;
    int32_t *ir = P.idx + ((int64_t)b * P.Hq_r + (int64_t)g * G + h) * P.N + base;
    if (tid == 0) S.nkeep = 0;
    __syncthreads();
    resolve_set<G>(P, rg, h, ir, cap, S);
    __syncthreads();
    const uint32_t kb = min(S.nkeep, cap);
    if (tid == 0) P.count[(int64_t)b * P.Hq_r + (int64_t)g * G + h] = (int32_t)(base + kb);
    // The kept boundary rows (listed in LDS, the rest read back from idx).
    wait_vmem();
    slots_clear(S);
    __syncthreads();
    const int64_t kvb = ((int64_t)b * P.Hkv + g) * P.kv_cap * 128 + sub * 8;
    float qf[8];
    load_q8(P.q + ((int64_t)b * P.Hq + (int64_t)g * G + h) * 128 + sub * 8, P.qscale, qf);
    AttState a;
    att_reset(a);
    bool any = false;
    for (int64_t e0 = (int64_t)w * kBatch; e0 < kb; e0 += (int64_t)kNW * kBatch) {
        int tok[kRU];
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
            const int64_t e = e0 + lg + 4 * u;
            tok[u] = e < kb ? (e < kBkCap ? S.bk[e] : ld_agent_i(ir + e)) : -1;
        }
        att_rows(P.K + kvb, P.V + kvb, qf, tok, P.N, a);
        any = true;
    }
    if (any) att_flush(a, w, 0, S);
    __syncthreads();
    float *bp = P.ws.att2 + (((int64_t)rg * (P.ngrp + 1) + P.ngrp) * kMH + h) * kPF;
    slots_to_partial(1, bp, kPF, S);
    if (arrive_last_blk(&ctl.att_row[h], (uint32_t)P.ngrp + 1u, S)) {
        float *outp = P.out + ((int64_t)b * P.Hq + (int64_t)g * G + h) * 128;
        merge_records(P.ws.att2 + ((int64_t)rg * (P.ngrp + 1) * kMH + h) * kPF,
                      (int64_t)kMH * kPF, P.ngrp + 1, 1, 1u, nullptr, outp);
    }
    __syncthreads();
    if (tid == 0) fin_arrive<G>(P, ctl);
    __syncthreads();
}

// ---------------------------------------------------------------- kernel

template <int G>
__global__ __launch_bounds__(kT) void layer_kernel(LayerParams P)
{
    __shared__ LayerLds S;
    const int tid = threadIdx.x;
    const int blk = blockIdx.x;
    if (blk >= P.NBr) {
        // A block beyond the rows: local heads only (no wait on any block).
        for (int item = blk - P.NBr; item < P.NI; item += P.NX) local_item<G>(P, item, S);
        return;
    }
    const int rg = blk / P.bpr, c = blk - rg * P.bpr;
    const int b = rg / P.Hkv_r, g = rg - b * P.Hkv_r;
    const int grp = c / kGS;
    const int ngs = min(kGS, P.bpr - grp * kGS);
    const int64_t c0 = (int64_t)c * P.C;
    const int cn = (int)min((int64_t)P.C, (int64_t)P.N - c0);
    RgCtl &ctl = P.ws.ctl[rg];

    // ---- scan: the key rows first, then the block's constants to LDS while
    // they arrive; scores in registers
    float4 kv[kTPT][4];
    scan_load(P, b, g, c0, cn, kv);
    asm volatile("" ::: "memory");
    for (int i = tid; i < kMH * kNB; i += kT) S.a.h.hist[i / kNB][i % kNB] = 0.0;
    if (tid < kExpTable) S.etbl[tid] = kLayerExpTbl[tid];
    if (tid < G * 16) S.qr[tid / 16][tid % 16] = P.q_r[((int64_t)b * P.Hq_r + g * G) * 16 + tid];
    __syncthreads();
    switch ((cn + kT - 1) / kT) {
    case 1: block_scan_hist<G, 1>(P, b, g, c0, cn, kv, S); break;
    case 2: block_scan_hist<G, 2>(P, b, g, c0, cn, kv, S); break;
    case 3: block_scan_hist<G, 3>(P, b, g, c0, cn, kv, S); break;
    default: block_scan_hist<G, 4>(P, b, g, c0, cn, kv, S); break;
    }
    {
        HistRec *hr = P.ws.h1 + blk;
        const int hh = tid / kNB, j = tid % kNB;
        if (hh < G) st_agent(&hr->mass[hh][j], S.a.h.hist[hh][j]);
        if (tid < G) {
            st_agent(&hr->m[tid], S.mb[tid]);
            st_agent_i(&hr->T[tid], S.Tb[tid]);
        }
    }
    wait_vmem();
    __syncthreads();
    if (tid == 0) ctr_arrive(&ctl.hist_row);

    // ---- the row's thresholds: head h is reduced by block r0 + h % nr of
    // the row (the last nr blocks), once every block has published
    const int nr = min(G, P.bpr), r0 = P.bpr - nr;
    if (c >= r0) {
        if (tid == 0) wait_level(&ctl.hist_row, (uint32_t)P.bpr, P.spin_limit, P.status);
        __syncthreads();
        uint32_t nh = 0;
        for (int h = c - r0; h < G; h += nr) {
            reduce_head<G>(P, rg, h, S);
            __syncthreads();
            ++nh;
        }
        wait_vmem();
        __syncthreads();
        if (tid == 0) ctr_add(&ctl.pick_ready, nh);
    }

    // ---- local heads while the thresholds are found (blocks that reduce
    // nothing, when there are any), unless blocks beyond the rows take them
    const int nlb = (P.NBr / P.bpr) * r0;
    if (P.NX > 0) {
    } else if (nlb > 0) {
        if (c < r0)
            for (int item = rg * r0 + c; item < P.NI; item += nlb) local_item<G>(P, item, S);
    } else {
        for (int item = blk; item < P.NI; item += P.NBr) local_item<G>(P, item, S);
    }

    if (tid == 0) wait_level(&ctl.pick_ready, (uint32_t)G, P.spin_limit, P.status);
    __syncthreads();
    if (tid < G) {
        const PickRec *pr = P.ws.pick + (int64_t)rg * kMH + tid;
        PickRec r;
        r.M = ld_agent(&pr->M);
        r.T = ld_agent_i(&pr->T);
        r.jstar = ld_agent_i(&pr->jstar);
        r.pad = 0;
        r.A = ld_agent(&pr->A);
        r.Pt = ld_agent(&pr->Pt);
        S.pick[tid] = r;
    }
    __syncthreads();
    classify<G>(P, rg, b, g, c0, cn, S);
    if (tid == 0) ctr_arrive(&ctl.classified);
    level1_idx<G>(P, b, g, c0, S);

    // ---- the heads' level-2 thresholds, by the same blocks as level 1; the
    // other blocks attend their level-1 rows meanwhile
    const bool picker = c >= r0;
    if (picker) {
        if (tid == 0) wait_level(&ctl.classified, (uint32_t)P.bpr, P.spin_limit, P.status);
        __syncthreads();
        uint32_t nh = 0;
        for (int h = c - r0; h < G; h += nr) {
            fine_head<G>(P, rg, h, S);
            __syncthreads();
            ++nh;
        }
        if (r0 > 0 && tid < G) {
            uint2 *pd = P.ws.pdesc + ((int64_t)rg * kMH + (c - r0)) * kMH + tid;
            st_cand2(pd, make_uint2(S.kgb[tid], S.kc[tid]));
        }
        wait_vmem();
        __syncthreads();
        if (tid == 0) ctr_add(&ctl.pick2_ready, nh);
        // Its heads' boundary digits right away, unless a digit holds more
        // candidates than LDS takes (then they are compacted in place, after
        // every block has read the list).
        for (int h = c - r0; h < G; h += nr)
            if (!(S.pick2[h].mode == 0 && S.pick2[h].cstar > (uint32_t)kResCap))
                resolve_head<G>(P, rg, b, g, h, S);
    } else {
        slots_clear(S);
        gather_lists<G>(P, b, g, c0, nullptr, S.kc, S);
    }

    // ---- the block's level-2 rows
    if (tid == 0) wait_level(&ctl.pick2_ready, (uint32_t)G, P.spin_limit, P.status);
    __syncthreads();
    if (tid < G) {
        const Pick2Rec *pr = P.ws.pick2 + (int64_t)rg * kMH + tid;
        Pick2Rec r;
        r.j2 = ld_agent_i(&pr->j2);
        r.mode = ld_agent_i(&pr->mode);
        r.ka = ld_agent(&pr->ka);
        r.k2 = ld_agent(&pr->k2);
        r.cstar = ld_agent(&pr->cstar);
        r.nc = ld_agent(&pr->nc);
        r.A2 = ld_agent(&pr->A2);
        S.pick2[tid] = r;
    }
    if (!picker && tid < nr * G) {
        const int q = tid / G, h = tid % G;
        S.pd[q][h] = ld_cand2(P.ws.pdesc + ((int64_t)rg * kMH + q) * kMH + h);
    }
    __syncthreads();
    level2_lists<G>(P, rg, b, g, c0, S);
    if (tid == 0) fin_arrive<G>(P, ctl);
    if (picker) {
        // The boundary digits left, then the block's level-2 rows (its
        // level-1 rows go to the other blocks; with none, both lists).
        for (int h = c - r0; h < G; h += nr)
            if (S.pick2[h].mode == 0 && S.pick2[h].cstar > (uint32_t)kResCap)
                resolve_head<G>(P, rg, b, g, h, S);
        slots_clear(S);
        if (r0 > 0) {
            gather_lists<G>(P, b, g, c0, S.kc, S.n2, S);
        } else {
            if (tid < G) S.kt[tid] = S.kc[tid] + S.n2[tid];
            gather_lists<G>(P, b, g, c0, nullptr, S.kt, S);
        }
    } else {
        gather_lists<G>(P, b, g, c0, S.kc, S.n2, S);
        gather_reducer_rows<G>(P, b, g, c, r0, nr, S);
    }
    slots_to_partial(G, P.ws.att1 + (int64_t)blk * kMH * kPF, kPF, S);
    if (arrive_last_blk(P.ws.att_grp + (int64_t)rg * P.ngrp + grp, (uint32_t)ngs, S)) {
        float *gp = P.ws.att2 + ((int64_t)rg * (P.ngrp + 1) + grp) * kMH * kPF;
        merge_records(P.ws.att1 + ((int64_t)rg * P.bpr + grp * kGS) * kMH * kPF,
                      (int64_t)kMH * kPF, ngs, G, 0xFFu, gp, nullptr);
        wait_vmem();
        __syncthreads();
        if (tid < G) {
            const bool last = ctr_arrive(&ctl.att_row[tid]) == (uint32_t)P.ngrp;
            if (last) ctr_reset(&ctl.att_row[tid]);
            S.hlast[tid] = last ? 1 : 0;
        }
        __syncthreads();
        uint32_t hm = 0;
        for (int h = 0; h < G; ++h) hm |= S.hlast[h] ? (1u << h) : 0u;
        if (hm) {
            merge_records(P.ws.att2 + (int64_t)rg * (P.ngrp + 1) * kMH * kPF,
                          (int64_t)kMH * kPF, P.ngrp + 1, G, hm, nullptr,
                          P.out + ((int64_t)b * P.Hq + (int64_t)g * G) * 128);
        }
    }
}

}  // namespace

// ------------------------------------------------------------------- host

LayerGeom layer_geom(int cus, int B, int Hq, int Hkv, int N, int Hq_r, int n_sink, int window)
{
    LayerGeom L{};
    L.ok = false;
    if (Hkv < 1 || Hq % Hkv) return L;
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return L;
    if (Hq_r < G || Hq_r % G) return L;
    L.G = G;
    L.Hkv_r = Hq_r / G;
    L.RG = B * L.Hkv_r;
    if (L.RG > cus) return L;
    const int cmax = kChunk;
    int bpr = min(cus / L.RG, kGS * kGS);
    const int64_t want = ((int64_t)N + 1023) / 1024;
    if (want < bpr) bpr = (int)want;
    if (bpr < 1) bpr = 1;
    const int64_t C = ((int64_t)N + bpr - 1) / bpr;
    if (C > cmax) return L;
    L.C = (int)C;
    L.bpr = (int)(((int64_t)N + C - 1) / C);
    L.NB = L.RG * L.bpr;
    L.ngrp = (L.bpr + kGS - 1) / kGS;
    L.n_lkv = Hkv - L.Hkv_r;
    const int64_t w0 = N > window ? (int64_t)N - window : 0;
    const int64_t sink_end = n_sink < w0 ? n_sink : w0;
    L.w0 = (int)w0;
    L.sink_end = (int)sink_end;
    L.nl_rows = (int)(sink_end + (N - w0));
    L.nlt = (L.nl_rows + kTile - 1) / kTile;
    L.NI = L.n_lkv > 0 ? B * L.n_lkv * L.nlt : 0;
    L.NX = L.NI > 0 ? min(cus - L.NB, L.NI) : 0;
    if (L.NX < 0) L.NX = 0;
    L.ok = true;
    return L;
}

static size_t layer_ws_layout(const LayerGeom &L, int B, int N, LayerWs *W, void *base)
{
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes, 256);
        return o;
    };
    const size_t h1 = take((size_t)L.NB * sizeof(HistRec));
    const size_t pk = take((size_t)L.RG * kMH * sizeof(PickRec));
    const size_t p2 = take((size_t)L.RG * kMH * sizeof(Pick2Rec));
    const size_t ctl = take((size_t)L.RG * sizeof(RgCtl));
    const size_t ag = take((size_t)L.RG * L.ngrp * 8);
    const size_t lc = take((size_t)B * (L.n_lkv > 0 ? L.n_lkv : 1) * 8);
    const size_t a1 = take((size_t)L.NB * kMH * kPF * sizeof(float));
    const size_t a2 = take((size_t)L.RG * (L.ngrp + 1) * kMH * kPF * sizeof(float));
    const size_t lo = take((size_t)(L.NI > 0 ? L.NI : 1) * kMH * kPF * sizeof(float));
    const size_t cd = take((size_t)L.RG * L.G * N * sizeof(uint2));
    const size_t pd = take((size_t)L.RG * kMH * kMH * sizeof(uint2));
    if (W) {
        char *p = static_cast<char *>(base);
        W->h1 = reinterpret_cast<HistRec *>(p + h1);
        W->pick = reinterpret_cast<PickRec *>(p + pk);
        W->pick2 = reinterpret_cast<Pick2Rec *>(p + p2);
        W->ctl = reinterpret_cast<RgCtl *>(p + ctl);
        W->att_grp = reinterpret_cast<unsigned long long *>(p + ag);
        W->loc_ctr = reinterpret_cast<unsigned long long *>(p + lc);
        W->att1 = reinterpret_cast<float *>(p + a1);
        W->att2 = reinterpret_cast<float *>(p + a2);
        W->loc = reinterpret_cast<float *>(p + lo);
        W->cand = reinterpret_cast<uint2 *>(p + cd);
        W->pdesc = reinterpret_cast<uint2 *>(p + pd);
    }
    return off;
}

size_t layer_ws_bytes(const LayerGeom &L, int B, int N)
{
    return layer_ws_layout(L, B, N, nullptr, nullptr);
}

hipError_t launch_decode_layer(const LayerGeom &L, const float *q_r, const float *k_r,
                               int64_t kr_cap, const uint16_t *q, const uint16_t *K,
                               const uint16_t *V, int64_t kv_cap, int B, int Hq, int Hkv, int N,
                               int Hq_r, float p, float scale, float *out, int32_t *idx,
                               int32_t *count, float *scores, void *ws, uint32_t spin_limit,
                               uint32_t *status, hipStream_t stream)
{
    LayerParams P{};
    P.q_r = q_r;
    P.k_r = k_r;
    P.q = q;
    P.K = K;
    P.V = V;
    P.out = out;
    P.idx = idx;
    P.count = count;
    P.scores = scores;
    P.kr_cap = kr_cap;
    P.kv_cap = kv_cap;
    P.B = B;
    P.Hq = Hq;
    P.Hkv = Hkv;
    P.N = N;
    P.Hq_r = Hq_r;
    P.Hkv_r = L.Hkv_r;
    P.bpr = L.bpr;
    P.C = L.C;
    P.ngrp = L.ngrp;
    P.n_lkv = L.n_lkv;
    P.nlt = L.nlt;
    P.NI = L.NI;
    P.NBr = L.NB;
    P.NX = L.NX;
    P.nl_rows = L.nl_rows;
    P.sink_end = L.sink_end;
    P.w0 = L.w0;
    P.keep_all = p >= 1.0f ? 1 : 0;
    P.pd = (double)p;
    P.qscale = scale * kLog2eF;
    P.spin_limit = spin_limit;
    P.status = status;
    layer_ws_layout(L, B, N, &P.ws, ws);
    const dim3 grid((unsigned)(L.NB + L.NX)), block(kT);
    switch (L.G) {
    case 1: return launch(layer_kernel<1>, grid, block, 0, stream, P);
    case 2: return launch(layer_kernel<2>, grid, block, 0, stream, P);
    case 4: return launch(layer_kernel<4>, grid, block, 0, stream, P);
    default: return launch(layer_kernel<8>, grid, block, 0, stream, P);
    }
}

}  // namespace rtp
