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
// scale*log2(e) folded into q); its partial (max, sum, o[128]) record is
// merged inside the same kernel in two levels (groups of splits, then the
// groups).
//
// Local heads: the 8 query heads of a KV head share each row read.  Each lane
// forms 8 partial dot products; a butterfly over the 16 lanes of a row
// reduces all 8 in 8 exchanges (each step halves the heads a lane carries).
#include <float.h>
#include <atomic>
#include <math.h>

#include "rtp_device.h"
#include "rtp_launch.h"
#include "scan_tile.h"

namespace rtp {

constexpr int kAttThreads = 256;
constexpr int kGroups = kAttThreads / 16;  // 16-lane row groups per block
constexpr int kPart = 132;                 // floats per partial: m, l, pad, o[128]
constexpr int kSparseU = 8;                // rows per group per iteration
constexpr int kLocalU = 4;
constexpr int kLocalRows = 64;       // rows per local split (at least)
constexpr int kMaxLocalSplits = 128;
constexpr float kLog2e = 1.4426950408889634f;

// Sum over each row of 16 lanes, in every lane of the row (DPP: quads,
// then mirrored halves, then mirrored rows).
__device__ __forceinline__ float sum16(float v)
{
    v += dpp<kDppQuadXor1>(v, v);
    v += dpp<kDppQuadXor2>(v, v);
    v += dpp<kDppRowHalfMirror>(v, v);
    v += dpp<kDppRowMirror>(v, v);
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
constexpr int kSlice = 32;  // split partials merged per block in the first merge level
constexpr int kMaxSlices = (kSparseTarget + 1 + kSlice - 1) / kSlice;
static_assert(kMaxSlices <= kSlice, "the second merge level takes at most kSlice partials");

int sparse_grid(int64_t R) { return (int)(kSparseTarget + R); }

struct SparseWs {
    float *part;           // one partial per attention block
    float *super;          // [R][kMaxSlices] slice merges
    uint32_t *part_flag;   // one hand-off flag per partial
    uint32_t *super_flag;  // [R][kMaxSlices]
    WaitCtl wc;            // poll limit of the flag waits, where a give-up is reported
};

static size_t sparse_ws_layout(int64_t R, SparseWs *W, void *base)
{
    size_t off = 0;
    const size_t part = off;
    off += align_up((size_t)sparse_grid(R) * kPart * sizeof(float), 256);
    const size_t sup = off;
    off += align_up((size_t)R * kMaxSlices * kPart * sizeof(float), 256);
    const size_t pf = off;
    off += align_up((size_t)sparse_grid(R) * sizeof(uint32_t), 256);
    const size_t sf = off;
    off += align_up((size_t)R * kMaxSlices * sizeof(uint32_t), 256);
    if (W) {
        char *b = static_cast<char *>(base);
        W->part = reinterpret_cast<float *>(b + part);
        W->super = reinterpret_cast<float *>(b + sup);
        W->part_flag = reinterpret_cast<uint32_t *>(b + pf);
        W->super_flag = reinterpret_cast<uint32_t *>(b + sf);
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

// Every thread of the block must call this; all get the same plan.  Wave 0
// computes it (one pass over the counts, 64 head rows at a time) and
// publishes it through LDS, so the block pays one barrier.  Finds either the
// split that global index j falls in (j >= 0) or, for j < 0, the splits of
// head row `row`.
__device__ SplitPlan plan_splits(const int32_t *count, int R, int N, int rows_per_iter, int j,
                                 int row, SplitPlan *sh)
{
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        int64_t tot = 0;
        for (int r = lane; r < R; r += kWave) tot += clamp_count(count[r], N);
        const int64_t T = wave_sum(tot);
        int64_t chunk = (T + kSparseTarget - 1) / kSparseTarget;
        if (chunk < rows_per_iter) chunk = rows_per_iter;
        chunk = (chunk + rows_per_iter - 1) / rows_per_iter * rows_per_iter;
        int base = 0, hit_r = -1, hit_first = 0, hit_splits = 0;
        for (int r0 = 0; r0 < R; r0 += kWave) {
            const int r = r0 + lane;
            const int sp = r < R ? (int)((clamp_count(count[r], N) + chunk - 1) / chunk) : 0;
            const int inc = wave_inclusive_scan(sp);
            const int first = base + inc - sp;
            const bool hit = r < R && (j >= 0 ? (j >= first && j < first + sp) : r == row);
            const uint64_t hm = __ballot(hit);
            if (hm && hit_r < 0) {
                const int src = __ffsll((unsigned long long)hm) - 1;
                hit_r = __shfl(r, src);
                hit_first = __shfl(first, src);
                hit_splits = __shfl(sp, src);
            }
            base += __shfl(inc, kWave - 1);
        }
        if (lane == 0) {
            sh->chunk = (int)chunk;
            sh->r = hit_r;
            sh->first = hit_first;
            sh->splits = hit_splits;
        }
    }
    __syncthreads();
    return *sh;
}

// Counts this block on `ctr` once its agent-scope stores have completed,
// and tells whether it was the last of `expected` blocks; the last one then
// reads the others' results with agent-scope loads.
__device__ bool arrive_last(unsigned long long *ctr, int expected, int *flag)
{
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        *flag = ctr_arrive(ctr) == (uint32_t)(expected - 1);
        if (*flag) ctr_reset(ctr);
    }
    __syncthreads();
    return *flag != 0;
}

// Merges n <= kSlice partials (max, sum, o[128]) with a block of
// kAttThreads (two groups of 128 threads, one per output dimension, take
// alternate partials).  Writes a merged partial (dst_part) or the
// normalised output row (dst_out).
struct MergeShared {
    float f[kSlice];
    float o[kAttThreads / 128][128];
    float M, L;
};

__device__ void merge_partials(const float *pr, int n, float *dst_part, float *dst_out,
                               MergeShared &S)
{
    constexpr int kG = kAttThreads / 128;
    constexpr int kPer = kSlice / kG;   // partials per thread
    constexpr int kW = (kSlice + kWave - 1) / kWave;  // partials per lane of wave 0
    const int tid = threadIdx.x;
    const int c = tid & 127, grp = tid >> 7;
    // Every load is issued before any is used: the output columns of this
    // thread's partials, and (wave 0) their max and sum.
    float ov[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int k = grp + i * kG;
        ov[i] = k < n ? ld_agent(pr + (int64_t)k * kPart + 4 + c) : 0.0f;
    }
    if (tid < kWave) {
        // wave 0: the merged max, the factors and the merged sum
        float m[kW], lp[kW];
        float mm = -INFINITY;
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            const int k = tid + i * kWave;
            m[i] = k < n ? ld_agent(pr + (int64_t)k * kPart) : -INFINITY;
            lp[i] = k < n ? ld_agent(pr + (int64_t)k * kPart + 1) : 0.0f;
            mm = fmaxf(mm, m[i]);
        }
        const float M = wave_max(mm);
        float ls = 0.0f;
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            const int k = tid + i * kWave;
            const float f = k < n ? rescale(m[i], M) : 0.0f;
            ls = fmaf(lp[i], f, ls);
            if (k < n) S.f[k] = f;
        }
        const float l = wave_sum(ls);
        if (tid == 0) {
            S.M = M;
            S.L = l;
        }
    }
    __syncthreads();
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int k = grp + i * kG;
        if (k < n) o = fmaf(ov[i], S.f[k], o);
    }
    S.o[grp][c] = o;
    __syncthreads();
    if (grp == 0) {
        float t = 0.0f;
#pragma unroll
        for (int g = 0; g < kG; ++g) t += S.o[g][c];
        if (dst_out) dst_out[c] = S.L > 0.0f ? t / S.L : 0.0f;
        if (dst_part) {
            st_agent(dst_part + 4 + c, t);
            if (c == 0) {
                st_agent(dst_part, S.M);
                st_agent(dst_part + 1, S.L);
            }
        }
    }
    __syncthreads();
}

struct SparseShared {
    float wm[kAttThreads / kWave], wl[kAttThreads / kWave];
    float wo[kAttThreads / kWave][128];
    SplitPlan plan;
    MergeShared ms;
};

// Per-head sparse attention, split blk of the plan over all heads' kept rows.
__device__ void sparse_block(const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
                             const uint16_t *__restrict__ V, const int32_t *__restrict__ idx,
                             const int32_t *__restrict__ count, int N, int64_t kv_cap, int Hq,
                             int Hkv, int q_head_begin, int n_q, int R, float qscale,
                             const SparseWs &W, float *__restrict__ out, int blk,
                             SparseShared &SS)
{
    float *wm = SS.wm, *wl = SS.wl;
    float(*wo)[128] = SS.wo;
    MergeShared &MS = SS.ms;
    constexpr int kRowsPerIter = kGroups * kSparseU;
    const SplitPlan plan = plan_splits(count, R, N, kRowsPerIter, blk, -1, &SS.plan);
    if (plan.r < 0) return;  // past the last split: no partial to write
    const int prow = plan.r;
    const int b = prow / n_q, hr = prow % n_q;
    const int h = q_head_begin + hr;
    const int g = h / (Hq / Hkv);
    float *pr = W.part + (int64_t)blk * kPart;
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

    // The next iteration's row indices are requested while this one's rows
    // are gathered and used.
    int tn[kSparseU];
    auto load_idx = [&](int base) {
#pragma unroll
        for (int u = 0; u < kSparseU; ++u) {
            const int j = base + u * kGroups + w * 4 + grp;
            tn[u] = j < end ? ir[j] : -1;
        }
    };
    if (begin < end) load_idx(begin);
    for (int base = begin; base < end; base += kRowsPerIter) {
        uint4 kw[kSparseU], vw[kSparseU];
        bool ok[kSparseU];
#pragma unroll
        for (int u = 0; u < kSparseU; ++u) {
            ok[u] = (unsigned)tn[u] < (unsigned)N;
            const int64_t off = ok[u] ? (int64_t)tn[u] * 128 : 0;
            kw[u] = ld_nt16(Kb + off);
            vw[u] = ld_nt16(Vb + off);
        }
        if (base + kRowsPerIter < end) load_idx(base + kRowsPerIter);
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
        st_agent(pr + 4 + threadIdx.x, O);
        if (threadIdx.x == 0) {
            st_agent(pr, M);
            st_agent(pr + 1, L);
        }
    }

    // Two-level merge inside the kernel.  The last split of each slice of
    // kSlice splits merges the slice once the slice's other blocks have
    // published their partials; the merger of the row's last slice merges
    // the slices once the other slice mergers have published theirs.  A
    // merger waits only for blocks with lower indices.
    const int k = blk - plan.first;
    const int slice = k / kSlice;
    const int slices = (plan.splits + kSlice - 1) / kSlice;
    const int in_slice = min(kSlice, plan.splits - slice * kSlice);
    const int k0 = plan.first + slice * kSlice;  // the slice's first block
    float *dst = out + ((int64_t)b * Hq + h) * 128;
    if (blk != k0 + in_slice - 1) {
        publish_flag(W.part_flag + blk);
        return;
    }
    wait_vmem();  // this block's own partial, read back below by other threads
    await_flags(W.part_flag + k0, in_slice - 1, W.wc);
    const float *first = W.part + (int64_t)k0 * kPart;
    if (slices == 1) {
        merge_partials(first, in_slice, nullptr, dst, MS);
        return;
    }
    float *sp = W.super + ((int64_t)prow * kMaxSlices) * kPart;
    uint32_t *sf = W.super_flag + (int64_t)prow * kMaxSlices;
    merge_partials(first, in_slice, sp + (int64_t)slice * kPart, nullptr, MS);
    if (slice != slices - 1) {
        publish_flag(sf + slice);
        return;
    }
    wait_vmem();
    await_flags(sf, slices - 1, W.wc);
    merge_partials(sp, slices, nullptr, dst, MS);
}

// ------------------------------------------- 8 query heads per KV row
//
// Local heads and the union mode of sparse heads read each K/V row once for
// all (up to 8) query heads of its KV head that attend it.  A row is spread
// over 16 lanes (8 bf16 each); each lane forms 8 partial dot products, and a
// butterfly over the 16 lanes reduces all 8 in 8 exchanges (each step
// halves the heads a lane carries).  Each block produces one partial
// (max, sum, o[128]) per head for its split; splits are merged in two levels
// inside the kernel, as for the per-head sparse kernel.

struct GroupWs {
    float *part;                    // [R][S] per-split partials
    float *super;                   // [R][max_slices] slice merges
    unsigned long long *slice_ctr;  // [R][max_slices], by a chunk's first head row
    unsigned long long *group_ctr;  // [R]
    int slice;                      // splits merged per block, first level
    int max_slices;
};

static size_t group_ws_layout(int64_t R, int max_splits, int slice, GroupWs *W, void *base)
{
    const int max_slices = (max_splits + slice - 1) / slice;
    size_t off = 0;
    const size_t part = off;
    off += align_up((size_t)R * max_splits * kPart * sizeof(float), 256);
    const size_t sup = off;
    off += align_up((size_t)R * max_slices * kPart * sizeof(float), 256);
    const size_t sc = off;
    off += align_up((size_t)R * max_slices * sizeof(unsigned long long), 256);
    const size_t gc = off;
    off += align_up((size_t)R * sizeof(unsigned long long), 256);
    if (W) {
        char *b = static_cast<char *>(base);
        W->part = reinterpret_cast<float *>(b + part);
        W->super = reinterpret_cast<float *>(b + sup);
        W->slice_ctr = reinterpret_cast<unsigned long long *>(b + sc);
        W->group_ctr = reinterpret_cast<unsigned long long *>(b + gc);
        W->slice = slice;
        W->max_slices = max_slices;
    }
    return off;
}

// Merges n partials for each of nh <= 8 heads at once: thread t takes head
// t/32 and output dimensions 4*(t%32) .. +3.  Head hh's partials start at
// first + hh*head_stride (floats), kPart apart.  Writes merged partials
// (dst_part, same head stride) or output rows (dst_out, 128 apart).
__device__ void merge_heads(const float *first, int64_t head_stride, int n, int nh,
                            float *dst_part, int64_t dst_stride, float *dst_out)
{
    const int hh = threadIdx.x >> 5, d = (threadIdx.x & 31) * 4;
    if (hh >= nh) return;
    const float *src = first + hh * head_stride;
    // One pass: kB partials loaded together, merged with a running max.
    constexpr int kB = 8;
    float M = -INFINITY, L = 0.0f;
    float O[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < n; k0 += kB) {
        float pm[kB], pl[kB];
        float4 po[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const bool ok = k0 + u < n;
            const float *pk = src + (int64_t)(ok ? k0 + u : k0) * kPart;
            pm[u] = ok ? ld_agent(pk) : -INFINITY;
            pl[u] = ld_agent(pk + 1);
            po[u] = make_float4(ld_agent(pk + 4 + d), ld_agent(pk + 5 + d), ld_agent(pk + 6 + d),
                                ld_agent(pk + 7 + d));
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < kB; ++u) mb = fmaxf(mb, pm[u]);
        if (mb == -INFINITY) continue;
        const float c = rescale(M, mb);
        L *= c;
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] *= c;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const float f = rescale(pm[u], mb);
            L = fmaf(pl[u], f, L);
            O[0] = fmaf(po[u].x, f, O[0]);
            O[1] = fmaf(po[u].y, f, O[1]);
            O[2] = fmaf(po[u].z, f, O[2]);
            O[3] = fmaf(po[u].w, f, O[3]);
        }
        M = mb;
    }
    if (dst_out) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        *reinterpret_cast<float4 *>(dst_out + hh * 128 + d) =
            make_float4(O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv);
    }
    if (dst_part) {
        float *pd = dst_part + hh * dst_stride;
#pragma unroll
        for (int e = 0; e < 4; ++e) st_agent(pd + 4 + d + e, O[e]);
        if (d == 0) {
            st_agent(pd, M);
            st_agent(pd + 1, L);
        }
    }
}

// After split s of S has stored its partials for heads r0 .. r0 + nh - 1:
// the two-level merge of the splits, for all nh heads at once (counters
// indexed by r0).  The last block of a slice merges the slice; the last
// slice merger writes the output rows dst (128 floats apart).
// `merge` has merge_heads' signature (first, head_stride, n, nh, dst_part,
// dst_stride, dst_out).
template <class Merge>
__device__ void merge_group_splits(int nh, int s, int S, int64_t r0, const GroupWs &W,
                                   float *dst, int *last, Merge merge)
{
    const int slice = s / W.slice;
    const int slices = (S + W.slice - 1) / W.slice;
    const int in_slice = min(W.slice, S - slice * W.slice);
    if (!arrive_last(W.slice_ctr + r0 * W.max_slices + slice, in_slice, last)) return;
    const float *first = W.part + (r0 * S + slice * W.slice) * kPart;
    if (slices == 1) {
        merge(first, (int64_t)S * kPart, in_slice, nh, nullptr, 0, dst);
        return;
    }
    float *sp = W.super + r0 * W.max_slices * kPart;
    merge(first, (int64_t)S * kPart, in_slice, nh, sp + (int64_t)slice * kPart,
          (int64_t)W.max_slices * kPart, nullptr);
    if (!arrive_last(W.group_ctr + r0, slices, last)) return;
    merge(sp, (int64_t)W.max_slices * kPart, slices, nh, nullptr, 0, dst);
}

// Per-lane state of the 8-head online softmax.  A row is spread over 16
// lanes (8 bf16 each, one 16-B load); each lane forms 8 partial dot
// products, and a butterfly over the 16 lanes reduces all 8 in 8 exchanges
// (each step halves the heads a lane carries).  A wave works on 4 rows at a
// time, kLocalU times over, before it updates the softmax state.
struct Heads8 {
    float qf[8][8];  // q * scale * log2(e), this lane's 8 dimensions
    float m[8], l[8], o[8][8];
    int b3, b2, b1;  // lane bits of the butterfly
};

__device__ __forceinline__ void heads8_init(Heads8 &st, const uint16_t *__restrict__ q, int64_t q0,
                                            int nh, float qscale, int sub)
{
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        if (hh < nh) {
            const uint4 qw = *reinterpret_cast<const uint4 *>(q + q0 + hh * 128 + sub * 8);
            bf16x8_to_f32(qw, st.qf[hh]);
#pragma unroll
            for (int c = 0; c < 8; ++c) st.qf[hh][c] *= qscale;
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) st.qf[hh][c] = 0.0f;
        }
        st.m[hh] = -INFINITY;
        st.l[hh] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) st.o[hh][c] = 0.0f;
    }
    st.b3 = (sub >> 3) & 1;
    st.b2 = (sub >> 2) & 1;
    st.b1 = (sub >> 1) & 1;
}

// One online-softmax step over kLocalU rows of this lane group: kw/vw hold
// the rows' K and V (8 bf16 per lane), bit hh of hb[u] says whether head hh
// attends row u.
__device__ __forceinline__ void heads8_step(Heads8 &st, const uint4 (&kw)[kLocalU],
                                            const uint4 (&vw)[kLocalU],
                                            const uint32_t (&hb)[kLocalU])
{
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
            for (int c = 0; c < 8; ++c) a = fmaf(st.qf[hh][c], kf[c], a);
            d[hh] = a;
        }
        // Butterfly: after the steps over lane bits 3, 2, 1 a lane holds
        // one head, 4*b3 + 2*b2 + b1, summed over 8 lanes; bit 0 finishes.
        float d4[4], d2[2], d1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float send = st.b3 ? d[k] : d[k + 4];
            const float keep = st.b3 ? d[k + 4] : d[k];
            d4[k] = keep + __shfl_xor(send, 8, 16);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float send = st.b2 ? d4[k] : d4[k + 2];
            const float keep = st.b2 ? d4[k + 2] : d4[k];
            d2[k] = keep + __shfl_xor(send, 4, 16);
        }
        {
            const float send = st.b1 ? d2[0] : d2[1];
            const float keep = st.b1 ? d2[1] : d2[0];
            d1 = keep + __shfl_xor(send, 2, 16);
        }
        d1 += __shfl_xor(d1, 1, 16);
        // Head hh's logit sits in lanes 2*hh and 2*hh + 1 of the group.
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const float v = __shfl(d1, 2 * hh, 16);
            lg[u][hh] = (hb[u] >> hh) & 1u ? v : -INFINITY;
        }
    }
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        float mx = lg[0][hh];
#pragma unroll
        for (int u = 1; u < kLocalU; ++u) mx = fmaxf(mx, lg[u][hh]);
        const float mn = fmaxf(st.m[hh], mx);
        if (mn == -INFINITY) continue;
        const float corr = rescale(st.m[hh], mn);
        st.l[hh] *= corr;
#pragma unroll
        for (int c = 0; c < 8; ++c) st.o[hh][c] *= corr;
        st.m[hh] = mn;
    }
#pragma unroll
    for (int u = 0; u < kLocalU; ++u) {
        float vf[8];
        bf16x8_to_f32(vw[u], vf);
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const float pw = (hb[u] >> hh) & 1u ? exp2f(lg[u][hh] - st.m[hh]) : 0.0f;
            st.l[hh] += pw;
#pragma unroll
            for (int c = 0; c < 8; ++c) st.o[hh][c] = fmaf(pw, vf[c], st.o[hh][c]);
        }
    }
}

struct Heads8Shared {
    float wm[kAttThreads / kWave][8], wl[kAttThreads / kWave][8];
    float wo[kAttThreads / kWave][8][128];
    int last;
};

// Merges the block's lane groups and waves into one partial per head for
// split s of S, then
// merges the splits: the last block of a slice merges the slice, the last
// slice merger writes out[b][h_lo .. h_lo + nh).  Rows of the partials are
// R = B * n_q, head row r0 = b * n_q + (h_lo - q_head_begin).
__device__ void heads8_finish(Heads8 &st, Heads8Shared &sh, int nh, int s, int S, int64_t r0,
                              const GroupWs &W, float *dst)
{
    const int lane = lane_id(), w = threadIdx.x / kWave, sub = lane & 15;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
#pragma unroll
        for (int off = 16; off < kWave; off <<= 1) {
            const float mo = __shfl_xor(st.m[hh], off);
            const float lo = __shfl_xor(st.l[hh], off);
            const float mn = fmaxf(st.m[hh], mo);
            const float a = rescale(st.m[hh], mn), bb = rescale(mo, mn);
            st.l[hh] = st.l[hh] * a + lo * bb;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float oo = __shfl_xor(st.o[hh][c], off);
                st.o[hh][c] = st.o[hh][c] * a + oo * bb;
            }
            st.m[hh] = mn;
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
#pragma unroll
            for (int c = 0; c < 8; ++c) sh.wo[w][hh][sub * 8 + c] = st.o[hh][c];
            if (lane == 0) {
                sh.wm[w][hh] = st.m[hh];
                sh.wl[w][hh] = st.l[hh];
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nh * 128; e += kAttThreads) {
        const int hh = e / 128, c = e % 128;
        float M = -INFINITY;
        for (int i = 0; i < kAttThreads / kWave; ++i) M = fmaxf(M, sh.wm[i][hh]);
        float L = 0.0f, O = 0.0f;
        for (int i = 0; i < kAttThreads / kWave; ++i) {
            const float f = rescale(sh.wm[i][hh], M);
            L += sh.wl[i][hh] * f;
            O += sh.wo[i][hh][c] * f;
        }
        float *pr = W.part + ((r0 + hh) * S + s) * kPart;
        st_agent(pr + 4 + c, O);
        if (c == 0) {
            st_agent(pr, M);
            st_agent(pr + 1, L);
        }
    }

    merge_group_splits(nh, s, S, r0, W, dst, &sh.last,
                       [](const float *first, int64_t hs, int n, int nh_, float *dp, int64_t ds,
                          float *dout) { merge_heads(first, hs, n, nh_, dp, ds, dout); });
}

// Heads of KV head g handled by block row y: chunk ck of up to 8 query heads
// of g within [q_head_begin, q_head_begin + n_q).
struct HeadChunk {
    int g, h_lo, nh;
};

__device__ __forceinline__ HeadChunk head_chunk(int y, int G, int q_head_begin, int n_q,
                                                int chunks_per_g)
{
    HeadChunk c;
    c.g = q_head_begin / G + y / chunks_per_g;
    const int ck = y % chunks_per_g;
    c.h_lo = max(q_head_begin, c.g * G + ck * 8);
    const int h_hi = min(q_head_begin + n_q, min(c.g * G + G, c.g * G + ck * 8 + 8));
    c.nh = h_hi - c.h_lo;
    return c;
}

// ------------------------------------------------------------- local
//
// Local heads: each K/V row is read once for the (up to 8) query heads of a
// chunk of its KV head.  Two 16-lane groups take each row, one for heads 0-3
// of the chunk and one for heads 4-7 (their loads of the row are the same
// lines); a lane holds 8 dims of the row and forms 4 partial dot products.
// A butterfly over the 16 lanes leaves each head's full dot in 4 lanes:
// lanes i and i^8 trade head pairs {0,1} / {2,3}, lanes i and i^7 trade the
// heads of the pair, then i^2 and i^1 add; head 2*b3 + b2 (lane bits) ends
// in lanes 4h .. 4h+3, and a per-row broadcast hands every lane all 4.
// All exchanges are DPP moves.

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

constexpr int kLocalSlice = 16;  // split partials merged per block, first level

// The row list never exceeds N rows, so sizing with N bounds every
// n_sink / window.
size_t local_ws_bytes(int64_t B, int64_t n_q, int N)
{
    return group_ws_layout(B * n_q, local_splits(N), kLocalSlice, nullptr, nullptr);
}

constexpr int kLocSlots = kAttThreads / 32;         // rows in progress per block step

constexpr int kLocTile = 64;  // rows staged in LDS at a time

// Factors of one merge of split partials: per head, the merged max and sum
// and each partial's weight.
struct HeadMergeShared {
    float f[8][kLocalSlice];
    float M[8], L[8];
};

struct LocalShared {
    union {
        struct {  // a tile of K and V rows (16 pieces of 16 B per row)
            uint4 k[kLocTile][16], v[kLocTile][16];
        } st;
        struct {  // the row slots' softmax states, merged per head
            float m[kLocSlots][8], l[kLocSlots][8];
            float o[kLocSlots][8][128];
        } mg;
        HeadMergeShared hm;
    };
    int last;
};

__device__ __forceinline__ float max16(float v)
{
    v = fmaxf(v, dpp<kDppQuadXor1>(v, v));
    v = fmaxf(v, dpp<kDppQuadXor2>(v, v));
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v, v));
    v = fmaxf(v, dpp<kDppRowMirror>(v, v));
    return v;
}

// Merges n <= kLocalSlice split partials for each of nh <= 8 heads with one
// round of loads, all in flight together: thread t owns output column
// t % 128 of heads t / 128 + 2j (j < 4), so each load instruction of a wave
// reads 256 contiguous bytes of one partial; threads 0..127 take the max
// and sum of partial t % 16 of head t / 16 (one head per 16-lane row, so
// the per-head max and sum are row reductions), and the weights go through
// LDS.  Head hh's partials start at first + hh * head_stride (floats),
// kPart apart.  Writes merged partials (dst_part, dst_stride apart) or
// output rows (dst_out, 128 apart).
__device__ void merge_heads16(const float *first, int64_t head_stride, int n, int nh,
                              float *dst_part, int64_t dst_stride, float *dst_out,
                              HeadMergeShared &S)
{
    constexpr int kG = kAttThreads / 128;  // thread groups, one head each at a time
    constexpr int kH = 8 / kG;             // heads per thread
    static_assert(8 * kLocalSlice <= kAttThreads, "one thread per (head, partial)");
    const int tid = threadIdx.x, c = tid & 127, g = tid >> 7;
    float ov[kH][kLocalSlice];
#pragma unroll
    for (int j = 0; j < kH; ++j) {
        const int hh = g + j * kG;
        const float *ph = first + hh * head_stride + 4 + c;
#pragma unroll
        for (int k = 0; k < kLocalSlice; ++k)
            ov[j][k] = hh < nh && k < n ? ld_agent(ph + k * kPart) : 0.0f;
    }
    if (tid < 8 * kLocalSlice) {
        const int hh = tid / kLocalSlice, k = tid % kLocalSlice;
        const bool ok = hh < nh && k < n;
        const float *pk = first + hh * head_stride + k * kPart;
        const float m = ok ? ld_agent(pk) : -INFINITY;
        const float l = ok ? ld_agent(pk + 1) : 0.0f;
        const float M = max16(m);
        const float f = ok ? rescale(m, M) : 0.0f;
        const float L = sum16(l * f);
        S.f[hh][k] = f;
        if (k == 0) {
            S.M[hh] = M;
            S.L[hh] = L;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kH; ++j) {
        const int hh = g + j * kG;
        if (hh >= nh) continue;
        float o = 0.0f;
#pragma unroll
        for (int k = 0; k < kLocalSlice; ++k) o = fmaf(ov[j][k], S.f[hh][k], o);
        const float L = S.L[hh];
        if (dst_out) dst_out[hh * 128 + c] = o * (L > 0.0f ? 1.0f / L : 0.0f);
        if (dst_part) {
            float *pd = dst_part + hh * dst_stride;
            st_agent(pd + 4 + c, o);
            if (c == 0) {
                st_agent(pd, S.M[hh]);
                st_agent(pd + 1, L);
            }
        }
    }
}

struct Heads4 {
    float qf[4][8];  // q * scale * log2(e) of this group's heads, this lane's 8 dims
    float m[4], l[4], o[4][8];
};

// q words (8 bf16 of this lane's dims for each of the group's 4 heads, zero
// for heads past the chunk) to the scaled fp32 state; softmax state empty.
__device__ __forceinline__ void heads4_init(Heads4 &st, const uint4 (&qw)[4], float qscale)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bf16x8_to_f32(qw[k], st.qf[k]);
#pragma unroll
        for (int c = 0; c < 8; ++c) st.qf[k][c] *= qscale;
        st.m[k] = -INFINITY;
        st.l[k] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) st.o[k][c] = 0.0f;
    }
}

// One online-softmax step over kLocalU rows of this lane group.
__device__ __forceinline__ void heads4_step(Heads4 &st, const uint4 (&kw)[kLocalU],
                                            const uint4 (&vw)[kLocalU],
                                            const bool (&ok)[kLocalU], bool b3, bool b2)
{
    float lg[kLocalU][4];
#pragma unroll
    for (int u = 0; u < kLocalU; ++u) {
        float kf[8];
        bf16x8_to_f32(kw[u], kf);
        float d[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float a = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) a = fmaf(st.qf[k][c], kf[c], a);
            d[k] = a;
        }
        float d2[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float keep = b3 ? d[2 + k] : d[k];
            const float send = b3 ? d[k] : d[2 + k];
            d2[k] = keep + dpp<kDppRowRor8>(send, send);
        }
        const float keep = b2 ? d2[1] : d2[0];
        const float send = b2 ? d2[0] : d2[1];
        float d1 = keep + dpp<kDppRowHalfMirror>(send, send);
        d1 += dpp<kDppQuadXor2>(d1, d1);
        d1 += dpp<kDppQuadXor1>(d1, d1);
        lg[u][0] = ok[u] ? dpp<kDppRowNewBcast0>(d1, d1) : -INFINITY;
        lg[u][1] = ok[u] ? dpp<kDppRowNewBcast0 + 4>(d1, d1) : -INFINITY;
        lg[u][2] = ok[u] ? dpp<kDppRowNewBcast0 + 8>(d1, d1) : -INFINITY;
        lg[u][3] = ok[u] ? dpp<kDppRowNewBcast0 + 12>(d1, d1) : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float mx = lg[0][k];
#pragma unroll
        for (int u = 1; u < kLocalU; ++u) mx = fmaxf(mx, lg[u][k]);
        const float mn = fmaxf(st.m[k], mx);
        if (mn == -INFINITY) continue;
        const float corr = rescale(st.m[k], mn);
        st.l[k] *= corr;
#pragma unroll
        for (int c = 0; c < 8; ++c) st.o[k][c] *= corr;
        st.m[k] = mn;
    }
#pragma unroll
    for (int u = 0; u < kLocalU; ++u) {
        float vf[8];
        bf16x8_to_f32(vw[u], vf);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float pw = ok[u] ? exp2f(lg[u][k] - st.m[k]) : 0.0f;
            st.l[k] += pw;
#pragma unroll
            for (int c = 0; c < 8; ++c) st.o[k][c] = fmaf(pw, vf[c], st.o[k][c]);
        }
    }
}

struct LocalArgs {
    int q_head_begin, n_q, n_sink, window;
    int ring;          // K/V hold n_sink + window slots: token i >= n_sink at
                       // slot n_sink + (i - n_sink) % window
    int S;             // splits of the row list
    int ny;            // head chunks (block rows)
    int chunks_per_g;
    int blocks;        // S * ny * B
    GroupWs W;
};

// Local block i: split s, head chunk y, batch row b.  The rows of split s of
// the row list (sinks, then the window) for the chunk's heads.
__device__ void local_block(const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
                            const uint16_t *__restrict__ V, int N, int64_t kv_cap, int Hq,
                            int Hkv, float qscale, const LocalArgs &A, float *__restrict__ out,
                            int i, LocalShared &sh)
{
    const int s = i % A.S, y = (i / A.S) % A.ny, b = i / (A.S * A.ny);
    const HeadChunk hc = head_chunk(y, Hq / Hkv, A.q_head_begin, A.n_q, A.chunks_per_g);
    if (hc.nh <= 0) return;

    const int64_t w_start = N > A.window ? (int64_t)N - A.window : 0;
    const int64_t sink_end = A.n_sink < w_start ? A.n_sink : w_start;
    const int64_t n_rows = sink_end + (N - w_start);
    int64_t chunk = (n_rows + A.S - 1) / A.S;
    chunk = (chunk + kLocTile - 1) / kLocTile * kLocTile;
    const int64_t begin = (int64_t)s * chunk;
    const int64_t end = min(n_rows, begin + chunk);

    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int grp = lane >> 4, sub = lane & 15;
    const int half = grp & 1, slot = w * 2 + (grp >> 1);
    const int64_t kvb = ((int64_t)b * Hkv + hc.g) * kv_cap * 128;
    const uint16_t *Kb = K + kvb;
    const uint16_t *Vb = V + kvb;
    // A tile of kLocTile rows is staged in LDS with every load in flight at
    // once (the rows of a split are contiguous apart from the sink/window
    // seam): thread t moves 16-B pieces t + 256 i of the tile's K and V.
    constexpr int kPieces = kLocTile * 16 / kAttThreads;
    uint4 kx[kPieces], vx[kPieces];
    auto load_tile = [&](int64_t t0, int nt) {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int e = threadIdx.x + i * kAttThreads, row = e >> 4, pc = e & 15;
            const int64_t j = t0 + (row < nt ? row : 0);
            int64_t g = j < sink_end ? j : w_start + (j - sink_end);
            if (A.ring && g >= A.n_sink) g = A.n_sink + (g - A.n_sink) % A.window;
            kx[i] = *reinterpret_cast<const uint4 *>(Kb + g * 128 + pc * 8);
            vx[i] = *reinterpret_cast<const uint4 *>(Vb + g * 128 + pc * 8);
        }
    };
    // q and the first tile are requested together; q is converted once the
    // tile is in LDS.
    uint4 qw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int hh = half * 4 + k;
        qw[k] = hh < hc.nh ? *reinterpret_cast<const uint4 *>(
                                 q + ((int64_t)b * Hq + hc.h_lo + hh) * 128 + sub * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int e = threadIdx.x + i * kAttThreads;
            sh.st.k[e >> 4][e & 15] = kx[i];
            sh.st.v[e >> 4][e & 15] = vx[i];
        }
    };
    Heads4 st;
    if (begin < end) {
        load_tile(begin, (int)min<int64_t>(kLocTile, end - begin));
        store_tile();
    }
    heads4_init(st, qw, qscale);
    const bool b3 = (sub >> 3) & 1, b2 = (sub >> 2) & 1;
    for (int64_t t0 = begin; t0 < end; t0 += kLocTile) {
        const int nt = (int)min<int64_t>(kLocTile, end - t0);
        if (t0 != begin) {
            load_tile(t0, nt);
            store_tile();
        }
        __syncthreads();
        // Lane group (slot, half) takes rows slot, slot + kLocSlots, ...
        // (kLocalU rows at a time: reading more from LDS ahead of use would
        // not fit the register budget).
#pragma unroll 1
        for (int u0 = 0; u0 < kLocTile / kLocSlots; u0 += kLocalU) {
            uint4 kw[kLocalU], vw[kLocalU];
            bool ok[kLocalU];
#pragma unroll
            for (int u = 0; u < kLocalU; ++u) {
                const int j = (u0 + u) * kLocSlots + slot;
                ok[u] = j < nt;
                kw[u] = sh.st.k[j][sub];
                vw[u] = sh.st.v[j][sub];
            }
            heads4_step(st, kw, vw, ok, b3, b2);
        }
        __syncthreads();  // the tile area is reused by the next tile and the merge
    }

    // The block's row slots, merged in LDS: one partial per head of the chunk.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int hh = half * 4 + k;
#pragma unroll
        for (int c = 0; c < 8; ++c) sh.mg.o[slot][hh][sub * 8 + c] = st.o[k][c];
        if (sub == 0) {
            sh.mg.m[slot][hh] = st.m[k];
            sh.mg.l[slot][hh] = st.l[k];
        }
    }
    __syncthreads();
    const int64_t r0 = (int64_t)b * A.n_q + (hc.h_lo - A.q_head_begin);
    {
        const int hh = threadIdx.x >> 5, d = (threadIdx.x & 31) * 4;
        if (hh < hc.nh) {
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k < kLocSlots; ++k) M = fmaxf(M, sh.mg.m[k][hh]);
            float L = 0.0f, O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < kLocSlots; ++k) {
                const float f = rescale(sh.mg.m[k][hh], M);
                L = fmaf(sh.mg.l[k][hh], f, L);
                const float4 ov = *reinterpret_cast<const float4 *>(&sh.mg.o[k][hh][d]);
                O[0] = fmaf(ov.x, f, O[0]);
                O[1] = fmaf(ov.y, f, O[1]);
                O[2] = fmaf(ov.z, f, O[2]);
                O[3] = fmaf(ov.w, f, O[3]);
            }
            float *pr = A.W.part + ((r0 + hh) * A.S + s) * kPart;
#pragma unroll
            for (int e = 0; e < 4; ++e) st_agent(pr + 4 + d + e, O[e]);
            if (d == 0) {
                st_agent(pr, M);
                st_agent(pr + 1, L);
            }
        }
    }
    merge_group_splits(hc.nh, s, A.S, r0, A.W, out + ((int64_t)b * Hq + hc.h_lo) * 128,
                       &sh.last,
                       [&sh](const float *first, int64_t hs, int n, int nh, float *dp,
                             int64_t ds, float *dout) {
                           merge_heads16(first, hs, n, nh, dp, ds, dout, sh.hm);
                       });
}

static dim3 group_grid(int S, int B, int Hq, int Hkv, int q_head_begin, int n_q_heads,
                       int *chunks_per_g)
{
    const int G = Hq / Hkv;
    const int g_first = q_head_begin / G;
    const int g_last = (q_head_begin + n_q_heads - 1) / G;
    *chunks_per_g = (G + 7) / 8;
    return dim3(S, (g_last - g_first + 1) * *chunks_per_g, B);
}

// ------------------------------------------------------ attention launch
//
// One kernel serves local heads, per-head sparse heads or both: blocks
// [0, L.blocks) are local blocks, the rest sparse splits.  Run together, the
// two sets share the launch, so neither waits on the other's tail.

struct SparseArgs {
    const int32_t *idx, *count;
    int q_head_begin, n_q, R;
    int blocks;  // 0: no sparse heads
    SparseWs W;
};

union AttendShared {
    SparseShared sp;
    LocalShared lo;
};

__global__ __launch_bounds__(kAttThreads, 4) void attend_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int N, int64_t kv_cap, int Hq, int Hkv, float qscale,
    LocalArgs L, SparseArgs P, float *__restrict__ out)
{
    __shared__ AttendShared sh;
    const int i = blockIdx.x;
    if (i < L.blocks)
        local_block(q, K, V, N, kv_cap, Hq, Hkv, qscale, L, out, i, sh.lo);
    else
        sparse_block(q, K, V, P.idx, P.count, N, kv_cap, Hq, Hkv, P.q_head_begin, P.n_q, P.R,
                     qscale, P.W, out, i - L.blocks, sh.sp);
}

static LocalArgs local_args(int B, int Hq, int Hkv, int N, int q_head_begin, int n_q_heads,
                            int n_sink, int window, void *ws)
{
    LocalArgs A{};
    if (n_q_heads <= 0) return A;
    A.q_head_begin = q_head_begin;
    A.n_q = n_q_heads;
    A.n_sink = n_sink;
    A.window = window;
    A.S = local_splits(local_rows_count(N, n_sink, window));
    const dim3 g = group_grid(A.S, B, Hq, Hkv, q_head_begin, n_q_heads, &A.chunks_per_g);
    A.ny = (int)g.y;
    A.blocks = A.S * A.ny * B;
    group_ws_layout((int64_t)B * n_q_heads, local_splits(N), kLocalSlice, &A.W, ws);
    return A;
}

static SparseArgs sparse_args(const int32_t *idx, const int32_t *count, int B, int q_head_begin,
                              int n_q_heads, void *ws)
{
    SparseArgs A{};
    if (n_q_heads <= 0) return A;
    A.idx = idx;
    A.count = count;
    A.q_head_begin = q_head_begin;
    A.n_q = n_q_heads;
    A.R = B * n_q_heads;
    A.blocks = sparse_grid(A.R);
    sparse_ws_layout(A.R, &A.W, ws);
    return A;
}

static hipError_t launch_attend(const uint16_t *q, const uint16_t *K, const uint16_t *V, int N,
                                int64_t kv_cap, int Hq, int Hkv, float scale, const LocalArgs &L,
                                const SparseArgs &P, float *out, hipStream_t stream)
{
    const int blocks = L.blocks + P.blocks;
    if (blocks == 0) return hipSuccess;
    SparseArgs Pw = P;
    RTP_TRY(wait_ctl(&Pw.W.wc));
    return launch(attend_kernel, dim3(blocks), dim3(kAttThreads), 0, stream, q, K, V, N, kv_cap,
                  Hq, Hkv, scale * kLog2e, L, Pw, out);
}

// Scratch of rtp_sparse_decode_noalloc, for callers that cannot allocate:
// the per-call workspace of the sparse attention (split partials, slice
// merges, hand-off flags) in a file-scope device array, one per device, held
// until the process ends.  Flags and counters in it need no clearing (each
// call leaves them as it found them).  Calls that overlap on one device
// share it and race.
constexpr size_t kNoAllocScratch = size_t(4) << 20;
static __device__ __align__(256) unsigned char rtp_noalloc_scratch[kNoAllocScratch];

size_t noalloc_scratch_bytes() { return kNoAllocScratch; }

// The current device's copy of the scratch array (looked up once per device:
// in host code the array's name is not a device address).
static hipError_t noalloc_scratch(void **p)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> cache[kMaxDevices];
    int dev = 0;
    RTP_TRY(hipGetDevice(&dev));
    void *a = dev >= 0 && dev < kMaxDevices ? cache[dev].load(std::memory_order_acquire) : nullptr;
    if (!a) {
        RTP_TRY(hipGetSymbolAddress(&a, HIP_SYMBOL(rtp_noalloc_scratch)));
        if (dev >= 0 && dev < kMaxDevices) cache[dev].store(a, std::memory_order_release);
    }
    *p = a;
    return hipSuccess;
}

hipError_t launch_sparse_decode_noalloc(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                        const int32_t *idx, const int32_t *count, int B, int Hq,
                                        int Hkv, int N, int64_t kv_cap, int q_head_begin,
                                        int n_q_heads, float scale, float *out,
                                        hipStream_t stream)
{
    void *ws = nullptr;
    RTP_TRY(noalloc_scratch(&ws));
    return launch_sparse_decode(q, K, V, idx, count, B, Hq, Hkv, N, kv_cap, q_head_begin,
                                n_q_heads, scale, out, ws, stream);
}

hipError_t launch_sparse_decode(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                const int32_t *idx, const int32_t *count, int B, int Hq,
                                int Hkv, int N, int64_t kv_cap, int q_head_begin,
                                int n_q_heads, float scale, float *out, void *ws,
                                hipStream_t stream)
{
    return launch_attend(q, K, V, N, kv_cap, Hq, Hkv, scale, LocalArgs{},
                         sparse_args(idx, count, B, q_head_begin, n_q_heads, ws), out, stream);
}

hipError_t launch_local_decode(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                               int B, int Hq, int Hkv, int N, int64_t kv_cap,
                               int q_head_begin, int n_q_heads, int n_sink, int window,
                               float scale, float *out, void *ws, hipStream_t stream)
{
    return launch_attend(q, K, V, N, kv_cap, Hq, Hkv, scale,
                         local_args(B, Hq, Hkv, N, q_head_begin, n_q_heads, n_sink, window, ws),
                         SparseArgs{}, out, stream);
}

hipError_t launch_local_decode_ring(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                    int B, int Hq, int Hkv, int N, int64_t kv_cap,
                                    int q_head_begin, int n_q_heads, int n_sink, int window,
                                    float scale, float *out, void *ws, hipStream_t stream)
{
    LocalArgs L = local_args(B, Hq, Hkv, N, q_head_begin, n_q_heads, n_sink, window, ws);
    L.ring = 1;
    return launch_attend(q, K, V, N, kv_cap, Hq, Hkv, scale, L, SparseArgs{}, out, stream);
}

size_t attend_ws_bytes(int64_t B, int64_t n_sparse, int64_t n_local, int N)
{
    size_t off = 0;
    if (n_sparse > 0) off += align_up(sparse_ws_bytes(B, n_sparse, N), 256);
    if (n_local > 0) off += local_ws_bytes(B, n_local, N);
    return off;
}

hipError_t launch_decode_attend(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                const int32_t *idx, const int32_t *count, int B, int Hq,
                                int Hkv, int N, int64_t kv_cap, int sparse_head_begin,
                                int n_sparse_heads, int local_head_begin, int n_local_heads,
                                int n_sink, int window, float scale, float *out, void *ws,
                                hipStream_t stream)
{
    char *base = static_cast<char *>(ws);
    const size_t sp = n_sparse_heads > 0 ? align_up(sparse_ws_bytes(B, n_sparse_heads, N), 256)
                                         : 0;
    return launch_attend(
        q, K, V, N, kv_cap, Hq, Hkv, scale,
        local_args(B, Hq, Hkv, N, local_head_begin, n_local_heads, n_sink, window, base + sp),
        sparse_args(idx, count, B, sparse_head_begin, n_sparse_heads, base), out, stream);
}

// ------------------------------------------------- scan + local heads
//
// The indexer scan of a layer's retrieval heads and the attention of its
// local heads in one launch (the head-role split of the gist.science summary,
// method section 1, and the scan of method section 2).  Neither reads what
// the other writes.  Blocks [0, L.blocks) are local blocks, dispatched first
// because their split merges form a chain of dependent steps; the rest are
// scan blocks, whose streaming read of k_r runs meanwhile.  The scan blocks
// are as many as fit beside the local blocks in one wave of the device
// (kFusedPerCU blocks per compute unit), and each takes every scan_blocks-th
// tile, so no scan tile waits for a second dispatch round.

constexpr int kFusedTPT = 1;    // tokens per thread of a scan tile in this launch
constexpr int kFusedPerCU = 4;  // resident blocks per compute unit (128 VGPRs, 256 threads)
static_assert(kScanThreads == kAttThreads, "scan tiles and local blocks share the block size");

struct ScanArgs {
    const float *q_r, *k_r;
    float *scores;
    int64_t kr_cap;
    int Hq_r, Hkv_r;
    ScanGeom g;
    int scan_blocks;  // blocks that run scan tiles
};

template <int G>
__global__ __launch_bounds__(kAttThreads, 4) void scan_local_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int N, int64_t kv_cap, int Hq, int Hkv, float qscale,
    LocalArgs L, ScanArgs C, float *__restrict__ out)
{
    __shared__ LocalShared sh;
    const int i = blockIdx.x;
    if (i < L.blocks) {
        local_block(q, K, V, N, kv_cap, Hq, Hkv, qscale, L, out, i, sh);
        return;
    }
    const int tiles = C.g.gx * C.g.gy;
    for (int j = i - L.blocks; j < tiles; j += C.scan_blocks)
        scan_tile<G, kFusedTPT>(C.q_r, C.k_r, C.scores, N, C.kr_cap, C.Hq_r, C.Hkv_r, C.g.group,
                                C.g.head_chunks, j % C.g.gx, j / C.g.gx);
}

hipError_t device_cus(int *cus)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];  // zero: not queried yet
    int dev = 0;
    RTP_TRY(hipGetDevice(&dev));
    const bool cached = dev >= 0 && dev < kMaxDevices;
    int c = cached ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (c < 1) {
        RTP_TRY(hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev));
        c = c < 1 ? 1 : c;
        if (cached) cache[dev].store(c, std::memory_order_relaxed);
    }
    *cus = c;
    return hipSuccess;
}

static int scan_chunk_heads(int Hq_r, int Hkv_r)
{
    const int group = Hq_r / Hkv_r;
    return group == 1 ? 1 : group == 2 ? 2 : group <= 4 ? 4 : 8;
}

int64_t scan_local_blocks(int B, int Hq_r, int Hkv_r, int Hq, int Hkv, int N,
                          int local_head_begin, int n_local_heads)
{
    const int G = scan_chunk_heads(Hq_r, Hkv_r);
    const int64_t group = Hq_r / Hkv_r;
    const int64_t tile = (int64_t)kScanThreads * kFusedTPT;
    const int64_t scan = ((int64_t)N + tile - 1) / tile * B * Hkv_r * ((group + G - 1) / G);
    const int64_t Gq = Hq / Hkv;
    const int64_t groups =
        ((int64_t)local_head_begin + n_local_heads - 1) / Gq - local_head_begin / Gq + 1;
    const int64_t local = (int64_t)B * groups * ((Gq + 7) / 8) * local_splits(N);
    return scan + local;
}

hipError_t launch_scan_local(const float *q_r, const float *k_r, float *scores, int Hq_r,
                             int Hkv_r, int64_t kr_cap, const uint16_t *q, const uint16_t *K,
                             const uint16_t *V, int B, int Hq, int Hkv, int N, int64_t kv_cap,
                             int local_head_begin, int n_local_heads, int n_sink, int window,
                             float scale, float *out, void *ws, hipStream_t stream)
{
    const LocalArgs L = local_args(B, Hq, Hkv, N, local_head_begin, n_local_heads, n_sink,
                                   window, ws);
    int cus = 0;
    RTP_TRY(device_cus(&cus));
    auto go = [&](auto kern, int G) {
        ScanArgs C{q_r, k_r, scores, kr_cap, Hq_r, Hkv_r,
                   scan_geom(B, Hq_r, Hkv_r, N, G, kFusedTPT), 0};
        const int tiles = C.g.gx * C.g.gy;
        const int room = kFusedPerCU * cus - L.blocks;  // slots left by the local blocks
        C.scan_blocks = room >= kFusedPerCU * cus / 2 ? min(tiles, room) : tiles;
        const unsigned blocks = (unsigned)(L.blocks + C.scan_blocks);
        return launch(kern, dim3(blocks), dim3(kAttThreads), 0, stream, q, K, V, N, kv_cap, Hq,
                      Hkv, scale * kLog2e, L, C, out);
    };
    switch (scan_chunk_heads(Hq_r, Hkv_r)) {
    case 1: return go(scan_local_kernel<1>, 1);
    case 2: return go(scan_local_kernel<2>, 2);
    case 4: return go(scan_local_kernel<4>, 4);
    default: return go(scan_local_kernel<8>, 8);
    }
}

// ------------------------------------------------------------- union
//
// Sparse heads in union mode: each split is a range of token words; a block
// ORs the keep bitmaps of its heads over the range, lists the union's tokens
// with their head masks in LDS, and gathers each listed row once for every
// head that kept it.

constexpr int kUnionWordsPerSplit = 16;  // at least (512 tokens)
constexpr int kMaxUnionSplits = 512;
constexpr int kUnionSlice = 32;
constexpr int kUnionRound = kWave;  // words listed per round (by wave 0)
constexpr int kUnionCap = kUnionRound * 32;

int union_splits(int N)
{
    const int64_t words = ((int64_t)N + 31) / 32;
    const int64_t s = (words + kUnionWordsPerSplit - 1) / kUnionWordsPerSplit;
    return (int)(s < 1 ? 1 : (s > kMaxUnionSplits ? kMaxUnionSplits : s));
}

size_t union_ws_bytes(int64_t B, int64_t n_q, int N)
{
    return group_ws_layout(B * n_q, union_splits(N), kUnionSlice, nullptr, nullptr);
}

// Block (s, y, b): the heads of head_chunk(y), token words of split s.
__global__ __launch_bounds__(kAttThreads) void union_attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint32_t *__restrict__ keep_bits, int N,
    int64_t kv_cap, int Hq, int Hkv, int q_head_begin, int n_q, float qscale, int S,
    int chunks_per_g, GroupWs W, float *__restrict__ out)
{
    __shared__ Heads8Shared sh;
    __shared__ uint32_t tok[kUnionCap];
    __shared__ uint8_t msk[kUnionCap];
    __shared__ uint32_t listed;
    const int s = blockIdx.x, b = blockIdx.z;
    const HeadChunk hc = head_chunk(blockIdx.y, Hq / Hkv, q_head_begin, n_q, chunks_per_g);
    if (hc.nh <= 0) return;

    const int64_t n_words = ((int64_t)N + 31) / 32;
    const int64_t per = (n_words + S - 1) / S;
    const int64_t w_begin = (int64_t)s * per;
    const int64_t w_end = min(n_words, w_begin + per);
    const int64_t r0 = (int64_t)b * n_q + (hc.h_lo - q_head_begin);
    const uint32_t *kb = keep_bits + r0 * n_words;

    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int grp = lane >> 4, sub = lane & 15;
    // Wave 0 lists the union's tokens of up to kUnionRound words per round,
    // with each token's head mask.  Bits past token N - 1 are ignored.
    uint32_t hw[8];
    auto load_words = [&](int64_t w0) {
        const int64_t wi = w0 + lane;
        const uint32_t valid = wi == n_words - 1 && (N & 31) ? (1u << (N & 31)) - 1u : ~0u;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh)
            hw[hh] = (hh < hc.nh && wi < w_end) ? kb[hh * n_words + wi] & valid : 0u;
    };
    // The first round's words are requested before q, so both loads overlap.
    if (w == 0) load_words(w_begin);
    Heads8 st;
    heads8_init(st, q, ((int64_t)b * Hq + hc.h_lo) * 128, hc.nh, qscale, sub);
    const int64_t kvb = ((int64_t)b * Hkv + hc.g) * kv_cap * 128 + sub * 8;
    const uint16_t *Kb = K + kvb;
    const uint16_t *Vb = V + kvb;
    constexpr int kRowsPerIter = kGroups * kLocalU;

    for (int64_t w0 = w_begin; w0 < w_end; w0 += kUnionRound) {
        if (w == 0) {
            if (w0 != w_begin) load_words(w0);
            const int64_t wi = w0 + lane;
            uint32_t un = 0;
#pragma unroll
            for (int hh = 0; hh < 8; ++hh) un |= hw[hh];
            const uint32_t cnt = (uint32_t)__popc(un);
            const uint32_t inc = wave_inclusive_scan(cnt);
            uint32_t pos = inc - cnt;
            for (uint32_t m = un; m; m &= m - 1) {
                const int bit = __ffs(m) - 1;
                uint32_t mk = 0;
#pragma unroll
                for (int hh = 0; hh < 8; ++hh) mk |= ((hw[hh] >> bit) & 1u) << hh;
                tok[pos] = (uint32_t)(wi * 32 + bit);
                msk[pos] = (uint8_t)mk;
                ++pos;
            }
            if (lane == kWave - 1) listed = inc;
        }
        __syncthreads();
        const uint32_t total = listed;
        for (uint32_t base = 0; base < total; base += kRowsPerIter) {
            uint4 kw[kLocalU], vw[kLocalU];
            uint32_t hb[kLocalU];
#pragma unroll
            for (int u = 0; u < kLocalU; ++u) {
                const uint32_t j = base + u * kGroups + w * 4 + grp;
                const bool ok = j < total;
                hb[u] = ok ? msk[j] : 0u;
                const int64_t off = ok ? (int64_t)tok[j] * 128 : 0;
                kw[u] = *reinterpret_cast<const uint4 *>(Kb + off);
                vw[u] = *reinterpret_cast<const uint4 *>(Vb + off);
            }
            heads8_step(st, kw, vw, hb);
        }
        __syncthreads();  // the list is rebuilt next round
    }
    heads8_finish(st, sh, hc.nh, s, S, r0, W, out + ((int64_t)b * Hq + hc.h_lo) * 128);
}

hipError_t launch_sparse_decode_union(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                      const uint32_t *keep_bits, int B, int Hq, int Hkv, int N,
                                      int64_t kv_cap, int q_head_begin, int n_q_heads,
                                      float scale, float *out, void *ws, hipStream_t stream)
{
    const int S = union_splits(N);
    int chunks_per_g;
    const dim3 grid = group_grid(S, B, Hq, Hkv, q_head_begin, n_q_heads, &chunks_per_g);
    GroupWs W;
    group_ws_layout((int64_t)B * n_q_heads, S, kUnionSlice, &W, ws);
    return launch(union_attn_kernel, grid, dim3(kAttThreads), 0, stream, q, K, V, keep_bits, N,
                  kv_cap, Hq, Hkv, q_head_begin, n_q_heads, scale * kLog2e, S, chunks_per_g, W,
                  out);
}

}  // namespace rtp
