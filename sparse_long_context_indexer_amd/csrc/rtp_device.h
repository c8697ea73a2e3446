// Device helpers shared by the gfx950 kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtp {

constexpr int kWave = 64;

// Order-preserving map from an fp32 score to uint32: a larger key means a
// larger score, and equal scores (with -0 folded into +0) give equal keys.
__device__ __forceinline__ uint32_t score_key(float s)
{
    const uint32_t u = __float_as_uint(s + 0.0f);  // -0 + 0 is +0; nothing else changes
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// bf16 pairs packed in one 32-bit word: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void bf16x8_to_f32(const uint4 &w, float f[8])
{
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// ---- cross-lane moves (DPP, gfx9 encoding; no LDS round trip)
//
// dpp<Ctrl, RowMask>(old, v): lane i receives v from the lane Ctrl names;
// lanes in rows outside RowMask, or whose source lies outside their row,
// receive `old`.  Works on any 4- or 8-byte type.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111;     // row_shr:n = 0x110 + n
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138;    // lane i <- lane i-1 across the wave
constexpr int kDppRowMirror = 0x140;   // i <- 15-i within 16 lanes
constexpr int kDppRowHalfMirror = 0x141;  // i <- 7-i within 8 lanes
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3
constexpr int kDppRowRor8 = 0x128;     // i <- (i+8) mod 16 within 16 lanes (= i ^ 8)
constexpr int kDppRowNewBcast0 = 0x150;  // + n: lane n of each row -> the whole row

template <int Ctrl, int RowMask = 0xf, typename T>
__device__ __forceinline__ T dpp(T old, T v)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte lanes");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(
            T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                           Ctrl, RowMask, 0xf, false));
    } else {
        const unsigned long long o = __builtin_bit_cast(unsigned long long, old);
        const unsigned long long x = __builtin_bit_cast(unsigned long long, v);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)x,
                                                                  Ctrl, RowMask, 0xf, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(
            (int)(uint32_t)(o >> 32), (int)(uint32_t)(x >> 32), Ctrl, RowMask, 0xf, false);
        return __builtin_bit_cast(T, (unsigned long long)lo | ((unsigned long long)hi << 32));
    }
}

// Value of v in lane `lane` (wave-uniform), for every lane.
template <typename T>
__device__ __forceinline__ T read_lane(T v, int lane)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte lanes");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
    } else {
        const unsigned long long x = __builtin_bit_cast(unsigned long long, v);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
        return __builtin_bit_cast(T, (unsigned long long)lo | ((unsigned long long)hi << 32));
    }
}

// Slot reservation for a wave: every lane of the wave must call this with
// the same counter.  Lanes with pred=true get distinct slots (one atomic per
// wave); the others get -1.
__device__ __forceinline__ int64_t wave_append(bool pred, uint32_t *counter)
{
    const uint64_t mask = __ballot(pred);
    if (mask == 0) return -1;
    const int leader = __ffsll((unsigned long long)mask) - 1;
    const int lane = lane_id();
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = read_lane(base, leader);
    if (!pred) return -1;
    const uint64_t below = (lane == 0) ? 0ull : (mask & (~0ull >> (64 - lane)));
    return (int64_t)base + __popcll(below);
}

// Inclusive prefix sum over the wave in lane order: a scan within each row
// of 16 lanes, then the row totals carried into the rows above.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v)
{
    v += dpp<kDppRowShr1>(T(0), v);
    v += dpp<kDppRowShr2>(T(0), v);
    v += dpp<kDppRowShr4>(T(0), v);
    v += dpp<kDppRowShr8>(T(0), v);
    v += dpp<kDppRowBcast15, 0xa>(T(0), v);
    v += dpp<kDppRowBcast31, 0xc>(T(0), v);
    return v;
}

// The exclusive prefix from the inclusive one: each lane takes the lane
// below's (lane 0 takes 0).
template <typename T>
__device__ __forceinline__ T wave_shift_up(T inc)
{
    return dpp<kDppWaveShr1>(T(0), inc);
}

// Sum over the wave, in every lane: each row of 16 lanes is reduced in
// place, then the four row totals are added in row order.
template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
    v += dpp<kDppQuadXor1>(v, v);
    v += dpp<kDppQuadXor2>(v, v);
    v += dpp<kDppRowHalfMirror>(v, v);
    v += dpp<kDppRowMirror>(v, v);
    return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp<kDppQuadXor1>(v, v));
    v = fmaxf(v, dpp<kDppQuadXor2>(v, v));
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v, v));
    v = fmaxf(v, dpp<kDppRowMirror>(v, v));
    return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}

// Exclusive prefix sum over a block of NT threads in thread order; every
// thread must call it.  `scratch` holds NT/64 elements of LDS.  Returns
// the exclusive prefix; *total receives the block-wide sum.  Every thread
// adds the wave totals in the same order, so all agree on *total.  With
// kReuse false the caller promises not to write `scratch` again, and the
// closing barrier is skipped.
template <int NT, typename T, bool kReuse = true>
__device__ __forceinline__ T block_exclusive_scan(T v, T *scratch, T *total)
{
    constexpr int NW = NT / kWave;
    const int w = (int)threadIdx.x / kWave;
    const T inc = wave_inclusive_scan(v);
    const T prev = wave_shift_up(inc);
    if (lane_id() == kWave - 1) scratch[w] = inc;
    __syncthreads();
    T before = T(0), run = T(0);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const T t = scratch[i];
        if (i == w) before = run;
        run += t;
    }
    *total = run;
    if (kReuse) __syncthreads();
    return before + prev;
}

// Cross-block hand-off inside one kernel.  Data another block of the same
// kernel will read is written with agent-scope stores (global_store sc1:
// written through the per-XCD L2) and read with agent-scope loads (sc1);
// before a block counts itself done, each wave waits for its stores to
// complete.  No L2 write-back or invalidate is needed.
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(double *p, double v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent(const double *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-B load with the nontemporal hint: for data read once and not again
// soon (gathered K/V rows), so it does not displace what is.
__device__ __forceinline__ uint4 ld_nt16(const void *p)
{
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// Waits until every vector memory operation this wave issued has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Polls before a wait on other blocks gives up, unless the host sets
// another limit (rtp_set_wait_limit).  A wait ends long before this; the
// bound only keeps a fault elsewhere from hanging the device.
constexpr uint32_t kSpinMax = 1u << 24;

// Bits of the library's sticky status word (rtp_device_status).
constexpr uint32_t kStatusWaitTimeout = 1u;  // a bounded wait gave up

// What a waiting kernel needs: the poll limit and where to report a give-up.
struct WaitCtl {
    uint32_t limit;
    uint32_t *status;
};

__device__ __forceinline__ void report_timeout(const WaitCtl &wc)
{
    if (wc.status) atomicOr(wc.status, kStatusWaitTimeout);
}

// Hand-off flags: a block publishes a result it stored with agent-scope
// stores by setting a flag word to kFlagTag once every thread's stores have
// completed; the consumer waits for the tag and clears the word again, so a
// finished call leaves every flag it used at 0.  kFlagTag is a NaN payload,
// like kCtrTag.
constexpr uint32_t kFlagTag = 0x7FC3A96Bu;

__device__ __forceinline__ void publish_flag(uint32_t *flag)
{
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, kFlagTag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Threads 0 .. n-1 each wait for one of the flags f[0 .. n) and clear it;
// the block then continues together.  n must not exceed the block size.
// A flag still unset after wc.limit polls is given up on and the give-up
// reported in the status word.
__device__ __forceinline__ void await_flags(uint32_t *f, int n, const WaitCtl &wc)
{
    if ((int)threadIdx.x < n) {
        for (uint32_t it = 0;; ++it) {
            if (__hip_atomic_load(f + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                kFlagTag)
                break;
            if (it >= wc.limit) {
                report_timeout(wc);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __hip_atomic_store(f + threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
}

// Counters shared by the blocks of one call (arrivals, output slots).  A
// counter word holds a tag (low 32 bits) and a count (high 32 bits); after
// every call it is left as (kCtrTag, 0), so a block normally counts with one
// atomicAdd.  A word without the tag (fresh or reused memory) is claimed with
// a compare-and-swap: the add that landed on it is void, and the first block
// to swap in (kCtrTag, its n) starts the count.  Adds to the high half never
// change the tag.  kCtrTag is a NaN payload that arithmetic never produces,
// so no float or index the library writes can look like a counter.
constexpr uint32_t kCtrTag = 0x7FA5C3E1u;

// Adds n (every participant adds, even 0, so the word is always claimed) and
// returns the count before the add.
__device__ __forceinline__ uint32_t ctr_add(unsigned long long *ctr, uint32_t n)
{
    const unsigned long long add = (unsigned long long)n << 32;
    const unsigned long long old = atomicAdd(ctr, add);
    if ((uint32_t)old == kCtrTag) return (uint32_t)(old >> 32);
    unsigned long long cur = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        if ((uint32_t)cur == kCtrTag) return (uint32_t)(atomicAdd(ctr, add) >> 32);
        const unsigned long long prev = atomicCAS(ctr, cur, add | kCtrTag);
        if (prev == cur) return 0u;
        cur = prev;
    }
}

// Arrival: returns how many blocks of this call arrived before the caller.
__device__ __forceinline__ uint32_t ctr_arrive(unsigned long long *ctr) { return ctr_add(ctr, 1u); }

// Called by the last block of a call, when no other block of the call will
// touch the counter again.
__device__ __forceinline__ void ctr_reset(unsigned long long *ctr) { atomicExch(ctr, (unsigned long long)kCtrTag); }

}  // namespace rtp
