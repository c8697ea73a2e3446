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
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
    base = __shfl(base, leader);
    if (!pred) return -1;
    const uint64_t below = (lane == 0) ? 0ull : (mask & (~0ull >> (64 - lane)));
    return (int64_t)base + __popcll(below);
}

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        T o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Exclusive prefix sum over a block of NT threads in thread order; every
// thread must call it.  `scratch` holds NT/64 + 1 elements of LDS.  Returns
// the exclusive prefix; *total receives the block-wide sum.
template <int NT, typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T *scratch, T *total)
{
    constexpr int NW = NT / kWave;
    const int lane = lane_id();
    const int w = (int)threadIdx.x / kWave;
    T inc = wave_inclusive_scan(v);
    T prev = __shfl_up(inc, 1);
    if (lane == kWave - 1) scratch[w] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        T run = T(0);
        for (int i = 0; i < NW; ++i) {
            T t = scratch[i];
            scratch[i] = run;
            run += t;
        }
        scratch[NW] = run;
    }
    __syncthreads();
    T ex = scratch[w] + (lane == 0 ? T(0) : prev);
    *total = scratch[NW];
    __syncthreads();
    return ex;
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
// Waits until every vector memory operation this wave issued has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
