// Internal host-side launchers behind the C ABI in include/rtp.h.  Each is
// called only after the ABI layer has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rtp {

// Poll limit and status word for kernels whose blocks wait on each other
// (rtp_device.h); filled from the host-set limit and the current device's
// status word.
struct WaitCtl;
hipError_t wait_ctl(WaitCtl *wc);

// ---- indexer scan (scan.hip)
hipError_t launch_index_scores(const float *q_r, const float *k_r, float *scores,
                               int B, int Hq_r, int Hkv_r, int N, int64_t kr_cap,
                               hipStream_t stream);

// ---- top-p selection (select.hip)
struct SelLayout {
    int64_t nblk;     // score chunks per row
    size_t rows;      // per-row state
    size_t hist1;     // per-row level-1 histogram
    size_t hist2;     // per-row histogram of the boundary bin's candidates
    size_t tops;      // per-chunk top-bin records
    size_t cand;      // boundary-bin candidates (key, index)
    size_t total;
};
SelLayout sel_layout(int64_t R, int64_t N);
hipError_t launch_topp_select(const float *scores, int64_t R, int N, float p,
                              int32_t *idx, int32_t *count, uint32_t *keep_bits,
                              void *ws, hipStream_t stream);
hipError_t launch_topk_select(const float *scores, int64_t R, int N, int k, int32_t *idx,
                              int32_t *count, uint32_t *keep_bits, void *ws, hipStream_t stream);
hipError_t launch_index_scores_bf16(const float *q_r, const uint16_t *k_r, float *scores,
                                    int B, int Hq_r, int Hkv_r, int N, int64_t kr_cap,
                                    hipStream_t stream);
hipError_t launch_local_decode_ring(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                    int B, int Hq, int Hkv, int N, int64_t kv_cap,
                                    int q_head_begin, int n_q_heads, int n_sink, int window,
                                    float scale, float *out, void *ws, hipStream_t stream);
hipError_t launch_keep_local(uint32_t *keep_bits, int64_t R, int N, int n_sink, int window,
                             hipStream_t stream);
hipError_t launch_prefill_attend(const uint16_t *q, const uint16_t *K, const uint16_t *V, int B,
                                 int Hq, int Hkv, int T, int64_t kv_cap, int head_begin,
                                 int n_heads, int n_sink, int window, float scale, float *out,
                                 hipStream_t stream);
hipError_t launch_index_project(const uint16_t *x, int B, int Hx, int64_t x_cap, int head_begin,
                                int H, int T, const uint16_t *W, float *out, int64_t out_cap,
                                int64_t out_pos, hipStream_t stream);
hipError_t launch_topp_hist(const float *scores, int64_t R, int N, void *ws,
                            hipStream_t stream);

// ---- attention (attend.hip)
size_t sparse_ws_bytes(int64_t B, int64_t n_q, int N);
int sparse_grid(int64_t R);
hipError_t launch_sparse_decode(const uint16_t *q, const uint16_t *K,
                                const uint16_t *V, const int32_t *idx,
                                const int32_t *count, int B, int Hq, int Hkv,
                                int N, int64_t kv_cap, int q_head_begin,
                                int n_q_heads, float scale, float *out,
                                void *ws, hipStream_t stream);

// rtp_sparse_decode with its workspace in a static device array.
size_t noalloc_scratch_bytes();
hipError_t launch_sparse_decode_noalloc(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                        const int32_t *idx, const int32_t *count, int B, int Hq,
                                        int Hkv, int N, int64_t kv_cap, int q_head_begin,
                                        int n_q_heads, float scale, float *out,
                                        hipStream_t stream);

size_t union_ws_bytes(int64_t B, int64_t n_q, int N);
hipError_t launch_sparse_decode_union(const uint16_t *q, const uint16_t *K,
                                      const uint16_t *V, const uint32_t *keep_bits,
                                      int B, int Hq, int Hkv, int N, int64_t kv_cap,
                                      int q_head_begin, int n_q_heads, float scale,
                                      float *out, void *ws, hipStream_t stream);

// Local and per-head sparse heads in one launch; the workspace holds the
// sparse workspace, then (256-B aligned) the local one.
size_t attend_ws_bytes(int64_t B, int64_t n_sparse, int64_t n_local, int N);
hipError_t launch_decode_attend(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                const int32_t *idx, const int32_t *count, int B, int Hq,
                                int Hkv, int N, int64_t kv_cap, int sparse_head_begin,
                                int n_sparse_heads, int local_head_begin, int n_local_heads,
                                int n_sink, int window, float scale, float *out, void *ws,
                                hipStream_t stream);

int local_splits(int64_t n_rows);
size_t local_ws_bytes(int64_t B, int64_t n_q, int N);
hipError_t launch_local_decode(const uint16_t *q, const uint16_t *K,
                               const uint16_t *V, int B, int Hq, int Hkv, int N,
                               int64_t kv_cap, int q_head_begin, int n_q_heads,
                               int n_sink, int window, float scale, float *out,
                               void *ws, hipStream_t stream);

// Indexer scan and local heads in one launch (the local workspace as for
// launch_local_decode).  scan_local_blocks bounds the launch's block count
// for any n_sink / window.
int64_t scan_local_blocks(int B, int Hq_r, int Hkv_r, int Hq, int Hkv, int N,
                          int local_head_begin, int n_local_heads);
hipError_t launch_scan_local(const float *q_r, const float *k_r, float *scores, int Hq_r,
                             int Hkv_r, int64_t kr_cap, const uint16_t *q, const uint16_t *K,
                             const uint16_t *V, int B, int Hq, int Hkv, int N, int64_t kv_cap,
                             int local_head_begin, int n_local_heads, int n_sink, int window,
                             float scale, float *out, void *ws, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- one-launch decode layer (layer.hip)
struct LayerGeom {
    bool ok;       // false: the shape is outside what one launch holds
    int G;         // query heads per KV head
    int Hkv_r;     // retrieval KV heads
    int RG;        // B * Hkv_r score rows of G heads
    int bpr;       // blocks per row
    int C;         // tokens per block
    int NB;        // blocks (at most one per compute unit)
    int ngrp;      // groups of up to 16 blocks per row
    int n_lkv;     // local KV heads
    int nlt;       // local tiles per (batch row, local KV head)
    int NI;        // local items
    int NX;        // extra blocks that run only local items (compute units the rows leave free)
    int nl_rows;   // sink + window rows
    int sink_end;  // sinks are rows [0, sink_end)
    int w0;        // the window is rows [w0, N)
};
LayerGeom layer_geom(int cus, int B, int Hq, int Hkv, int N, int Hq_r, int n_sink, int window);
size_t layer_ws_bytes(const LayerGeom &L, int B, int N);
hipError_t launch_decode_layer(const LayerGeom &L, const float *q_r, const float *k_r,
                               int64_t kr_cap, const uint16_t *q, const uint16_t *K,
                               const uint16_t *V, int64_t kv_cap, int B, int Hq, int Hkv, int N,
                               int Hq_r, float p, float scale, float *out, int32_t *idx,
                               int32_t *count, float *scores, void *ws, uint32_t spin_limit,
                               uint32_t *status, hipStream_t stream);

// ---- top-p selection and attention over the kept rows in one launch (select.hip)
// Score row b * H_r + h is query head h of batch row b (the retrieval heads
// are query heads [0, H_r)); heads [H_r, Hq) are local heads.
size_t topp_attend_ws_bytes(int cus, int B, int Hq, int Hkv, int N, int H_r, int n_sink,
                            int window);
bool topp_attend_fits(int cus, int B, int Hq, int Hkv, int N, int H_r, int n_sink, int window);
hipError_t launch_topp_attend(const float *scores, const uint16_t *q, const uint16_t *K,
                              const uint16_t *V, int B, int Hq, int Hkv, int N, int64_t kv_cap,
                              int H_r, int n_sink, int window, float p, float scale, float *out,
                              int32_t *idx, int32_t *count, void *ws, hipStream_t stream);


// Compute units of the current device (queried once per device).
hipError_t device_cus(int *cus);


template <typename... KArgs>
hipError_t launch_impl(const void *k, dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                       KArgs... args)
{
    void *ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(k, grid, block, ptrs, shmem, stream);
}

// Launches kernel k and returns the status of this launch alone
// (hipGetLastError would also report errors left by unrelated HIP calls).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*k)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    return launch_impl<KArgs...>(reinterpret_cast<const void *>(k), grid, block, shmem, stream,
                                 static_cast<KArgs>(args)...);
}

#define RTP_TRY(expr)                          \
    do {                                       \
        hipError_t rtp_e_ = (expr);            \
        if (rtp_e_ != hipSuccess) return rtp_e_; \
    } while (0)

}  // namespace rtp
