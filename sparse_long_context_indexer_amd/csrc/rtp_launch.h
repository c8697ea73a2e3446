// Internal host-side launchers behind the C ABI in include/rtp.h.  Each is
// called only after the ABI layer has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rtp {

// ---- indexer scan (scan.hip)
hipError_t launch_index_scores(const float *q_r, const float *k_r, float *scores,
                               int B, int Hq_r, int Hkv_r, int N, int64_t kr_cap,
                               hipStream_t stream);

// ---- top-p selection (select.hip)
struct SelLayout {
    int64_t nblk;     // score chunks per row
    size_t rows;      // per-row state
    size_t mass1;     // level-1 histogram mass, fp64
    size_t cnt1;      // level-1 histogram count, u32
    size_t zero_end;  // [rows, zero_end) is cleared at the start of a call
    size_t pmax;      // per-chunk maxima
    size_t cand;      // boundary-bin candidates (key, index)
    size_t total;
};
SelLayout sel_layout(int64_t R, int64_t N);
hipError_t launch_topp_select(const float *scores, int64_t R, int N, float p,
                              int32_t *idx, int32_t *count, void *ws,
                              hipStream_t stream);

// ---- attention (attend.hip)
int sparse_splits(int N);
size_t sparse_ws_bytes(int64_t B, int64_t n_q, int N);
hipError_t launch_sparse_decode(const uint16_t *q, const uint16_t *K,
                                const uint16_t *V, const int32_t *idx,
                                const int32_t *count, int B, int Hq, int Hkv,
                                int N, int64_t kv_cap, int q_head_begin,
                                int n_q_heads, float scale, float *out,
                                void *ws, hipStream_t stream);

int local_splits(int64_t n_rows);
size_t local_ws_bytes(int64_t B, int64_t n_q, int N);
hipError_t launch_local_decode(const uint16_t *q, const uint16_t *K,
                               const uint16_t *V, int B, int Hq, int Hkv, int N,
                               int64_t kv_cap, int q_head_begin, int n_q_heads,
                               int n_sink, int window, float scale, float *out,
                               void *ws, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace rtp
