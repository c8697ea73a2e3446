// C ABI (include/rtp.h): host-side validation, workspace sizing, dispatch.
// Every argument is checked before anything is enqueued; no C++ exception
// crosses the boundary.
#include <math.h>
#include <stdint.h>


#include <atomic>

#include "rtp.h"
#include "rtp_device.h"
#include "rtp_launch.h"

// The library's sticky status word, one per device (each device holds its
// own copy of a __device__ variable; its address is looked up per device).
static __device__ uint32_t rtp_status_word;

namespace {

std::atomic<uint32_t> g_wait_limit{rtp::kSpinMax};

// The current device's status word (looked up once per device).
hipError_t status_word(uint32_t **p)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<uint32_t *> cache[kMaxDevices];
    int dev = 0;
    RTP_TRY(hipGetDevice(&dev));
    uint32_t *w = dev >= 0 && dev < kMaxDevices ? cache[dev].load(std::memory_order_acquire)
                                                : nullptr;
    if (!w) {
        void *a = nullptr;
        RTP_TRY(hipGetSymbolAddress(&a, HIP_SYMBOL(rtp_status_word)));
        w = static_cast<uint32_t *>(a);
        if (dev >= 0 && dev < kMaxDevices) cache[dev].store(w, std::memory_order_release);
    }
    *p = w;
    return hipSuccess;
}

constexpr int kMaxGridY = 65535;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

thread_local int32_t last_hip_error = 0;

rtp_status from_hip(hipError_t e)
{
    if (e == hipSuccess) return RTP_OK;
    last_hip_error = (int32_t)e;
    return RTP_ERR_HIP;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

rtp_status check_attention_common(const void *q, const void *K, const void *V, const void *out,
                                  const void *ws, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t N, int64_t kv_cap, int32_t d,
                                  int32_t q_head_begin, int32_t n_q_heads, float scale)
{
    if (!q || !K || !V || !out || !ws) return RTP_ERR_NULL;
    if (d != 128) return RTP_ERR_UNSUPPORTED;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || N < 1 || kv_cap < N) return RTP_ERR_SHAPE;
    if (q_head_begin < 0 || n_q_heads < 1 || (int64_t)q_head_begin + n_q_heads > Hq)
        return RTP_ERR_SHAPE;
    if (B > kMaxGridY || n_q_heads > kMaxGridY) return RTP_ERR_SHAPE;
    if (!isfinite(scale)) return RTP_ERR_VALUE;
    if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 4) ||
        !aligned(ws, 256))
        return RTP_ERR_ALIGN;
    return RTP_OK;
}

}  // namespace

namespace rtp {

hipError_t wait_ctl(WaitCtl *wc)
{
    wc->limit = g_wait_limit.load(std::memory_order_relaxed);
    return status_word(&wc->status);
}

}  // namespace rtp

extern "C" {

const char *rtp_status_string(rtp_status s)
{
    switch (s) {
    case RTP_OK: return "ok";
    case RTP_ERR_NULL: return "a required pointer is NULL";
    case RTP_ERR_SHAPE: return "a size is out of range or inconsistent";
    case RTP_ERR_UNSUPPORTED: return "unsupported dimension (r must be 16, d must be 128)";
    case RTP_ERR_VALUE: return "a parameter value is out of range";
    case RTP_ERR_ALIGN: return "a pointer breaks the required alignment";
    case RTP_ERR_WORKSPACE: return "workspace missing or too small";
    case RTP_ERR_HIP: return "the HIP runtime reported an error";
    case RTP_ERR_LIMIT: return "the sizes exceed the no-allocation entry point's scratch";
    }
    return "unknown status";
}

int32_t rtp_last_hip_error(void) { return last_hip_error; }

rtp_status rtp_set_wait_limit(uint32_t polls)
{
    g_wait_limit.store(polls, std::memory_order_relaxed);
    return RTP_OK;
}

rtp_status rtp_device_status(uint32_t *flags, int32_t clear)
{
    if (!flags) return RTP_ERR_NULL;
    uint32_t *w = nullptr;
    hipError_t e = status_word(&w);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(flags, w, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) {
        const uint32_t zero = 0;
        e = hipMemcpy(w, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
    }
    return from_hip(e);
}

rtp_status rtp_workspace_size(int32_t which, int32_t B, int32_t H, int32_t N, size_t *bytes)
{
    if (!bytes) return RTP_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return RTP_ERR_SHAPE;
    switch (which) {
    case RTP_WS_TOPP_SELECT: *bytes = rtp::sel_layout((int64_t)B * H, N).total; return RTP_OK;
    case RTP_WS_SPARSE_DECODE: *bytes = rtp::sparse_ws_bytes(B, H, N); return RTP_OK;
    case RTP_WS_LOCAL_DECODE: *bytes = rtp::local_ws_bytes(B, H, N); return RTP_OK;
    case RTP_WS_SPARSE_UNION: *bytes = rtp::union_ws_bytes(B, H, N); return RTP_OK;
    case RTP_WS_DECODE_ATTEND: *bytes = rtp::attend_ws_bytes(B, H, H, N); return RTP_OK;
    default: return RTP_ERR_VALUE;
    }
}

rtp_status rtp_index_scores(const float *q_r, const float *k_r, float *scores, int32_t B,
                            int32_t Hq_r, int32_t Hkv_r, int32_t N, int64_t kr_cap, int32_t r,
                            void *stream)
{
    if (!q_r || !k_r || !scores) return RTP_ERR_NULL;
    if (r != 16) return RTP_ERR_UNSUPPORTED;
    if (B < 1 || Hq_r < 1 || Hkv_r < 1 || Hq_r % Hkv_r != 0 || N < 1 || kr_cap < N)
        return RTP_ERR_SHAPE;
    const int64_t group = Hq_r / Hkv_r;
    if ((int64_t)B * Hkv_r * ((group + 7) / 8) > kMaxGridY) return RTP_ERR_SHAPE;
    if (!aligned(q_r, 16) || !aligned(k_r, 16) || !aligned(scores, 4)) return RTP_ERR_ALIGN;
    return from_hip(rtp::launch_index_scores(q_r, k_r, scores, B, Hq_r, Hkv_r, N, kr_cap,
                                             as_stream(stream)));
}

rtp_status rtp_index_scores_bf16(const float *q_r, const rtp_bf16 *k_r, float *scores,
                                 int32_t B, int32_t Hq_r, int32_t Hkv_r, int32_t N,
                                 int64_t kr_cap, int32_t r, void *stream)
{
    if (!q_r || !k_r || !scores) return RTP_ERR_NULL;
    if (r != 16) return RTP_ERR_UNSUPPORTED;
    if (B < 1 || Hq_r < 1 || Hkv_r < 1 || Hq_r % Hkv_r != 0 || N < 1 || kr_cap < N)
        return RTP_ERR_SHAPE;
    const int64_t group = Hq_r / Hkv_r;
    if ((int64_t)B * Hkv_r * ((group + 7) / 8) > kMaxGridY) return RTP_ERR_SHAPE;
    if (!aligned(q_r, 16) || !aligned(k_r, 16) || !aligned(scores, 4)) return RTP_ERR_ALIGN;
    return from_hip(rtp::launch_index_scores_bf16(q_r, k_r, scores, B, Hq_r, Hkv_r, N, kr_cap,
                                                  as_stream(stream)));
}

rtp_status rtp_topp_select(const float *scores, int32_t B, int32_t H, int32_t N, float p,
                           int32_t *idx, int32_t *count, uint32_t *keep_bits, void *workspace,
                           size_t ws_bytes, void *stream)
{
    if (!scores || !idx || !count || !workspace) return RTP_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || (int64_t)B * H > kMaxGridY) return RTP_ERR_SHAPE;
    if (!(p > 0.0f && p <= 1.0f)) return RTP_ERR_VALUE;  // NaN fails too
    if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(count, 4) ||
        !aligned(keep_bits, 4) || !aligned(workspace, 256))
        return RTP_ERR_ALIGN;
    const int64_t R = (int64_t)B * H;
    if (ws_bytes < rtp::sel_layout(R, N).total) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_topp_select(scores, R, N, p, idx, count, keep_bits, workspace,
                                            as_stream(stream)));
}

rtp_status rtp_index_project(const rtp_bf16 *x, int32_t B, int32_t Hx, int64_t x_cap,
                             int32_t head_begin, int32_t H, int32_t T, int32_t d,
                             const rtp_bf16 *W, int32_t r, float *out, int64_t out_cap,
                             int64_t out_pos, void *stream)
{
    if (!x || !W || !out) return RTP_ERR_NULL;
    if (d != 128 || r != 16) return RTP_ERR_UNSUPPORTED;
    // Token indices (plus a block's worth of tiles) stay within int32.
    if (B < 1 || Hx < 1 || H < 1 || T < 1 || T > INT32_MAX - 1024 || head_begin < 0 ||
        head_begin > Hx - H ||
        x_cap < T || out_pos < 0 || out_cap < T || out_pos > out_cap - T ||
        (int64_t)B * H > kMaxGridY)
        return RTP_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(out, 4)) return RTP_ERR_ALIGN;
    return from_hip(rtp::launch_index_project(x, B, Hx, x_cap, head_begin, H, T, W, out, out_cap,
                                              out_pos, as_stream(stream)));
}

rtp_status rtp_topk_select(const float *scores, int32_t B, int32_t H, int32_t N, int32_t k,
                           int32_t *idx, int32_t *count, uint32_t *keep_bits, void *workspace,
                           size_t ws_bytes, void *stream)
{
    if (!scores || !idx || !count || !workspace) return RTP_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || (int64_t)B * H > kMaxGridY) return RTP_ERR_SHAPE;
    if (k < 1) return RTP_ERR_VALUE;
    if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(count, 4) ||
        !aligned(keep_bits, 4) || !aligned(workspace, 256))
        return RTP_ERR_ALIGN;
    const int64_t R = (int64_t)B * H;
    if (ws_bytes < rtp::sel_layout(R, N).total) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_topk_select(scores, R, N, k, idx, count, keep_bits, workspace,
                                            as_stream(stream)));
}

rtp_status rtp_keep_bits_add_local(uint32_t *keep_bits, int32_t B, int32_t H, int32_t N,
                                   int32_t n_sink, int32_t window, void *stream)
{
    if (!keep_bits) return RTP_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || (int64_t)B * H > kMaxGridY) return RTP_ERR_SHAPE;
    if (n_sink < 0 || window < 1) return RTP_ERR_VALUE;
    if (!aligned(keep_bits, 4)) return RTP_ERR_ALIGN;
    return from_hip(rtp::launch_keep_local(keep_bits, (int64_t)B * H, N, n_sink, window,
                                           as_stream(stream)));
}

rtp_status rtp_topp_hist(const float *scores, int32_t B, int32_t H, int32_t N, void *workspace,
                         size_t ws_bytes, void *stream)
{
    if (!scores || !workspace) return RTP_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || (int64_t)B * H > kMaxGridY) return RTP_ERR_SHAPE;
    if (!aligned(scores, 4) || !aligned(workspace, 256)) return RTP_ERR_ALIGN;
    const int64_t R = (int64_t)B * H;
    if (ws_bytes < rtp::sel_layout(R, N).total) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_topp_hist(scores, R, N, workspace, as_stream(stream)));
}

rtp_status rtp_sparse_decode(const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V,
                             const int32_t *idx, const int32_t *count, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                             int32_t q_head_begin, int32_t n_q_heads, float scale, float *out,
                             void *workspace, size_t ws_bytes, void *stream)
{
    if (!idx || !count) return RTP_ERR_NULL;
    rtp_status st = check_attention_common(q, K, V, out, workspace, B, Hq, Hkv, N, kv_cap, d,
                                           q_head_begin, n_q_heads, scale);
    if (st != RTP_OK) return st;
    if (!aligned(idx, 4) || !aligned(count, 4)) return RTP_ERR_ALIGN;
    if (ws_bytes < rtp::sparse_ws_bytes(B, n_q_heads, N)) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_sparse_decode(q, K, V, idx, count, B, Hq, Hkv, N, kv_cap,
                                              q_head_begin, n_q_heads, scale, out, workspace,
                                              as_stream(stream)));
}

rtp_status rtp_sparse_decode_noalloc(const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V,
                                     const int32_t *idx, const int32_t *count, int32_t B,
                                     int32_t Hq, int32_t Hkv, int32_t N, int64_t kv_cap,
                                     int32_t d, int32_t q_head_begin, int32_t n_q_heads,
                                     float scale, float *out, void *stream)
{
    if (!idx || !count) return RTP_ERR_NULL;
    // check_attention_common wants a workspace pointer: the scratch stands in.
    static const char kScratch alignas(256) = 0;
    rtp_status st = check_attention_common(q, K, V, out, &kScratch, B, Hq, Hkv, N, kv_cap, d,
                                           q_head_begin, n_q_heads, scale);
    if (st != RTP_OK) return st;
    if (!aligned(idx, 4) || !aligned(count, 4)) return RTP_ERR_ALIGN;
    if (rtp::sparse_ws_bytes(B, n_q_heads, N) > rtp::noalloc_scratch_bytes()) return RTP_ERR_LIMIT;
    return from_hip(rtp::launch_sparse_decode_noalloc(q, K, V, idx, count, B, Hq, Hkv, N, kv_cap,
                                                      q_head_begin, n_q_heads, scale, out,
                                                      as_stream(stream)));
}

rtp_status rtp_sparse_decode_union(const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V,
                                   const uint32_t *keep_bits, int32_t B, int32_t Hq,
                                   int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                                   int32_t q_head_begin, int32_t n_q_heads, float scale,
                                   float *out, void *workspace, size_t ws_bytes, void *stream)
{
    if (!keep_bits) return RTP_ERR_NULL;
    rtp_status st = check_attention_common(q, K, V, out, workspace, B, Hq, Hkv, N, kv_cap, d,
                                           q_head_begin, n_q_heads, scale);
    if (st != RTP_OK) return st;
    if (!aligned(keep_bits, 4)) return RTP_ERR_ALIGN;
    const int64_t G = Hq / Hkv;
    const int64_t groups = ((int64_t)q_head_begin + n_q_heads - 1) / G - q_head_begin / G + 1;
    if (groups * ((G + 7) / 8) > kMaxGridY) return RTP_ERR_SHAPE;
    if (ws_bytes < rtp::union_ws_bytes(B, n_q_heads, N)) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_sparse_decode_union(q, K, V, keep_bits, B, Hq, Hkv, N, kv_cap,
                                                    q_head_begin, n_q_heads, scale, out,
                                                    workspace, as_stream(stream)));
}

rtp_status rtp_local_decode(const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                            int32_t q_head_begin, int32_t n_q_heads, int32_t n_sink,
                            int32_t window, float scale, float *out, void *workspace,
                            size_t ws_bytes, void *stream)
{
    rtp_status st = check_attention_common(q, K, V, out, workspace, B, Hq, Hkv, N, kv_cap, d,
                                           q_head_begin, n_q_heads, scale);
    if (st != RTP_OK) return st;
    if (n_sink < 0 || window < 1) return RTP_ERR_VALUE;
    const int64_t G = Hq / Hkv;
    const int64_t groups = ((int64_t)q_head_begin + n_q_heads - 1) / G - q_head_begin / G + 1;
    if (groups * ((G + 7) / 8) > kMaxGridY) return RTP_ERR_SHAPE;
    if (ws_bytes < rtp::local_ws_bytes(B, n_q_heads, N)) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_local_decode(q, K, V, B, Hq, Hkv, N, kv_cap, q_head_begin,
                                             n_q_heads, n_sink, window, scale, out, workspace,
                                             as_stream(stream)));
}

rtp_status rtp_local_decode_ring(const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int64_t kv_cap,
                                 int32_t d, int32_t q_head_begin, int32_t n_q_heads,
                                 int32_t n_sink, int32_t window, float scale, float *out,
                                 void *workspace, size_t ws_bytes, void *stream)
{
    if (N < 1) return RTP_ERR_SHAPE;
    if (n_sink < 0 || window < 1) return RTP_ERR_VALUE;
    // The ring holds every row it is asked for once it has n_sink + window
    // slots (fewer tokens than that never wrap).
    const int64_t ring = (int64_t)n_sink + window;
    const int32_t rows = (int32_t)(N < ring ? N : ring);
    rtp_status st = check_attention_common(q, K, V, out, workspace, B, Hq, Hkv, rows, kv_cap, d,
                                           q_head_begin, n_q_heads, scale);
    if (st != RTP_OK) return st;
    const int64_t G = Hq / Hkv;
    const int64_t groups = ((int64_t)q_head_begin + n_q_heads - 1) / G - q_head_begin / G + 1;
    if (groups * ((G + 7) / 8) > kMaxGridY) return RTP_ERR_SHAPE;
    if (ws_bytes < rtp::local_ws_bytes(B, n_q_heads, N)) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_local_decode_ring(q, K, V, B, Hq, Hkv, N, kv_cap, q_head_begin,
                                                  n_q_heads, n_sink, window, scale, out,
                                                  workspace, as_stream(stream)));
}

rtp_status rtp_prefill_attend(const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V, int32_t B,
                              int32_t Hq, int32_t Hkv, int32_t T, int64_t kv_cap, int32_t d,
                              int32_t head_begin, int32_t n_heads, int32_t n_sink,
                              int32_t window, float scale, float *out, void *stream)
{
    if (!q || !K || !V || !out) return RTP_ERR_NULL;
    if (d != 128) return RTP_ERR_UNSUPPORTED;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || T < 1 || T > INT32_MAX - 1024 ||
        kv_cap < T)
        return RTP_ERR_SHAPE;
    if (head_begin < 0 || n_heads < 1 || (int64_t)head_begin + n_heads > Hq ||
        (int64_t)B * n_heads > kMaxGridY)
        return RTP_ERR_SHAPE;
    if (!isfinite(scale) || (window >= 1 && n_sink < 0)) return RTP_ERR_VALUE;
    if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 4))
        return RTP_ERR_ALIGN;
    return from_hip(rtp::launch_prefill_attend(q, K, V, B, Hq, Hkv, T, kv_cap, head_begin,
                                               n_heads, window >= 1 ? n_sink : 0, window, scale,
                                               out, as_stream(stream)));
}

rtp_status rtp_decode_attend(const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V,
                             const int32_t *idx, const int32_t *count, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                             int32_t sparse_head_begin, int32_t n_sparse_heads,
                             int32_t local_head_begin, int32_t n_local_heads, int32_t n_sink,
                             int32_t window, float scale, float *out, void *workspace,
                             size_t ws_bytes, void *stream)
{
    if (n_sparse_heads < 0 || n_local_heads < 0) return RTP_ERR_SHAPE;
    if (n_sparse_heads == 0 && n_local_heads == 0) return RTP_ERR_SHAPE;
    if (n_sparse_heads > 0) {
        if (!idx || !count) return RTP_ERR_NULL;
        rtp_status st = check_attention_common(q, K, V, out, workspace, B, Hq, Hkv, N, kv_cap,
                                               d, sparse_head_begin, n_sparse_heads, scale);
        if (st != RTP_OK) return st;
        if (!aligned(idx, 4) || !aligned(count, 4)) return RTP_ERR_ALIGN;
    }
    int64_t local_blocks = 0;
    if (n_local_heads > 0) {
        rtp_status st = check_attention_common(q, K, V, out, workspace, B, Hq, Hkv, N, kv_cap,
                                               d, local_head_begin, n_local_heads, scale);
        if (st != RTP_OK) return st;
        if (n_sink < 0 || window < 1) return RTP_ERR_VALUE;
        const int64_t G = Hq / Hkv;
        const int64_t groups =
            ((int64_t)local_head_begin + n_local_heads - 1) / G - local_head_begin / G + 1;
        local_blocks = (int64_t)B * groups * ((G + 7) / 8) * rtp::local_splits(N);
    }
    if (n_sparse_heads > 0 && n_local_heads > 0 &&
        sparse_head_begin < (int64_t)local_head_begin + n_local_heads &&
        local_head_begin < (int64_t)sparse_head_begin + n_sparse_heads)
        return RTP_ERR_SHAPE;  // the two head ranges overlap
    const int64_t sparse_blocks = n_sparse_heads > 0 ? rtp::sparse_grid((int64_t)B * n_sparse_heads) : 0;
    if (local_blocks + sparse_blocks > INT32_MAX) return RTP_ERR_SHAPE;
    if (ws_bytes < rtp::attend_ws_bytes(B, n_sparse_heads, n_local_heads, N))
        return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_decode_attend(q, K, V, idx, count, B, Hq, Hkv, N, kv_cap,
                                              sparse_head_begin, n_sparse_heads,
                                              local_head_begin, n_local_heads, n_sink, window,
                                              scale, out, workspace, as_stream(stream)));
}

// The sizes of a one-launch layer, checked on the host alone.
static rtp_status layer_sizes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t Hq_r,
                              int32_t n_sink, int32_t window)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || N < 1 || Hq_r < 1 || Hq_r > Hq)
        return RTP_ERR_SHAPE;
    if (Hq_r % (Hq / Hkv) != 0) return RTP_ERR_SHAPE;  // whole KV heads
    if (Hq_r < Hq && (n_sink < 0 || window < 1)) return RTP_ERR_VALUE;
    return RTP_OK;
}

// The geometry of a one-launch layer on the current device (sizes checked).
static rtp_status layer_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t Hq_r,
                              int32_t n_sink, int32_t window, rtp::LayerGeom *L)
{
    const rtp_status st = layer_sizes(B, Hq, Hkv, N, Hq_r, n_sink, window);
    if (st != RTP_OK) return st;
    int cus = 0;
    const hipError_t e = rtp::device_cus(&cus);
    if (e != hipSuccess) return from_hip(e);
    *L = rtp::layer_geom(cus, B, Hq, Hkv, N, Hq_r, Hq_r < Hq ? n_sink : 0,
                         Hq_r < Hq ? window : 1);
    return L->ok ? RTP_OK : RTP_ERR_UNSUPPORTED;
}

rtp_status rtp_decode_layer_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                                           int32_t Hq_r, int32_t n_sink, int32_t window,
                                           size_t *bytes)
{
    if (!bytes) return RTP_ERR_NULL;
    rtp::LayerGeom L;
    const rtp_status st = layer_shape(B, Hq, Hkv, N, Hq_r, n_sink, window, &L);
    if (st != RTP_OK) return st;
    *bytes = rtp::layer_ws_bytes(L, B, N);
    return RTP_OK;
}

rtp_status rtp_decode_layer(const float *q_r, const float *k_r, int64_t kr_cap,
                            const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V,
                            int64_t kv_cap, int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                            int32_t d, int32_t r, int32_t Hq_r, int32_t n_sink, int32_t window,
                            float p, float scale, float *out, int32_t *idx, int32_t *count,
                            float *scores, void *workspace, size_t ws_bytes, void *stream)
{
    if (!q_r || !k_r || !q || !K || !V || !out || !idx || !count || !workspace)
        return RTP_ERR_NULL;
    if (d != 128 || r != 16) return RTP_ERR_UNSUPPORTED;
    if (N < 1 || kr_cap < N || kv_cap < N) return RTP_ERR_SHAPE;
    rtp_status st = layer_sizes(B, Hq, Hkv, N, Hq_r, n_sink, window);
    if (st != RTP_OK) return st;
    if (!(p > 0.0f && p <= 1.0f) || !isfinite(scale)) return RTP_ERR_VALUE;
    if (!aligned(q_r, 16) || !aligned(k_r, 16) || !aligned(q, 16) || !aligned(K, 16) ||
        !aligned(V, 16) || !aligned(out, 4) || !aligned(idx, 4) || !aligned(count, 4) ||
        !aligned(scores, 4) || !aligned(workspace, 256))
        return RTP_ERR_ALIGN;
    rtp::LayerGeom L;
    st = layer_shape(B, Hq, Hkv, N, Hq_r, n_sink, window, &L);
    if (st != RTP_OK) return st;
    if (ws_bytes < rtp::layer_ws_bytes(L, B, N)) return RTP_ERR_WORKSPACE;
    rtp::WaitCtl wc;
    hipError_t e = rtp::wait_ctl(&wc);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(rtp::launch_decode_layer(L, q_r, k_r, kr_cap, q, K, V, kv_cap, B, Hq, Hkv, N,
                                             Hq_r, p, scale, out, idx, count, scores, workspace,
                                             wc.limit, wc.status, as_stream(stream)));
}

// Sizes of a top-p + attention launch that need no device (checked first).
static rtp_status topp_attend_sizes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t Hq_r,
                                    int32_t n_sink, int32_t window)
{
    const rtp_status st = layer_sizes(B, Hq, Hkv, N, Hq_r, n_sink, window);
    if (st != RTP_OK) return st;
    if (Hq / Hkv > 8 || (int64_t)B * Hq_r > 1024 ||
        (int64_t)B * Hq_r * (int64_t)N > (int64_t)UINT32_MAX)
        return RTP_ERR_UNSUPPORTED;
    return RTP_OK;
}

// The launch shape on the current device (its compute units).
static rtp_status topp_attend_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t Hq_r,
                                    int32_t n_sink, int32_t window, int *cus)
{
    const hipError_t e = rtp::device_cus(cus);
    if (e != hipSuccess) return from_hip(e);
    return rtp::topp_attend_fits(*cus, B, Hq, Hkv, N, Hq_r, Hq_r < Hq ? n_sink : 0,
                                 Hq_r < Hq ? window : 1)
               ? RTP_OK
               : RTP_ERR_UNSUPPORTED;
}

rtp_status rtp_topp_attend_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                                          int32_t Hq_r, int32_t n_sink, int32_t window,
                                          size_t *bytes)
{
    if (!bytes) return RTP_ERR_NULL;
    rtp_status st = topp_attend_sizes(B, Hq, Hkv, N, Hq_r, n_sink, window);
    if (st != RTP_OK) return st;
    int cus = 0;
    st = topp_attend_shape(B, Hq, Hkv, N, Hq_r, n_sink, window, &cus);
    if (st != RTP_OK) return st;
    *bytes = rtp::topp_attend_ws_bytes(cus, B, Hq, Hkv, N, Hq_r, Hq_r < Hq ? n_sink : 0,
                                       Hq_r < Hq ? window : 1);
    return RTP_OK;
}

// rtp_topp_attend: checks, then the launch.
static rtp_status topp_attend_call(const float *scores, const rtp_bf16 *q, const rtp_bf16 *K,
                                   const rtp_bf16 *V, int32_t B, int32_t Hq, int32_t Hkv,
                                   int32_t N, int64_t kv_cap, int32_t d, int32_t Hq_r,
                                   int32_t n_sink, int32_t window, float p, float scale,
                                   float *out, int32_t *idx, int32_t *count, void *workspace,
                                   size_t ws_bytes, void *stream)
{
    if (!scores || !q || !K || !V || !out || !idx || !count || !workspace) return RTP_ERR_NULL;
    if (d != 128) return RTP_ERR_UNSUPPORTED;
    if (N < 1 || kv_cap < N) return RTP_ERR_SHAPE;
    rtp_status st = topp_attend_sizes(B, Hq, Hkv, N, Hq_r, n_sink, window);
    if (st != RTP_OK) return st;
    if (!(p > 0.0f && p <= 1.0f) || !isfinite(scale)) return RTP_ERR_VALUE;
    if (!aligned(scores, 4) || !aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) ||
        !aligned(out, 4) || !aligned(idx, 4) || !aligned(count, 4) || !aligned(workspace, 256))
        return RTP_ERR_ALIGN;
    int cus = 0;
    st = topp_attend_shape(B, Hq, Hkv, N, Hq_r, n_sink, window, &cus);
    if (st != RTP_OK) return st;
    const int ns = Hq_r < Hq ? n_sink : 0, win = Hq_r < Hq ? window : 1;
    if (ws_bytes < rtp::topp_attend_ws_bytes(cus, B, Hq, Hkv, N, Hq_r, ns, win))
        return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_topp_attend(scores, q, K, V, B, Hq, Hkv, N, kv_cap, Hq_r, ns, win,
                                            p, scale, out, idx, count, workspace,
                                            as_stream(stream)));
}

rtp_status rtp_topp_attend(const float *scores, const rtp_bf16 *q, const rtp_bf16 *K,
                           const rtp_bf16 *V, int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                           int64_t kv_cap, int32_t d, int32_t Hq_r, int32_t n_sink,
                           int32_t window, float p, float scale, float *out, int32_t *idx,
                           int32_t *count, void *workspace, size_t ws_bytes, void *stream)
{
    return topp_attend_call(scores, q, K, V, B, Hq, Hkv, N, kv_cap, d, Hq_r, n_sink, window, p,
                            scale, out, idx, count, workspace, ws_bytes, stream);
}

rtp_status rtp_scan_local(const float *q_r, const float *k_r, float *scores, int32_t Hq_r,
                          int32_t Hkv_r, int64_t kr_cap, int32_t r, const rtp_bf16 *q,
                          const rtp_bf16 *K, const rtp_bf16 *V, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                          int32_t local_head_begin, int32_t n_local_heads, int32_t n_sink,
                          int32_t window, float scale, float *out, void *workspace,
                          size_t ws_bytes, void *stream)
{
    if (!q_r || !k_r || !scores) return RTP_ERR_NULL;
    rtp_status st = check_attention_common(q, K, V, out, workspace, B, Hq, Hkv, N, kv_cap, d,
                                           local_head_begin, n_local_heads, scale);
    if (st != RTP_OK) return st;
    if (r != 16) return RTP_ERR_UNSUPPORTED;
    if (Hq_r < 1 || Hkv_r < 1 || Hq_r % Hkv_r != 0 || kr_cap < N) return RTP_ERR_SHAPE;
    if (n_sink < 0 || window < 1) return RTP_ERR_VALUE;
    const int64_t G = Hq / Hkv;
    const int64_t groups =
        ((int64_t)local_head_begin + n_local_heads - 1) / G - local_head_begin / G + 1;
    if (groups * ((G + 7) / 8) > kMaxGridY) return RTP_ERR_SHAPE;
    if (rtp::scan_local_blocks(B, Hq_r, Hkv_r, Hq, Hkv, N, local_head_begin, n_local_heads) >
        INT32_MAX)
        return RTP_ERR_SHAPE;
    if (!aligned(q_r, 16) || !aligned(k_r, 16) || !aligned(scores, 4)) return RTP_ERR_ALIGN;
    if (ws_bytes < rtp::local_ws_bytes(B, n_local_heads, N)) return RTP_ERR_WORKSPACE;
    return from_hip(rtp::launch_scan_local(q_r, k_r, scores, Hq_r, Hkv_r, kr_cap, q, K, V, B, Hq,
                                           Hkv, N, kv_cap, local_head_begin, n_local_heads,
                                           n_sink, window, scale, out, workspace,
                                           as_stream(stream)));
}

}  // extern "C"
