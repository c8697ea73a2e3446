/*
 * rtp.h -- C ABI of the RTPurbo sparse decode attention path on MI355X
 * (gfx950), "Full Attention Strikes Back: Transferring Full Attention into
 * Sparse within Hundred Training Steps" (arXiv 2605.16928).
 *
 * One decode step of one attention layer, per the pages' statement of the
 * method (gist.science summary, method sections 1-3 and 5):
 *   - retrieval heads score every cached token with a 16-dim low-rank
 *     indexer taken before RoPE            -> rtp_index_scores
 *   - keep the smallest set of tokens whose low-dim softmax mass reaches p,
 *     found by a sort-free histogram threshold       -> rtp_topp_select
 *   - exact attention over the selected K/V rows only -> rtp_sparse_decode
 *   - local heads attend sink tokens plus a sliding window
 *                                                     -> rtp_local_decode
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees, or keeps a pointer after the call.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream).  No call synchronises the host; results are ready when the
 *     stream reaches them.  Calls are stateless and may be captured in a HIP
 *     graph.  Calls that overlap on one device must use distinct workspaces.
 *   - Arguments are validated on the host before anything is launched.  On
 *     any error nothing is launched and no output is touched.  A failure
 *     reported by the HIP runtime at launch returns RTP_ERR_HIP.
 *   - Inputs must be finite; non-finite values give unspecified results.
 *   - bf16 tensors are passed as their 16-bit patterns (rtp_bf16).
 *   - Layouts are row-major.  "cap" is a cache's capacity in tokens (its
 *     row count per head); only the first N rows of each head are read.
 *   - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 */
#ifndef RTP_H
#define RTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t rtp_bf16; /* bfloat16 bit pattern */

typedef enum rtp_status {
    RTP_OK = 0,
    RTP_ERR_NULL = 1,        /* a required pointer is NULL                  */
    RTP_ERR_SHAPE = 2,       /* a size is out of range or inconsistent      */
    RTP_ERR_UNSUPPORTED = 3, /* r != 16, d != 128, too many heads per group */
    RTP_ERR_VALUE = 4,       /* p not in (0,1], bad window/sink, bad scale  */
    RTP_ERR_ALIGN = 5,       /* a pointer or capacity breaks alignment      */
    RTP_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required     */
    RTP_ERR_HIP = 7,         /* the HIP runtime reported an error           */
    RTP_ERR_LIMIT = 8        /* beyond the no-allocation entry point's scratch */
} rtp_status;

/* Workspace kinds for rtp_workspace_size. */
enum {
    RTP_WS_TOPP_SELECT = 1,
    RTP_WS_SPARSE_DECODE = 2,
    RTP_WS_LOCAL_DECODE = 3,
    RTP_WS_SPARSE_UNION = 4,
    RTP_WS_DECODE_ATTEND = 5
};

/*
 * rtp_index_scores -- indexer score of every cached token for each
 * retrieval query head (gist.science summary, method section 2: a 16-dim
 * projector applied to queries and keys before RoPE; the arXiv abstract
 * gives the indexer's width as 16).
 *
 *   scores[b][h][i] = q_r[b][h] . k_r[b][h / (Hq_r/Hkv_r)][i],  i < N,
 * in fp32, accumulated as one fused multiply-add per dimension in the order
 * j = 0..15 starting from +0, with a zero result stored as +0.  The result
 * is bit-exact: no reassociation, no flush of denormals.
 *
 *   q_r     fp32 [B][Hq_r][r]          16-B aligned
 *   k_r     fp32 [B][Hkv_r][kr_cap][r] 16-B aligned
 *   scores  fp32 [B][Hq_r][N]          out, 4-B aligned
 *   r must be 16; Hq_r must be a multiple of Hkv_r; 1 <= N <= kr_cap.
 */
rtp_status rtp_index_scores(const float *q_r, const float *k_r, float *scores,
                            int32_t B, int32_t Hq_r, int32_t Hkv_r, int32_t N,
                            int64_t kr_cap, int32_t r, void *stream);

/*
 * rtp_index_scores_bf16 -- rtp_index_scores over an indexer key cache stored
 * in bf16 (32 B per token instead of 64: the scan reads half the bytes).
 * Each bf16 element is widened exactly to fp32 and the score is then the
 * same fp32 fused multiply-add chain as rtp_index_scores, so it is
 * bit-exact to rtp_index_scores run on the widened cache.
 *
 *   q_r     fp32 [B][Hq_r][r]          16-B aligned
 *   k_r     bf16 [B][Hkv_r][kr_cap][r] 16-B aligned
 *   scores  fp32 [B][Hq_r][N]          out, 4-B aligned
 *   The same sizes and errors as rtp_index_scores.
 */
rtp_status rtp_index_scores_bf16(const float *q_r, const rtp_bf16 *k_r,
                                 float *scores, int32_t B, int32_t Hq_r,
                                 int32_t Hkv_r, int32_t N, int64_t kr_cap,
                                 int32_t r, void *stream);

/*
 * rtp_index_project -- the indexer's low-dim projection of query or key
 * features taken before RoPE (gist.science summary, method section 2: a
 * 16-dim projector applied to queries and keys before RoPE), for one decode
 * token (q_r of the retrieval heads, or the new k_r row appended to the
 * indexer key cache) or a whole prefill (the k_r cache of T tokens).
 *
 *   out[b][h][out_pos + t][j] = sum_{c < d} W[h][j][c] * x[b][head_begin + h][t][c]
 *
 * for t < T, j < r, h < H.  Each bf16 product is exact in fp32 and the sum
 * is accumulated in fp32 on the matrix cores, in an unspecified order: the
 * result is within 2 * d * 2^-24 * sum_c |W[h][j][c] * x[..][c]| of the
 * exact sum, and the same inputs always give the same bits (a token's row
 * does not depend on T or on the other tokens).
 *
 *   x        bf16 [B][Hx][x_cap][d]   16-B aligned; rows [0, T) of heads
 *                                     [head_begin, head_begin + H) are read
 *   W        bf16 [H][r][d]           16-B aligned; one projector per head
 *   out      fp32 [B][H][out_cap][r]  4-B aligned; rows [out_pos,
 *                                     out_pos + T) written, the rest untouched
 *   d must be 128 and r must be 16; 1 <= T <= x_cap, T <= 2^31 - 1025;
 *   0 <= out_pos <= out_cap - T; 0 <= head_begin <= Hx - H; B*H <= 65535.
 *
 * Errors: RTP_ERR_NULL, RTP_ERR_UNSUPPORTED (d or r), RTP_ERR_SHAPE,
 * RTP_ERR_ALIGN.
 */
rtp_status rtp_index_project(const rtp_bf16 *x, int32_t B, int32_t Hx,
                             int64_t x_cap, int32_t head_begin, int32_t H,
                             int32_t T, int32_t d, const rtp_bf16 *W,
                             int32_t r, float *out, int64_t out_cap,
                             int64_t out_pos, void *stream);

/*
 * rtp_topp_select -- dynamic top-p token selection per head (gist.science
 * summary, method section 3: the low-dim attention mass is summed, largest
 * first, until it reaches p; section 5: the threshold is found with a
 * histogram instead of a sort).
 *
 * For each of the B*H score rows, with e_i = exp(s_i - max s) in fp64 and
 * Z = sum of e_i over all N tokens: order tokens by score, descending, ties
 * to the lower index; keep the shortest prefix whose mass is >= p*Z
 * (p widened to fp64).  p == 1 keeps all N tokens.
 *
 *   scores     fp32  [B][H][N]   4-B aligned; -0 is treated as +0
 *   p          in (0, 1]
 *   idx        int32 [B][H][N]   out: the kept token indices of row (b,h)
 *                                in idx[b][h][0 .. count[b][h]), in no
 *                                particular order; the rest is untouched
 *   count      int32 [B][H]      out: size of each kept set (>= 1)
 *   keep_bits  uint32 [B][H][ceil(N/32)]  optional out (NULL: not written):
 *                                the same sets as a bitmap, bit i%32 of
 *                                word i/32 set iff token i is kept; every
 *                                word is written (no initialisation needed).
 *                                rtp_sparse_decode_union reads it.
 *   workspace  device memory of at least
 *              rtp_workspace_size(RTP_WS_TOPP_SELECT, B, H, N) bytes,
 *              256-B aligned; contents need no initialisation.
 */
rtp_status rtp_topp_select(const float *scores, int32_t B, int32_t H,
                           int32_t N, float p, int32_t *idx, int32_t *count,
                           uint32_t *keep_bits, void *workspace,
                           size_t ws_bytes, void *stream);

/*
 * rtp_topk_select -- static top-k token selection per head: the fixed
 * budget that dynamic top-p replaces (gist.science summary, method section
 * 3, dynamic top-p versus static top-k; arXiv abstract, third observation).
 *
 * For each of the B*H score rows: order tokens by score, descending, ties
 * to the lower index, and keep the first min(k, N).  It runs the machinery
 * of rtp_topp_select with every token weighing 1 instead of its mass.
 *
 *   scores     fp32  [B][H][N]   4-B aligned; -0 is treated as +0
 *   k          >= 1; k >= N keeps all N tokens
 *   idx, count, keep_bits, workspace, ws_bytes, stream
 *              as in rtp_topp_select (count[b][h] = min(k, N); the same
 *              workspace size)
 *
 * Errors: RTP_ERR_NULL (scores, idx, count or workspace NULL),
 * RTP_ERR_SHAPE (B, H or N < 1, or B*H > 65535), RTP_ERR_VALUE (k < 1),
 * RTP_ERR_ALIGN, RTP_ERR_WORKSPACE.
 */
rtp_status rtp_topk_select(const float *scores, int32_t B, int32_t H,
                           int32_t N, int32_t k, int32_t *idx, int32_t *count,
                           uint32_t *keep_bits, void *workspace,
                           size_t ws_bytes, void *stream);

/*
 * rtp_keep_bits_add_local -- adds the local rows (the first n_sink tokens
 * and the newest `window`, as rtp_local_decode reads them) to every keep
 * bitmap row, so that rtp_sparse_decode_union lets a retrieval head attend
 * its selected set plus the sinks and the window.  The pages let retrieval
 * heads switch to the selected set alone (gist.science summary, method
 * section 1); this is the variant where they keep the local rows too.
 *
 *   keep_bits  uint32 [B][H][ceil(N/32)]  in/out, 4-B aligned: bits are only set
 *   n_sink >= 0, window >= 1
 *
 * Errors: RTP_ERR_NULL, RTP_ERR_SHAPE (B, H or N < 1, B*H > 65535),
 * RTP_ERR_VALUE (n_sink or window), RTP_ERR_ALIGN.
 */
rtp_status rtp_keep_bits_add_local(uint32_t *keep_bits, int32_t B, int32_t H,
                                   int32_t N, int32_t n_sink, int32_t window,
                                   void *stream);

/*
 * rtp_topp_hist -- the histogram pass of rtp_topp_select on its own: the
 * per-row mass histograms (same passage) are left in the workspace and no
 * output is written.  rtp_topp_select runs this pass and the emit pass that
 * consumes the histograms in one launch (in two launches when B*H exceeds
 * 32767); calling rtp_topp_hist alone is harmless (a later rtp_topp_select
 * starts over).  It exists so that the histogram pass can be timed or
 * profiled apart.
 *
 *   scores, B, H, N, workspace as in rtp_topp_select.
 */
rtp_status rtp_topp_hist(const float *scores, int32_t B, int32_t H, int32_t N,
                         void *workspace, size_t ws_bytes, void *stream);

/*
 * rtp_sparse_decode -- exact attention of each retrieval query head over
 * its selected rows only (arXiv abstract: sparse attention over the
 * indexer's tokens; gist.science summary, method section 5: bandwidth-
 * optimised sparse decode).
 *
 *   out[b][h][:] = sum_{i in S} softmax_S(scale * q[b][h] . K[b][g][i])
 *                  * V[b][g][i][:],  g = h / (Hq/Hkv),
 * with S = idx[b][h - q_head_begin][0 .. count), fp32 arithmetic, softmax
 * renormalised over S.
 *
 *   q          bf16  [B][Hq][d]          16-B aligned
 *   K, V       bf16  [B][Hkv][kv_cap][d] 16-B aligned
 *   idx        int32 [B][n_q_heads][N]   as written by rtp_topp_select;
 *                                        every entry must be < N
 *   count      int32 [B][n_q_heads]      each in [1, N]
 *   heads      q_head_begin .. q_head_begin + n_q_heads - 1 (within Hq)
 *   out        fp32  [B][Hq][d]          only the heads in range written
 *   workspace  >= rtp_workspace_size(RTP_WS_SPARSE_DECODE, B, n_q_heads, N)
 *   d must be 128; 1 <= N <= kv_cap; scale finite.
 */
rtp_status rtp_sparse_decode(const rtp_bf16 *q, const rtp_bf16 *K,
                             const rtp_bf16 *V, const int32_t *idx,
                             const int32_t *count, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                             int32_t q_head_begin, int32_t n_q_heads,
                             float scale, float *out, void *workspace,
                             size_t ws_bytes, void *stream);

/*
 * rtp_sparse_decode_noalloc -- rtp_sparse_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with the
 * workspace taken from a static device array of the library (4 MiB per
 * device, held until the process ends) instead of a caller's buffer.  The
 * call allocates nothing.  Every call on one device shares that array:
 * calls that overlap on a device (different streams, threads) race and give
 * undefined results; calls in sequence are fine.
 *
 *   every argument as in rtp_sparse_decode, minus workspace and ws_bytes
 *   limit: rtp_workspace_size(RTP_WS_SPARSE_DECODE, B, n_q_heads, N) must
 *   fit in the 4 MiB (B * n_q_heads <= 256 always does)
 *
 * Errors: those of rtp_sparse_decode, and RTP_ERR_LIMIT when the sizes need
 * more than the static scratch.
 */
rtp_status rtp_sparse_decode_noalloc(const rtp_bf16 *q, const rtp_bf16 *K,
                                     const rtp_bf16 *V, const int32_t *idx,
                                     const int32_t *count, int32_t B, int32_t Hq,
                                     int32_t Hkv, int32_t N, int64_t kv_cap,
                                     int32_t d, int32_t q_head_begin,
                                     int32_t n_q_heads, float scale, float *out,
                                     void *stream);

/*
 * rtp_sparse_decode_union -- the same attention as rtp_sparse_decode, with
 * the kept sets given as keep bitmaps (as written by rtp_topp_select) and
 * each K/V row read once for all query heads of its KV head that kept it
 * (grouped-query attention: the heads of one KV head share its rows).
 *
 *   out[b][h][:] = sum_{i in S_h} softmax_{S_h}(scale * q[b][h] . K[b][g][i])
 *                  * V[b][g][i][:],  g = h / (Hq/Hkv),
 * with S_h = { i < N : bit i%32 of keep_bits[b][h - q_head_begin][i/32] },
 * fp32 arithmetic, softmax renormalised over S_h.  Bits at or past N in the
 * last word are ignored.  Every S_h must be non-empty.
 *
 *   q          bf16   [B][Hq][d]                 16-B aligned
 *   K, V       bf16   [B][Hkv][kv_cap][d]        16-B aligned
 *   keep_bits  uint32 [B][n_q_heads][ceil(N/32)] 4-B aligned
 *   heads      q_head_begin .. q_head_begin + n_q_heads - 1 (within Hq)
 *   out        fp32   [B][Hq][d]                 only the heads in range written
 *   workspace  >= rtp_workspace_size(RTP_WS_SPARSE_UNION, B, n_q_heads, N)
 *   d must be 128; 1 <= N <= kv_cap; scale finite.
 */
rtp_status rtp_sparse_decode_union(const rtp_bf16 *q, const rtp_bf16 *K,
                                   const rtp_bf16 *V, const uint32_t *keep_bits,
                                   int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                                   int64_t kv_cap, int32_t d,
                                   int32_t q_head_begin, int32_t n_q_heads,
                                   float scale, float *out, void *workspace,
                                   size_t ws_bytes, void *stream);

/*
 * rtp_local_decode -- local heads: attention over the first n_sink cached
 * rows (attention sinks) plus the newest `window` rows, each row once
 * (gist.science summary, method section 1: local heads use a sliding window
 * with attention sinks).  The query is the newest token, whose K/V is row
 * N-1.  Each K/V row is read once per KV head and serves all its query
 * heads in range.
 *
 *   q, K, V, out, heads, d, scale as in rtp_sparse_decode
 *   n_sink >= 0, window >= 1
 *   workspace  >= rtp_workspace_size(RTP_WS_LOCAL_DECODE, B, n_q_heads, N)
 */
rtp_status rtp_local_decode(const rtp_bf16 *q, const rtp_bf16 *K,
                            const rtp_bf16 *V, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                            int32_t q_head_begin, int32_t n_q_heads,
                            int32_t n_sink, int32_t window, float scale,
                            float *out, void *workspace, size_t ws_bytes,
                            void *stream);

/*
 * rtp_local_decode_ring -- rtp_local_decode over a ring-buffer local cache
 * that keeps only the rows a local head can attend (arXiv abstract: the full
 * KV cache is kept for retrieval heads only; summary section 1: local heads
 * see sinks plus a window).  Token i < n_sink sits in slot i; token
 * i >= n_sink in slot n_sink + (i - n_sink) % window, so a cache of
 * n_sink + window slots always holds the newest window tokens.  N is the
 * number of tokens seen (the newest is N-1); the result is bit-identical to
 * rtp_local_decode on the linear cache.
 *
 *   K, V   bf16 [B][Hkv][kv_cap][d]  ring slots, kv_cap >= min(N, n_sink + window)
 *   every other argument, and the errors, as in rtp_local_decode
 *   (workspace sized with the same N)
 */
rtp_status rtp_local_decode_ring(const rtp_bf16 *q, const rtp_bf16 *K,
                                 const rtp_bf16 *V, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t N, int64_t kv_cap,
                                 int32_t d, int32_t q_head_begin,
                                 int32_t n_q_heads, int32_t n_sink,
                                 int32_t window, float scale, float *out,
                                 void *workspace, size_t ws_bytes,
                                 void *stream);

/*
 * rtp_prefill_attend -- causal prefill attention for a range of query heads,
 * dense (retrieval heads) or sinks + window (local heads) (gist.science
 * summary, method section 1: the two head roles; the arXiv abstract credits
 * the prefill speed-up at 1M context to them).  For query token t < T:
 *
 *   window <= 0  keys [0, t]
 *   window >= 1  keys [0, min(n_sink, w0)) and [w0, t], w0 = max(0, t+1-window)
 *   out[b][h][t][:] = sum_i softmax_i(scale * q[b][h][t] . K[b][g][i]) * V[b][g][i][:]
 *
 * with g = h / (Hq/Hkv): the local rows of each t are those rtp_local_decode
 * reads with N = t + 1.  Matrix cores with fp32 accumulation: q.K in bf16;
 * the second product takes the probabilities rounded to fp16 (2^-11
 * relative) and V converted to fp16 (exact for magnitudes in [2^-14, 2^16);
 * a block of 32 dimensions x 64 keys whose largest magnitude is 2^16 or
 * more, or below 2^-10, is scaled by a power of two, each value then kept
 * to within 2^-40 of the block's largest), and
 * the softmax sum adds the same rounded probabilities: each output is an
 * average of V rows under weights within 2^-10 (relative) of the exact
 * softmax, so its error is at most 2^-10 of the weighted mean of
 * |V - out|.  fp32 softmax and output.
 *
 *   q      bf16 [B][Hq][T][d]       16-B aligned (the prompt's queries, post-RoPE)
 *   K, V   bf16 [B][Hkv][kv_cap][d] 16-B aligned; rows [0, T) are the prompt
 *   out    fp32 [B][Hq][T][d]       4-B aligned; heads [head_begin,
 *                                   head_begin + n_heads) written
 *   d must be 128; 1 <= T <= kv_cap, T <= 2^31 - 1025; B*n_heads <= 65535; n_sink >= 0 when
 *   window >= 1; scale finite.
 *
 * Errors: RTP_ERR_NULL, RTP_ERR_UNSUPPORTED, RTP_ERR_SHAPE, RTP_ERR_VALUE,
 * RTP_ERR_ALIGN.
 */
rtp_status rtp_prefill_attend(const rtp_bf16 *q, const rtp_bf16 *K,
                              const rtp_bf16 *V, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t T, int64_t kv_cap, int32_t d,
                              int32_t head_begin, int32_t n_heads,
                              int32_t n_sink, int32_t window, float scale,
                              float *out, void *stream);

/*
 * rtp_decode_attend -- rtp_sparse_decode for the query heads
 * sparse_head_begin .. sparse_head_begin + n_sparse_heads - 1 and
 * rtp_local_decode for the query heads local_head_begin ..
 * local_head_begin + n_local_heads - 1, in one launch, so that neither set
 * waits for the other's tail (the head-role split of the gist.science
 * summary, method section 1: retrieval and local heads of one layer).  The
 * results are those of the two calls.  The two head ranges must not overlap;
 * either count may be 0, which skips that set (idx and count may then be
 * NULL; n_sink and window are ignored when n_local_heads is 0).
 *
 *   q, K, V, out, d, scale         as in rtp_sparse_decode
 *   idx, count                     as in rtp_sparse_decode, for the sparse heads
 *   n_sink, window                 as in rtp_local_decode
 *   workspace  >= rtp_workspace_size(RTP_WS_DECODE_ATTEND, B, Hq, N)
 */
rtp_status rtp_decode_attend(const rtp_bf16 *q, const rtp_bf16 *K,
                             const rtp_bf16 *V, const int32_t *idx,
                             const int32_t *count, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                             int32_t sparse_head_begin, int32_t n_sparse_heads,
                             int32_t local_head_begin, int32_t n_local_heads,
                             int32_t n_sink, int32_t window, float scale,
                             float *out, void *workspace, size_t ws_bytes,
                             void *stream);

/*
 * rtp_scan_local -- rtp_index_scores for the retrieval heads and
 * rtp_local_decode for the query heads local_head_begin ..
 * local_head_begin + n_local_heads - 1, in one launch: the scan of the
 * gist.science summary, method section 2, and the local heads of method
 * section 1, which read disjoint inputs and write disjoint outputs.  The
 * results are those of the two calls.  Both sides use the same batch size B
 * and token count N (scores [B][Hq_r][N], rows 0 .. N-1 of K and V).
 *
 *   q_r, k_r, scores, Hq_r, Hkv_r, kr_cap, r   as in rtp_index_scores
 *   q, K, V, out, Hq, Hkv, kv_cap, d, scale,
 *   n_sink, window                             as in rtp_local_decode
 *   workspace  >= rtp_workspace_size(RTP_WS_LOCAL_DECODE, B, n_local_heads, N)
 * Errors: those of either call, checked before anything is enqueued.
 */
rtp_status rtp_scan_local(const float *q_r, const float *k_r, float *scores,
                          int32_t Hq_r, int32_t Hkv_r, int64_t kr_cap, int32_t r,
                          const rtp_bf16 *q, const rtp_bf16 *K,
                          const rtp_bf16 *V, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t N, int64_t kv_cap, int32_t d,
                          int32_t local_head_begin, int32_t n_local_heads,
                          int32_t n_sink, int32_t window, float scale,
                          float *out, void *workspace, size_t ws_bytes,
                          void *stream);

/*
 * rtp_decode_layer -- one decode step of one attention layer in a single
 * launch: the indexer scan (rtp_index_scores), top-p selection
 * (rtp_topp_select) and exact sparse attention (rtp_sparse_decode) for the
 * retrieval heads, and sinks + window attention (rtp_local_decode) for the
 * local heads (gist.science summary, method section 1: the two head roles;
 * section 2: the 16-dim indexer; section 3: top-p mass; section 5: a
 * sort-free histogram threshold and bandwidth-optimised sparse decode).
 * The kept sets and outputs are those of the four calls run in sequence;
 * the scores stay on chip unless `scores` is given.
 *
 * Head roles: query heads 0 .. Hq_r-1 are retrieval heads (on KV heads
 * 0 .. Hq_r/G - 1, G = Hq/Hkv, so Hq_r must be a multiple of G); query heads
 * Hq_r .. Hq-1 are local heads.
 *
 *   q_r     fp32 [B][Hq_r][r]           16-B aligned
 *   k_r     fp32 [B][Hq_r/G][kr_cap][r] 16-B aligned
 *   q       bf16 [B][Hq][d]             16-B aligned
 *   K, V    bf16 [B][Hkv][kv_cap][d]    16-B aligned
 *   p       in (0, 1] (the top-p mass; 1 keeps every token)
 *   scale   finite (the attention scale, e.g. 1/sqrt(d))
 *   n_sink, window   as in rtp_local_decode (ignored when Hq_r == Hq)
 *   out     fp32 [B][Hq][d]             out, every head written
 *   idx     int32 [B][Hq_r][N]          out: kept indices, in no particular order
 *   count   int32 [B][Hq_r]             out: kept-set sizes
 *   scores  fp32 [B][Hq_r][N]           optional out (NULL: not written)
 *   workspace  >= rtp_decode_layer_workspace_size(...) bytes, 256-B aligned;
 *              contents need no initialisation
 *   d must be 128 and r must be 16; G must be 1, 2, 4 or 8.
 *
 * The launch is persistent: at most one block per compute unit, and the
 * blocks of a score row wait for each other once (for the row's threshold),
 * which needs them resident together; nothing else may run on the device
 * during the call.  One launch holds up to 4096 tokens per compute unit
 * (N <= 4096 * floor(CUs / (B * Hq_r / G))); larger shapes return
 * RTP_ERR_UNSUPPORTED (use the four calls).
 *
 * Errors: RTP_ERR_NULL, RTP_ERR_UNSUPPORTED (d, r, G, or the shape above),
 * RTP_ERR_SHAPE, RTP_ERR_VALUE (p, scale, n_sink, window), RTP_ERR_ALIGN,
 * RTP_ERR_WORKSPACE.
 */
rtp_status rtp_decode_layer(const float *q_r, const float *k_r, int64_t kr_cap,
                            const rtp_bf16 *q, const rtp_bf16 *K, const rtp_bf16 *V,
                            int64_t kv_cap, int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                            int32_t d, int32_t r, int32_t Hq_r, int32_t n_sink, int32_t window,
                            float p, float scale, float *out, int32_t *idx, int32_t *count,
                            float *scores, void *workspace, size_t ws_bytes, void *stream);

/*
 * rtp_decode_layer_workspace_size -- bytes of workspace rtp_decode_layer
 * needs for these sizes on the current device (host only).  The same errors
 * as rtp_decode_layer for the sizes, plus RTP_ERR_NULL when bytes is NULL.
 */
rtp_status rtp_decode_layer_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                                           int32_t Hq_r, int32_t n_sink, int32_t window,
                                           size_t *bytes);

/*
 * rtp_topp_attend -- rtp_topp_select over the retrieval heads' scores
 * followed by rtp_decode_attend (the retrieval heads' exact attention over
 * their kept rows, the local heads' sinks + window attention), in one
 * launch (gist.science summary, method section 3: top-p mass; section 5:
 * a sort-free histogram threshold and bandwidth-optimised sparse decode;
 * section 1: the two head roles).  The kept sets and outputs are those of
 * the two calls.  Attention over the tokens the selection lists first
 * overlaps the resolution of each row's boundary bin.
 *
 * Head roles as in rtp_decode_layer: query heads 0 .. Hq_r-1 are retrieval
 * heads with score rows [B][Hq_r] (Hq_r a multiple of G = Hq/Hkv), query
 * heads Hq_r .. Hq-1 local heads.
 *
 *   scores  fp32 [B][Hq_r][N]           4-B aligned (rtp_index_scores' output)
 *   q       bf16 [B][Hq][d]             16-B aligned
 *   K, V    bf16 [B][Hkv][kv_cap][d]    16-B aligned
 *   p       in (0, 1]; p = 1 keeps every token (then two launches)
 *   scale   finite
 *   n_sink, window   as in rtp_local_decode (ignored when Hq_r == Hq)
 *   out     fp32 [B][Hq][d]             out, every head written
 *   idx     int32 [B][Hq_r][N]          out: kept indices, in no particular order
 *   count   int32 [B][Hq_r]             out: kept-set sizes
 *   workspace  >= rtp_topp_attend_workspace_size(...) bytes, 256-B aligned;
 *              contents need no initialisation
 *   d must be 128; G must be at most 8; B * Hq_r at most 1024 and
 *   B * Hq_r * N below 2^32 (else RTP_ERR_UNSUPPORTED).
 *
 * The launch relies only on blocks being dispatched in index order: a
 * block waits only for blocks with lower indices.
 *
 * Errors: RTP_ERR_NULL, RTP_ERR_UNSUPPORTED, RTP_ERR_SHAPE, RTP_ERR_VALUE
 * (p, scale, n_sink, window), RTP_ERR_ALIGN, RTP_ERR_WORKSPACE.
 */
rtp_status rtp_topp_attend(const float *scores, const rtp_bf16 *q, const rtp_bf16 *K,
                           const rtp_bf16 *V, int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                           int64_t kv_cap, int32_t d, int32_t Hq_r, int32_t n_sink,
                           int32_t window, float p, float scale, float *out, int32_t *idx,
                           int32_t *count, void *workspace, size_t ws_bytes, void *stream);

/*
 * rtp_topp_attend_workspace_size -- bytes of workspace rtp_topp_attend needs
 * for these sizes on the current device (host only).  The same errors as
 * rtp_topp_attend for the sizes, plus RTP_ERR_NULL when bytes is NULL.
 */
rtp_status rtp_topp_attend_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t N,
                                          int32_t Hq_r, int32_t n_sink, int32_t window,
                                          size_t *bytes);

/*
 * Waits between blocks.  Some kernels hand data from block to block inside
 * one launch (rtp_topp_select, rtp_topk_select, rtp_sparse_decode,
 * rtp_decode_attend, rtp_decode_layer, rtp_topp_attend); a block that waits polls at most
 * `polls` times (default 2^24) and then gives up, sets the status bit
 * RTP_STATUS_WAIT_TIMEOUT in the device's sticky status word, and goes on,
 * so the kernel still ends; the results of that call, and the state of its
 * workspace, are then undefined (fill the workspace with zeros before
 * reusing it).  A wait never needs the limit unless something else is wrong.
 *
 * rtp_set_wait_limit sets the limit for launches that follow, in this
 * process (0 gives up at once: a test hook).  Always RTP_OK.
 *
 * rtp_device_status waits for the current device to finish its work, then
 * returns its status word in *flags and, when clear is nonzero, clears it.
 * Errors: RTP_ERR_NULL (flags NULL), RTP_ERR_HIP.
 */
#define RTP_STATUS_WAIT_TIMEOUT 1u
rtp_status rtp_set_wait_limit(uint32_t polls);
rtp_status rtp_device_status(uint32_t *flags, int32_t clear);

/*
 * rtp_workspace_size -- bytes of workspace a call needs (host only, pure).
 *   which  RTP_WS_TOPP_SELECT:   H = score rows per batch row
 *          RTP_WS_SPARSE_DECODE: H = n_q_heads
 *          RTP_WS_LOCAL_DECODE:  H = n_q_heads (sized for any n_sink,
 *                                window, since the row list is <= N)
 *          RTP_WS_SPARSE_UNION:  H = n_q_heads
 *          RTP_WS_DECODE_ATTEND: H = Hq (sized for any split of the Hq
 *                                heads into sparse and local heads)
 * Returns RTP_ERR_VALUE for an unknown `which`, RTP_ERR_SHAPE for sizes < 1,
 * RTP_ERR_NULL when bytes is NULL.
 */
rtp_status rtp_workspace_size(int32_t which, int32_t B, int32_t H, int32_t N,
                              size_t *bytes);

/* Static English text for a status code (host only). */
const char *rtp_status_string(rtp_status status);

/* The hipError_t code behind the most recent RTP_ERR_HIP returned on the
 * calling thread (0 = hipSuccess if there was none).  Host only. */
int32_t rtp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RTP_H */
