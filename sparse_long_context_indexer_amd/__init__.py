"""Python binding of librtp (include/rtp.h): the RTPurbo sparse decode path
on MI355X (arXiv 2605.16928).

Argument marshalling only: each function checks dtypes and shapes of the
torch tensors it is given, reads their device pointers and the current HIP
stream, and calls the C function of the same name.  Every step of the path
runs in the HIP kernels of librtp.so; there is no fallback.  If the library
is not built, calls raise RuntimeError.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librtp.so")

RTP_WS_TOPP_SELECT = 1
RTP_WS_SPARSE_DECODE = 2
RTP_WS_LOCAL_DECODE = 3
RTP_WS_SPARSE_UNION = 4
RTP_WS_DECODE_ATTEND = 5

STATUS = {0: "RTP_OK", 1: "RTP_ERR_NULL", 2: "RTP_ERR_SHAPE", 3: "RTP_ERR_UNSUPPORTED",
          4: "RTP_ERR_VALUE", 5: "RTP_ERR_ALIGN", 6: "RTP_ERR_WORKSPACE", 7: "RTP_ERR_HIP"}

# Every symbol include/rtp.h declares.
SYMBOLS = ("rtp_index_scores", "rtp_index_scores_bf16", "rtp_index_project", "rtp_topp_select", "rtp_topk_select", "rtp_topp_hist",
           "rtp_sparse_decode", "rtp_sparse_decode_union", "rtp_local_decode",
           "rtp_local_decode_ring", "rtp_keep_bits_add_local", "rtp_prefill_attend",
           "rtp_decode_attend", "rtp_scan_local", "rtp_workspace_size", "rtp_status_string",
           "rtp_last_hip_error")


class RtpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({status_string(status)})"
        if status == 7:
            msg += f"; hipError_t {lib().rtp_last_hip_error()}"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded librtp.so with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        # PyTorch ships its own HIP runtime (soname libamdhip64.so.7).  Loading
        # torch first makes librtp bind to that copy; loading librtp first
        # would map a second HIP runtime into the process.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_float, ctypes.c_size_t)
        L.rtp_index_scores.argtypes = [P, P, P, I32, I32, I32, I32, I64, I32, P]
        L.rtp_index_scores_bf16.argtypes = [P, P, P, I32, I32, I32, I32, I64, I32, P]
        L.rtp_topp_select.argtypes = [P, I32, I32, I32, F32, P, P, P, P, SZ, P]
        L.rtp_topk_select.argtypes = [P, I32, I32, I32, I32, P, P, P, P, SZ, P]
        L.rtp_index_project.argtypes = [P, I32, I32, I64, I32, I32, I32, I32, P, I32, P, I64,
                                        I64, P]
        L.rtp_topp_hist.argtypes = [P, I32, I32, I32, P, SZ, P]
        L.rtp_sparse_decode.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I64, I32,
                                        I32, I32, F32, P, P, SZ, P]
        L.rtp_sparse_decode_union.argtypes = [P, P, P, P, I32, I32, I32, I32, I64, I32, I32,
                                              I32, F32, P, P, SZ, P]
        L.rtp_local_decode.argtypes = [P, P, P, I32, I32, I32, I32, I64, I32, I32, I32,
                                       I32, I32, F32, P, P, SZ, P]
        L.rtp_local_decode_ring.argtypes = L.rtp_local_decode.argtypes
        L.rtp_keep_bits_add_local.argtypes = [P, I32, I32, I32, I32, I32, P]
        L.rtp_prefill_attend.argtypes = [P, P, P, I32, I32, I32, I32, I64, I32, I32, I32, I32,
                                         I32, F32, P, P]
        L.rtp_decode_attend.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I64, I32, I32, I32,
                                        I32, I32, I32, I32, F32, P, P, SZ, P]
        L.rtp_scan_local.argtypes = [P, P, P, I32, I32, I64, I32, P, P, P, I32, I32, I32, I32,
                                     I64, I32, I32, I32, I32, I32, F32, P, P, SZ, P]
        L.rtp_workspace_size.argtypes = [I32, I32, I32, I32, ctypes.POINTER(SZ)]
        L.rtp_status_string.argtypes = [I32]
        L.rtp_status_string.restype = ctypes.c_char_p
        L.rtp_last_hip_error.argtypes = []
        L.rtp_last_hip_error.restype = I32
        for name in SYMBOLS[:15]:
            getattr(L, name).restype = I32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().rtp_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise RtpError(status, where)


def workspace_size(which: int, B: int, H: int, N: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().rtp_workspace_size(which, B, H, N, ctypes.byref(out)), "rtp_workspace_size")
    return out.value


# ------------------------------------------------------------ torch glue

def _stream(t, stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, dtype, name, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _bf16(t, name, ndim):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return _dev(t, torch.int16, name, ndim)


def rtp_index_scores(q_r, k_r, scores, stream=None) -> None:
    """q_r f32 [B][Hq_r][16]; k_r f32 [B][Hkv_r][cap][16];
    scores f32 [B][Hq_r][N] (out)."""
    import torch
    B, Hq_r, r = q_r.shape
    _, Hkv_r, cap, _ = k_r.shape
    N = scores.shape[-1]
    _check(lib().rtp_index_scores(
        _dev(q_r, torch.float32, "q_r", 3), _dev(k_r, torch.float32, "k_r", 4),
        _dev(scores, torch.float32, "scores", 3), B, Hq_r, Hkv_r, N, cap, r,
        _stream(q_r, stream)), "rtp_index_scores")


def rtp_index_scores_bf16(q_r, k_r, scores, stream=None) -> None:
    """rtp_index_scores over a bf16 k_r cache: k_r bf16 [B][Hkv_r][cap][16]
    (torch.bfloat16 or its int16 bit patterns)."""
    import torch
    B, Hq_r, r = q_r.shape
    _, Hkv_r, cap, _ = k_r.shape
    N = scores.shape[-1]
    _check(lib().rtp_index_scores_bf16(
        _dev(q_r, torch.float32, "q_r", 3), _bf16(k_r, "k_r", 4),
        _dev(scores, torch.float32, "scores", 3), B, Hq_r, Hkv_r, N, cap, r,
        _stream(q_r, stream)), "rtp_index_scores_bf16")


def keep_words(N: int) -> int:
    """32-bit words per row of a keep bitmap over N tokens."""
    return (N + 31) // 32


def rtp_topp_select(scores, p, idx, count, workspace, keep_bits=None, stream=None) -> None:
    """scores f32 [B][H][N]; idx i32 [B][H][N] (out); count i32 [B][H] (out);
    keep_bits i32 [B][H][keep_words(N)] (optional out, the same sets as
    bitmaps); workspace uint8 [>= workspace_size(RTP_WS_TOPP_SELECT, B, H, N)]."""
    import torch
    B, H, N = scores.shape
    kb = None
    if keep_bits is not None:
        if tuple(keep_bits.shape) != (B, H, keep_words(N)):
            raise ValueError(f"keep_bits must have shape {(B, H, keep_words(N))}")
        kb = _dev(keep_bits, torch.int32, "keep_bits", 3)
    _check(lib().rtp_topp_select(
        _dev(scores, torch.float32, "scores", 3), B, H, N, float(p),
        _dev(idx, torch.int32, "idx", 3), _dev(count, torch.int32, "count", 2), kb,
        _dev(workspace, torch.uint8, "workspace", 1), workspace.numel(),
        _stream(scores, stream)), "rtp_topp_select")


def rtp_index_project(x, W, out, head_begin=0, T=None, out_pos=0, stream=None) -> None:
    """x bf16 [B][Hx][x_cap][128]; W bf16 [H][16][128] (one projector per
    head); out f32 [B][H][out_cap][16]: rows [out_pos, out_pos + T) of out
    get W[h] x for x rows [0, T) of heads [head_begin, head_begin + H)
    (T defaults to x_cap)."""
    import torch
    if x.dim() != 4 or W.dim() != 3 or out.dim() != 4:
        raise ValueError("x and out must be 4-D, W 3-D")
    B, Hx, x_cap, d = x.shape
    H, r, dw = W.shape
    if dw != d or tuple(out.shape[:2]) != (B, H) or out.shape[3] != r:
        raise ValueError("x, W and out disagree in shape")
    T = x_cap if T is None else T
    _check(lib().rtp_index_project(
        _bf16(x, "x", 4), B, Hx, x_cap, head_begin, H, T, d,
        _bf16(W, "W", 3), r, _dev(out, torch.float32, "out", 4), out.shape[2],
        out_pos, _stream(x, stream)), "rtp_index_project")


def rtp_topk_select(scores, k, idx, count, workspace, keep_bits=None, stream=None) -> None:
    """Static top-k: the first min(k, N) tokens of each row by (score
    descending, index ascending).  Arguments as in rtp_topp_select, with the
    integer budget k >= 1 in place of p."""
    import torch
    B, H, N = scores.shape
    kb = None
    if keep_bits is not None:
        if tuple(keep_bits.shape) != (B, H, keep_words(N)):
            raise ValueError(f"keep_bits must have shape {(B, H, keep_words(N))}")
        kb = _dev(keep_bits, torch.int32, "keep_bits", 3)
    _check(lib().rtp_topk_select(
        _dev(scores, torch.float32, "scores", 3), B, H, N, int(k),
        _dev(idx, torch.int32, "idx", 3), _dev(count, torch.int32, "count", 2), kb,
        _dev(workspace, torch.uint8, "workspace", 1), workspace.numel(),
        _stream(scores, stream)), "rtp_topk_select")


def rtp_keep_bits_add_local(keep_bits, N, n_sink, window, stream=None) -> None:
    """Sets the sink and window bits of every row of keep_bits
    (i32 [B][H][keep_words(N)])."""
    import torch
    B, H, nw = keep_bits.shape
    if nw != keep_words(N):
        raise ValueError(f"keep_bits must have {keep_words(N)} words per row")
    _check(lib().rtp_keep_bits_add_local(_dev(keep_bits, torch.int32, "keep_bits", 3), B, H, N,
                                         n_sink, window, _stream(keep_bits, stream)),
           "rtp_keep_bits_add_local")


def rtp_topp_hist(scores, workspace, stream=None) -> None:
    """The histogram pass of rtp_topp_select alone (no output written)."""
    import torch
    B, H, N = scores.shape
    _check(lib().rtp_topp_hist(
        _dev(scores, torch.float32, "scores", 3), B, H, N,
        _dev(workspace, torch.uint8, "workspace", 1), workspace.numel(),
        _stream(scores, stream)), "rtp_topp_hist")


def rtp_sparse_decode(q, K, V, idx, count, q_head_begin, scale, out, workspace,
                      N=None, stream=None) -> None:
    """q bf16 [B][Hq][d]; K, V bf16 [B][Hkv][cap][d]; idx i32 [B][n_q][N];
    count i32 [B][n_q]; out f32 [B][Hq][d] (heads in range written)."""
    import torch
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    n_q = count.shape[1]
    N = idx.shape[-1] if N is None else N
    _check(lib().rtp_sparse_decode(
        _bf16(q, "q", 3), _bf16(K, "K", 4), _bf16(V, "V", 4),
        _dev(idx, torch.int32, "idx", 3), _dev(count, torch.int32, "count", 2),
        B, Hq, Hkv, N, cap, d, q_head_begin, n_q, float(scale),
        _dev(out, torch.float32, "out", 3), _dev(workspace, torch.uint8, "workspace", 1),
        workspace.numel(), _stream(q, stream)), "rtp_sparse_decode")


def rtp_sparse_decode_union(q, K, V, keep_bits, N, q_head_begin, scale, out, workspace,
                            stream=None) -> None:
    """q bf16 [B][Hq][d]; K, V bf16 [B][Hkv][cap][d]; keep_bits i32
    [B][n_q][keep_words(N)] as written by rtp_topp_select; out f32 [B][Hq][d]."""
    import torch
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    n_q = keep_bits.shape[1]
    if tuple(keep_bits.shape) != (B, n_q, keep_words(N)):
        raise ValueError(f"keep_bits must have shape {(B, n_q, keep_words(N))}")
    _check(lib().rtp_sparse_decode_union(
        _bf16(q, "q", 3), _bf16(K, "K", 4), _bf16(V, "V", 4),
        _dev(keep_bits, torch.int32, "keep_bits", 3), B, Hq, Hkv, N, cap, d, q_head_begin, n_q,
        float(scale), _dev(out, torch.float32, "out", 3),
        _dev(workspace, torch.uint8, "workspace", 1), workspace.numel(), _stream(q, stream)),
        "rtp_sparse_decode_union")


def rtp_decode_attend(q, K, V, idx, count, N, sparse_head_begin, local_head_begin,
                      n_local_heads, n_sink, window, scale, out, workspace,
                      stream=None) -> None:
    """rtp_sparse_decode for the heads [sparse_head_begin, + count.shape[1])
    and rtp_local_decode for [local_head_begin, + n_local_heads), one launch.
    idx/count may be None (no sparse heads); workspace uint8
    [>= workspace_size(RTP_WS_DECODE_ATTEND, B, Hq, N)]."""
    import torch
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    n_sparse = 0 if count is None else count.shape[1]
    idx_p = None if idx is None else _dev(idx, torch.int32, "idx", 3)
    count_p = None if count is None else _dev(count, torch.int32, "count", 2)
    _check(lib().rtp_decode_attend(
        _bf16(q, "q", 3), _bf16(K, "K", 4), _bf16(V, "V", 4), idx_p, count_p,
        B, Hq, Hkv, N, cap, d, sparse_head_begin, n_sparse, local_head_begin, n_local_heads,
        n_sink, window, float(scale), _dev(out, torch.float32, "out", 3),
        _dev(workspace, torch.uint8, "workspace", 1), workspace.numel(), _stream(q, stream)),
        "rtp_decode_attend")


def rtp_scan_local(q_r, k_r, scores, q, K, V, N, local_head_begin, n_local_heads, n_sink,
                   window, scale, out, workspace, stream=None) -> None:
    """rtp_index_scores(q_r, k_r, scores) and rtp_local_decode for the heads
    [local_head_begin, + n_local_heads), one launch; scores f32 [B][Hq_r][N];
    workspace uint8 [>= workspace_size(RTP_WS_LOCAL_DECODE, B, n_local_heads, N)]."""
    import torch
    B, Hq_r, r = q_r.shape
    _, Hkv_r, kr_cap, _ = k_r.shape
    _, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    if tuple(scores.shape) != (B, Hq_r, N) or q.shape[0] != B:
        raise ValueError(f"scores must be [B][Hq_r][N] = {(B, Hq_r, N)} and q [B][Hq][d], "
                         f"got {tuple(scores.shape)} and {tuple(q.shape)}")
    _check(lib().rtp_scan_local(
        _dev(q_r, torch.float32, "q_r", 3), _dev(k_r, torch.float32, "k_r", 4),
        _dev(scores, torch.float32, "scores", 3), Hq_r, Hkv_r, kr_cap, r,
        _bf16(q, "q", 3), _bf16(K, "K", 4), _bf16(V, "V", 4), B, Hq, Hkv, N, cap, d,
        local_head_begin, n_local_heads, n_sink, window, float(scale),
        _dev(out, torch.float32, "out", 3), _dev(workspace, torch.uint8, "workspace", 1),
        workspace.numel(), _stream(q, stream)), "rtp_scan_local")


def rtp_prefill_attend(q, K, V, head_begin, n_heads, n_sink, window, scale, out,
                       stream=None) -> None:
    """q bf16 [B][Hq][T][128]; K, V bf16 [B][Hkv][cap][128]; out f32
    [B][Hq][T][128]: causal prefill for heads [head_begin, + n_heads), dense
    (window <= 0) or sinks + window."""
    import torch
    B, Hq, T, d = q.shape
    _, Hkv, cap, _ = K.shape
    _check(lib().rtp_prefill_attend(
        _bf16(q, "q", 4), _bf16(K, "K", 4), _bf16(V, "V", 4), B, Hq, Hkv, T, cap, d,
        head_begin, n_heads, n_sink, window, float(scale), _dev(out, torch.float32, "out", 4),
        _stream(q, stream)), "rtp_prefill_attend")


def rtp_local_decode_ring(q, K, V, N, q_head_begin, n_q_heads, n_sink, window, scale, out,
                          workspace, stream=None) -> None:
    """rtp_local_decode over ring-buffer caches of n_sink + window slots (token
    i >= n_sink in slot n_sink + (i - n_sink) % window); N tokens seen."""
    import torch
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    _check(lib().rtp_local_decode_ring(
        _bf16(q, "q", 3), _bf16(K, "K", 4), _bf16(V, "V", 4), B, Hq, Hkv, N, cap, d,
        q_head_begin, n_q_heads, n_sink, window, float(scale),
        _dev(out, torch.float32, "out", 3), _dev(workspace, torch.uint8, "workspace", 1),
        workspace.numel(), _stream(q, stream)), "rtp_local_decode_ring")


def rtp_local_decode(q, K, V, N, q_head_begin, n_q_heads, n_sink, window, scale, out,
                     workspace, stream=None) -> None:
    """Local heads [q_head_begin, q_head_begin + n_q_heads): sinks + window."""
    import torch
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    _check(lib().rtp_local_decode(
        _bf16(q, "q", 3), _bf16(K, "K", 4), _bf16(V, "V", 4), B, Hq, Hkv, N, cap, d,
        q_head_begin, n_q_heads, n_sink, window, float(scale),
        _dev(out, torch.float32, "out", 3), _dev(workspace, torch.uint8, "workspace", 1),
        workspace.numel(), _stream(q, stream)), "rtp_local_decode")
