"""Python binding of librtp (include/rtp.h): the RTPurbo sparse decode path
on MI355X (arXiv 2605.16928).

Argument marshalling only: each function checks the dtype, device and
full shape of every torch tensor it is given against the sizes the C call
will read (a mismatch raises ValueError or TypeError before anything is
launched, since the C ABI receives no tensor sizes), reads their device
pointers and the current HIP stream, and calls the C function of the same
name.  Every step of the path
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
          4: "RTP_ERR_VALUE", 5: "RTP_ERR_ALIGN", 6: "RTP_ERR_WORKSPACE", 7: "RTP_ERR_HIP",
          8: "RTP_ERR_LIMIT"}

# Every symbol include/rtp.h declares.
SYMBOLS = ("rtp_index_scores", "rtp_index_scores_bf16", "rtp_index_project", "rtp_topp_select",
           "rtp_topk_select", "rtp_topp_hist", "rtp_sparse_decode", "rtp_sparse_decode_noalloc",
           "rtp_sparse_decode_union",
           "rtp_local_decode", "rtp_local_decode_ring", "rtp_keep_bits_add_local",
           "rtp_prefill_attend", "rtp_decode_attend", "rtp_scan_local", "rtp_decode_layer",
           "rtp_decode_layer_workspace_size", "rtp_topp_attend", "rtp_topp_attend_workspace_size",
           "rtp_set_wait_limit", "rtp_device_status",
           "rtp_workspace_size", "rtp_status_string", "rtp_last_hip_error")

# Bit of the device status word (rtp_device_status): a bounded wait gave up.
RTP_STATUS_WAIT_TIMEOUT = 1


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
        L.rtp_sparse_decode_noalloc.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I64, I32,
                                                I32, I32, F32, P, P]
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
        L.rtp_decode_layer.argtypes = [P, P, I64, P, P, P, I64, I32, I32, I32, I32, I32, I32,
                                       I32, I32, I32, F32, F32, P, P, P, P, P, SZ, P]
        L.rtp_decode_layer_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32,
                                                      ctypes.POINTER(SZ)]
        L.rtp_topp_attend.argtypes = [P, P, P, P, I32, I32, I32, I32, I64, I32, I32, I32,
                                      I32, F32, F32, P, P, P, P, SZ, P]
        L.rtp_topp_attend_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32,
                                                     ctypes.POINTER(SZ)]
        L.rtp_set_wait_limit.argtypes = [ctypes.c_uint32]
        L.rtp_device_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), I32]
        L.rtp_workspace_size.argtypes = [I32, I32, I32, I32, ctypes.POINTER(SZ)]
        L.rtp_status_string.argtypes = [I32]
        L.rtp_status_string.restype = ctypes.c_char_p
        L.rtp_last_hip_error.argtypes = []
        L.rtp_last_hip_error.restype = I32
        for name in SYMBOLS[:-2]:
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
    _call("rtp_workspace_size", which, B, H, N, ctypes.byref(out))
    return out.value


def decode_layer_workspace_size(B: int, Hq: int, Hkv: int, N: int, Hq_r: int, n_sink: int,
                                window: int) -> int:
    """Workspace bytes of rtp_decode_layer on the current device."""
    out = ctypes.c_size_t(0)
    _call("rtp_decode_layer_workspace_size", B, Hq, Hkv, N, Hq_r, n_sink, window,
                                                 ctypes.byref(out))
    return out.value


def topp_attend_workspace_size(B: int, Hq: int, Hkv: int, N: int, Hq_r: int, n_sink: int,
                               window: int) -> int:
    """Workspace bytes of rtp_topp_attend on the current device."""
    out = ctypes.c_size_t(0)
    _call("rtp_topp_attend_workspace_size", B, Hq, Hkv, N, Hq_r, n_sink, window,
          ctypes.byref(out))
    return out.value


def set_wait_limit(polls: int) -> None:
    """Poll limit of the kernels' waits on other blocks, for later launches."""
    _call("rtp_set_wait_limit", int(polls))


def device_status(clear: bool = False) -> int:
    """The current device's sticky status word (waits for the device)."""
    v = ctypes.c_uint32(0)
    _call("rtp_device_status", ctypes.byref(v), 1 if clear else 0)
    return v.value


# ------------------------------------------------------------ torch glue

def _stream(t, stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, dtype, name, shape):
    """Device pointer of a contiguous device tensor of this dtype; `shape` is
    the expected shape (an int for the number of dims alone, or a tuple
    whose None entries match any size)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    ndim = shape if isinstance(shape, int) else len(shape)
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not isinstance(shape, int):
        for got, want in zip(t.shape, shape):
            if want is not None and got != want:
                raise ValueError(f"{name} must have shape "
                                 f"{tuple('*' if w is None else w for w in shape)}, "
                                 f"got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        return _OffDevice(name)  # reported by _call, once every shape is checked
    return t.data_ptr()


class _OffDevice:
    def __init__(self, name):
        self.name = name


def _call(name, *args):
    """Calls C function `name` once no argument is a host tensor."""
    for a in args:
        if isinstance(a, _OffDevice):
            raise ValueError(f"{a.name} must be a device tensor")
    _check(getattr(lib(), name)(*args), name)


def _bf16(t, name, shape):
    import torch
    if isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return _dev(t, torch.int16, name, shape)


def _ws(workspace):
    import torch
    return _dev(workspace, torch.uint8, "workspace", 1), workspace.numel()


def _qkv(q, K, V, out):
    """q bf16 [B][Hq][d], K and V bf16 [B][Hkv][cap][d], out f32 [B][Hq][d]:
    checked and marshalled; returns the pointers and (B, Hq, Hkv, cap, d)."""
    import torch
    if q.dim() != 3 or K.dim() != 4:
        raise ValueError("q must be [B][Hq][d] and K [B][Hkv][cap][d]")
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    ptrs = (_bf16(q, "q", (B, Hq, d)), _bf16(K, "K", (B, Hkv, cap, d)),
            _bf16(V, "V", (B, Hkv, cap, d)), _dev(out, torch.float32, "out", (B, Hq, d)))
    return ptrs, (B, Hq, Hkv, cap, d)


def rtp_index_scores(q_r, k_r, scores, stream=None) -> None:
    """q_r f32 [B][Hq_r][16]; k_r f32 [B][Hkv_r][cap][16];
    scores f32 [B][Hq_r][N] (out)."""
    import torch
    if q_r.dim() != 3 or k_r.dim() != 4 or scores.dim() != 3:
        raise ValueError("q_r must be 3-D, k_r 4-D, scores 3-D")
    B, Hq_r, r = q_r.shape
    Hkv_r, cap = k_r.shape[1], k_r.shape[2]
    N = scores.shape[-1]
    _call("rtp_index_scores", 
        _dev(q_r, torch.float32, "q_r", (B, Hq_r, r)),
        _dev(k_r, torch.float32, "k_r", (B, Hkv_r, cap, r)),
        _dev(scores, torch.float32, "scores", (B, Hq_r, N)), B, Hq_r, Hkv_r, N, cap, r,
        _stream(q_r, stream))


def rtp_index_scores_bf16(q_r, k_r, scores, stream=None) -> None:
    """rtp_index_scores over a bf16 k_r cache: k_r bf16 [B][Hkv_r][cap][16]
    (torch.bfloat16 or its int16 bit patterns)."""
    import torch
    if q_r.dim() != 3 or k_r.dim() != 4 or scores.dim() != 3:
        raise ValueError("q_r must be 3-D, k_r 4-D, scores 3-D")
    B, Hq_r, r = q_r.shape
    Hkv_r, cap = k_r.shape[1], k_r.shape[2]
    N = scores.shape[-1]
    _call("rtp_index_scores_bf16", 
        _dev(q_r, torch.float32, "q_r", (B, Hq_r, r)), _bf16(k_r, "k_r", (B, Hkv_r, cap, r)),
        _dev(scores, torch.float32, "scores", (B, Hq_r, N)), B, Hq_r, Hkv_r, N, cap, r,
        _stream(q_r, stream))


def keep_words(N: int) -> int:
    """32-bit words per row of a keep bitmap over N tokens."""
    return (N + 31) // 32


def _select_outs(scores, idx, count, keep_bits):
    import torch
    if scores.dim() != 3:
        raise ValueError("scores must be [B][H][N]")
    B, H, N = scores.shape
    kb = None
    if keep_bits is not None:
        kb = _dev(keep_bits, torch.int32, "keep_bits", (B, H, keep_words(N)))
    return (B, H, N), (_dev(scores, torch.float32, "scores", (B, H, N)),
                       _dev(idx, torch.int32, "idx", (B, H, N)),
                       _dev(count, torch.int32, "count", (B, H)), kb)


def rtp_topp_select(scores, p, idx, count, workspace, keep_bits=None, stream=None) -> None:
    """scores f32 [B][H][N]; idx i32 [B][H][N] (out); count i32 [B][H] (out);
    keep_bits i32 [B][H][keep_words(N)] (optional out, the same sets as
    bitmaps); workspace uint8 [>= workspace_size(RTP_WS_TOPP_SELECT, B, H, N)]."""
    (B, H, N), (sp, ip, cp, kb) = _select_outs(scores, idx, count, keep_bits)
    wp, wn = _ws(workspace)
    _call("rtp_topp_select", sp, B, H, N, float(p), ip, cp, kb, wp, wn,
                                 _stream(scores, stream))


def rtp_topk_select(scores, k, idx, count, workspace, keep_bits=None, stream=None) -> None:
    """Static top-k: the first min(k, N) tokens of each row by (score
    descending, index ascending).  Arguments as in rtp_topp_select, with the
    integer budget k >= 1 in place of p."""
    (B, H, N), (sp, ip, cp, kb) = _select_outs(scores, idx, count, keep_bits)
    wp, wn = _ws(workspace)
    _call("rtp_topk_select", sp, B, H, N, int(k), ip, cp, kb, wp, wn,
                                 _stream(scores, stream))


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
    _call("rtp_index_project", 
        _bf16(x, "x", (B, Hx, x_cap, d)), B, Hx, x_cap, head_begin, H, T, d,
        _bf16(W, "W", (H, r, d)), r, _dev(out, torch.float32, "out", (B, H, None, r)),
        out.shape[2], out_pos, _stream(x, stream))


def rtp_keep_bits_add_local(keep_bits, N, n_sink, window, stream=None) -> None:
    """Sets the sink and window bits of every row of keep_bits
    (i32 [B][H][keep_words(N)])."""
    import torch
    if keep_bits.dim() != 3:
        raise ValueError("keep_bits must be [B][H][keep_words(N)]")
    B, H, _ = keep_bits.shape
    _call("rtp_keep_bits_add_local", 
        _dev(keep_bits, torch.int32, "keep_bits", (B, H, keep_words(N))), B, H, N, n_sink,
        window, _stream(keep_bits, stream))


def rtp_topp_hist(scores, workspace, stream=None) -> None:
    """The histogram pass of rtp_topp_select alone (no output written)."""
    import torch
    if scores.dim() != 3:
        raise ValueError("scores must be [B][H][N]")
    B, H, N = scores.shape
    wp, wn = _ws(workspace)
    _call("rtp_topp_hist", _dev(scores, torch.float32, "scores", (B, H, N)), B, H, N, wp,
                               wn, _stream(scores, stream))


def rtp_sparse_decode(q, K, V, idx, count, q_head_begin, scale, out, workspace,
                      N=None, stream=None) -> None:
    """q bf16 [B][Hq][d]; K, V bf16 [B][Hkv][cap][d]; idx i32 [B][n_q][N];
    count i32 [B][n_q]; out f32 [B][Hq][d] (heads in range written)."""
    import torch
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    if count.dim() != 2 or idx.dim() != 3:
        raise ValueError("count must be [B][n_q] and idx [B][n_q][N]")
    n_q = count.shape[1]
    N = idx.shape[-1] if N is None else N
    wp, wn = _ws(workspace)
    _call("rtp_sparse_decode", 
        qp, Kp, Vp, _dev(idx, torch.int32, "idx", (B, n_q, N)),
        _dev(count, torch.int32, "count", (B, n_q)), B, Hq, Hkv, N, cap, d, q_head_begin, n_q,
        float(scale), op, wp, wn, _stream(q, stream))


def rtp_sparse_decode_noalloc(q, K, V, idx, count, q_head_begin, scale, out, N=None,
                              stream=None) -> None:
    """rtp_sparse_decode with the library's static scratch in place of a
    workspace (no device allocation); arguments as rtp_sparse_decode's."""
    import torch
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    if count.dim() != 2 or idx.dim() != 3:
        raise ValueError("count must be [B][n_q] and idx [B][n_q][N]")
    n_q = count.shape[1]
    N = idx.shape[-1] if N is None else N
    _call("rtp_sparse_decode_noalloc", qp, Kp, Vp, _dev(idx, torch.int32, "idx", (B, n_q, N)),
          _dev(count, torch.int32, "count", (B, n_q)), B, Hq, Hkv, N, cap, d, q_head_begin,
          n_q, float(scale), op, _stream(q, stream))


def rtp_sparse_decode_union(q, K, V, keep_bits, N, q_head_begin, scale, out, workspace,
                            stream=None) -> None:
    """q bf16 [B][Hq][d]; K, V bf16 [B][Hkv][cap][d]; keep_bits i32
    [B][n_q][keep_words(N)] as written by rtp_topp_select; out f32 [B][Hq][d]."""
    import torch
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    if keep_bits.dim() != 3:
        raise ValueError("keep_bits must be [B][n_q][keep_words(N)]")
    n_q = keep_bits.shape[1]
    wp, wn = _ws(workspace)
    _call("rtp_sparse_decode_union", 
        qp, Kp, Vp, _dev(keep_bits, torch.int32, "keep_bits", (B, n_q, keep_words(N))), B, Hq,
        Hkv, N, cap, d, q_head_begin, n_q, float(scale), op, wp, wn, _stream(q, stream))


def rtp_decode_attend(q, K, V, idx, count, N, sparse_head_begin, local_head_begin,
                      n_local_heads, n_sink, window, scale, out, workspace,
                      stream=None) -> None:
    """rtp_sparse_decode for the heads [sparse_head_begin, + count.shape[1])
    and rtp_local_decode for [local_head_begin, + n_local_heads), one launch.
    idx/count may be None (no sparse heads); workspace uint8
    [>= workspace_size(RTP_WS_DECODE_ATTEND, B, Hq, N)]."""
    import torch
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    n_sparse = 0 if count is None else count.shape[1]
    idx_p = count_p = None
    if n_sparse:
        if count.dim() != 2:
            raise ValueError("count must be [B][n_sparse]")
        idx_p = _dev(idx, torch.int32, "idx", (B, n_sparse, N))
        count_p = _dev(count, torch.int32, "count", (B, n_sparse))
    wp, wn = _ws(workspace)
    _call("rtp_decode_attend", 
        qp, Kp, Vp, idx_p, count_p, B, Hq, Hkv, N, cap, d, sparse_head_begin, n_sparse,
        local_head_begin, n_local_heads, n_sink, window, float(scale), op, wp, wn,
        _stream(q, stream))


def rtp_scan_local(q_r, k_r, scores, q, K, V, N, local_head_begin, n_local_heads, n_sink,
                   window, scale, out, workspace, stream=None) -> None:
    """rtp_index_scores(q_r, k_r, scores) and rtp_local_decode for the heads
    [local_head_begin, + n_local_heads), one launch; scores f32 [B][Hq_r][N];
    workspace uint8 [>= workspace_size(RTP_WS_LOCAL_DECODE, B, n_local_heads, N)]."""
    import torch
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    if q_r.dim() != 3 or k_r.dim() != 4:
        raise ValueError("q_r must be [B][Hq_r][16] and k_r [B][Hkv_r][cap][16]")
    Hq_r, r = q_r.shape[1], q_r.shape[2]
    Hkv_r, kr_cap = k_r.shape[1], k_r.shape[2]
    wp, wn = _ws(workspace)
    _call("rtp_scan_local", 
        _dev(q_r, torch.float32, "q_r", (B, Hq_r, r)),
        _dev(k_r, torch.float32, "k_r", (B, Hkv_r, kr_cap, r)),
        _dev(scores, torch.float32, "scores", (B, Hq_r, N)), Hq_r, Hkv_r, kr_cap, r,
        qp, Kp, Vp, B, Hq, Hkv, N, cap, d, local_head_begin, n_local_heads, n_sink, window,
        float(scale), op, wp, wn, _stream(q, stream))


def rtp_decode_layer(q_r, k_r, q, K, V, N, Hq_r, n_sink, window, p, scale, out, idx, count,
                     workspace, scores=None, stream=None) -> None:
    """One decode layer in one launch: query heads [0, Hq_r) are retrieval
    heads (scan, top-p select, sparse attention), [Hq_r, Hq) local heads
    (sinks + window).  q_r f32 [B][Hq_r][16]; k_r f32 [B][Hq_r/G][cap][16];
    q bf16 [B][Hq][d]; K, V bf16 [B][Hkv][cap][d]; out f32 [B][Hq][d];
    idx i32 [B][Hq_r][N] and count i32 [B][Hq_r] (out); scores f32
    [B][Hq_r][N] (optional out); workspace uint8
    [>= decode_layer_workspace_size(B, Hq, Hkv, N, Hq_r, n_sink, window)]."""
    import torch
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    if q_r.dim() != 3 or k_r.dim() != 4:
        raise ValueError("q_r must be [B][Hq_r][16] and k_r [B][Hkv_r][cap][16]")
    r = q_r.shape[2]
    G = Hq // Hkv
    if Hkv < 1 or Hq % Hkv or Hq_r % G:
        raise ValueError("Hq must be a multiple of Hkv and Hq_r of Hq / Hkv")
    kr_cap = k_r.shape[2]
    sp = None if scores is None else _dev(scores, torch.float32, "scores", (B, Hq_r, N))
    wp, wn = _ws(workspace)
    _call("rtp_decode_layer", 
        _dev(q_r, torch.float32, "q_r", (B, Hq_r, r)),
        _dev(k_r, torch.float32, "k_r", (B, Hq_r // G, kr_cap, r)), kr_cap, qp, Kp, Vp, cap,
        B, Hq, Hkv, N, d, r, Hq_r, n_sink, window, float(p), float(scale), op,
        _dev(idx, torch.int32, "idx", (B, Hq_r, N)), _dev(count, torch.int32, "count", (B, Hq_r)),
        sp, wp, wn, _stream(q, stream))


def _topp_attend(name, scores, q, K, V, n_sink, window, p, scale, out, idx, count, workspace,
                 stream):
    import torch
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    if scores.dim() != 3 or scores.shape[0] != B:
        raise ValueError("scores must be [B][Hq_r][N]")
    Hq_r, N = scores.shape[1], scores.shape[2]
    wp, wn = _ws(workspace)
    _call(name,
        _dev(scores, torch.float32, "scores", (B, Hq_r, N)), qp, Kp, Vp, B, Hq, Hkv, N, cap, d,
        Hq_r, n_sink, window, float(p), float(scale), op,
        _dev(idx, torch.int32, "idx", (B, Hq_r, N)), _dev(count, torch.int32, "count", (B, Hq_r)),
        wp, wn, _stream(q, stream))


def rtp_topp_attend(scores, q, K, V, n_sink, window, p, scale, out, idx, count, workspace,
                    stream=None) -> None:
    """Top-p selection over scores f32 [B][Hq_r][N] (query heads [0, Hq_r)
    are retrieval heads) and attention for every head in one launch: the
    retrieval heads over their kept rows, heads [Hq_r, Hq) over sinks +
    window.  q bf16 [B][Hq][d]; K, V bf16 [B][Hkv][cap][d]; out f32
    [B][Hq][d]; idx i32 [B][Hq_r][N] and count i32 [B][Hq_r] (out);
    workspace uint8 [>= topp_attend_workspace_size(B, Hq, Hkv, N, Hq_r,
    n_sink, window)]."""
    _topp_attend("rtp_topp_attend", scores, q, K, V, n_sink, window, p, scale, out, idx, count,
                 workspace, stream)


def rtp_prefill_attend(q, K, V, head_begin, n_heads, n_sink, window, scale, out,
                       stream=None) -> None:
    """q bf16 [B][Hq][T][128]; K, V bf16 [B][Hkv][cap][128]; out f32
    [B][Hq][T][128]: causal prefill for heads [head_begin, + n_heads), dense
    (window <= 0) or sinks + window."""
    import torch
    if q.dim() != 4 or K.dim() != 4:
        raise ValueError("q must be [B][Hq][T][d] and K [B][Hkv][cap][d]")
    B, Hq, T, d = q.shape
    _, Hkv, cap, _ = K.shape
    _call("rtp_prefill_attend", 
        _bf16(q, "q", (B, Hq, T, d)), _bf16(K, "K", (B, Hkv, cap, d)),
        _bf16(V, "V", (B, Hkv, cap, d)), B, Hq, Hkv, T, cap, d, head_begin, n_heads, n_sink,
        window, float(scale), _dev(out, torch.float32, "out", (B, Hq, T, d)),
        _stream(q, stream))


def rtp_local_decode_ring(q, K, V, N, q_head_begin, n_q_heads, n_sink, window, scale, out,
                          workspace, stream=None) -> None:
    """rtp_local_decode over ring-buffer caches of n_sink + window slots (token
    i >= n_sink in slot n_sink + (i - n_sink) % window); N tokens seen."""
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    wp, wn = _ws(workspace)
    _call("rtp_local_decode_ring", 
        qp, Kp, Vp, B, Hq, Hkv, N, cap, d, q_head_begin, n_q_heads, n_sink, window,
        float(scale), op, wp, wn, _stream(q, stream))


def rtp_local_decode(q, K, V, N, q_head_begin, n_q_heads, n_sink, window, scale, out,
                     workspace, stream=None) -> None:
    """Local heads [q_head_begin, q_head_begin + n_q_heads): sinks + window."""
    (qp, Kp, Vp, op), (B, Hq, Hkv, cap, d) = _qkv(q, K, V, out)
    wp, wn = _ws(workspace)
    _call("rtp_local_decode", 
        qp, Kp, Vp, B, Hq, Hkv, N, cap, d, q_head_begin, n_q_heads, n_sink, window,
        float(scale), op, wp, wn, _stream(q, stream))
