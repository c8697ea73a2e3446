"""One decode step of one attention layer through the four C-ABI calls.

Query heads [0, H_r) are retrieval heads (indexer scan, top-p select, sparse
attention); heads [H_r, Hq) are local heads (sinks + sliding window), as in
the head-role split of the gist.science summary of arXiv 2605.16928, method
section 1.  Buffers that one layer uses and the next reuses (scores, kept
indices, workspaces) are allocated once here.
"""
from __future__ import annotations

import torch

from . import (RTP_WS_DECODE_ATTEND, RTP_WS_LOCAL_DECODE, RTP_WS_SPARSE_DECODE,
               RTP_WS_SPARSE_UNION, RTP_WS_TOPP_SELECT, decode_layer_workspace_size, keep_words,
               rtp_decode_attend, rtp_decode_layer, rtp_index_scores, rtp_index_scores_bf16,
               rtp_local_decode, rtp_scan_local, rtp_sparse_decode, rtp_sparse_decode_union,
               rtp_topp_attend, rtp_topp_select, topp_attend_workspace_size, workspace_size)


class DecodeLayer:
    """mode "fused": the scan, the selection, then one rtp_decode_attend
    launch for the sparse heads (per-head index lists) and the local heads
    together; mode "scan_local": one rtp_scan_local launch runs the indexer
    scan and the local heads, then the selection, then rtp_decode_attend for
    the sparse heads alone; mode "per_head": rtp_sparse_decode and rtp_local_decode
    as separate calls; mode "union": the selector also writes keep bitmaps
    and the sparse heads run rtp_sparse_decode_union (each kept row read once
    per KV head); mode "layer": the whole layer in one rtp_decode_layer launch
    (scores kept on chip; with keep_scores they are also written out, for
    checking); mode "topp_attend": the scan, then one rtp_topp_attend launch
    for the selection and every head's attention."""

    def __init__(self, B: int, Hq: int, Hkv: int, N: int, H_r: int, n_sink: int,
                 window: int, device, d: int = 128, mode: str = "fused",
                 keep_scores: bool = True):
        if mode not in ("fused", "scan_local", "union", "per_head", "layer", "topp_attend"):
            raise ValueError(f"unknown mode {mode!r}")
        self.keep_scores = keep_scores
        self.B, self.Hq, self.Hkv, self.N, self.H_r = B, Hq, Hkv, N, H_r
        self.n_sink, self.window, self.d, self.mode = n_sink, window, d, mode
        self.H_l = Hq - H_r
        dev = torch.device(device)
        self.keep_bits = None
        if mode == "layer":
            if H_r < 1:
                raise ValueError("mode 'layer' needs retrieval heads")
            self.scores = (torch.empty((B, H_r, N), dtype=torch.float32, device=dev)
                           if keep_scores else None)
            self.idx = torch.empty((B, H_r, N), dtype=torch.int32, device=dev)
            self.count = torch.empty((B, H_r), dtype=torch.int32, device=dev)
            self.ws_layer = torch.empty(
                decode_layer_workspace_size(B, Hq, Hkv, N, H_r, n_sink, window),
                dtype=torch.uint8, device=dev)
            return
        if mode == "topp_attend":
            if H_r < 1:
                raise ValueError("mode 'topp_attend' needs retrieval heads")
            self.scores = torch.empty((B, H_r, N), dtype=torch.float32, device=dev)
            self.idx = torch.empty((B, H_r, N), dtype=torch.int32, device=dev)
            self.count = torch.empty((B, H_r), dtype=torch.int32, device=dev)
            self.ws_ta = torch.empty(
                topp_attend_workspace_size(B, Hq, Hkv, N, H_r, n_sink, window),
                dtype=torch.uint8, device=dev)
            return
        if H_r > 0:
            self.scores = torch.empty((B, H_r, N), dtype=torch.float32, device=dev)
            self.idx = torch.empty((B, H_r, N), dtype=torch.int32, device=dev)
            self.count = torch.empty((B, H_r), dtype=torch.int32, device=dev)
            self.ws_sel = torch.empty(workspace_size(RTP_WS_TOPP_SELECT, B, H_r, N),
                                      dtype=torch.uint8, device=dev)
            if mode == "union":
                self.keep_bits = torch.empty((B, H_r, keep_words(N)), dtype=torch.int32,
                                             device=dev)
                self.ws_sparse = torch.empty(workspace_size(RTP_WS_SPARSE_UNION, B, H_r, N),
                                             dtype=torch.uint8, device=dev)
            else:
                self.ws_sparse = torch.empty(workspace_size(RTP_WS_SPARSE_DECODE, B, H_r, N),
                                             dtype=torch.uint8, device=dev)
            if mode in ("fused", "scan_local"):
                self.ws_attend = torch.empty(workspace_size(RTP_WS_DECODE_ATTEND, B, Hq, N),
                                             dtype=torch.uint8, device=dev)
        if self.H_l > 0:
            self.ws_local = torch.empty(workspace_size(RTP_WS_LOCAL_DECODE, B, self.H_l, N),
                                        dtype=torch.uint8, device=dev)

    def scan(self, q_r, k_r, stream=None):
        """The indexer scan; a bf16 k_r cache (torch.bfloat16 or its int16
        bit patterns) takes rtp_index_scores_bf16."""
        import torch
        if k_r.dtype in (torch.bfloat16, torch.int16):
            rtp_index_scores_bf16(q_r, k_r, self.scores, stream=stream)
        else:
            rtp_index_scores(q_r, k_r, self.scores, stream=stream)

    def retrieval(self, q_r, k_r, q, K, V, p: float, scale: float, out, stream=None):
        self.scan(q_r, k_r, stream=stream)
        rtp_topp_select(self.scores, p, self.idx, self.count, self.ws_sel,
                        keep_bits=self.keep_bits, stream=stream)
        if self.mode == "union":
            rtp_sparse_decode_union(q, K, V, self.keep_bits, self.N, 0, scale, out,
                                    self.ws_sparse, stream=stream)
        else:
            rtp_sparse_decode(q, K, V, self.idx, self.count, 0, scale, out, self.ws_sparse,
                              stream=stream)

    def local(self, q, K, V, scale: float, out, stream=None):
        rtp_local_decode(q, K, V, self.N, self.H_r, self.H_l, self.n_sink, self.window,
                         scale, out, self.ws_local, stream=stream)

    def attend(self, q, K, V, scale: float, out, stream=None):
        """Sparse and local heads in one launch (mode "fused")."""
        rtp_decode_attend(q, K, V, self.idx, self.count, self.N, 0, self.H_r, self.H_l,
                          self.n_sink, self.window, scale, out, self.ws_attend, stream=stream)

    def __call__(self, q_r, k_r, q, K, V, p: float, scale: float, out, side_stream=None):
        """Runs the layer on the current stream.  In modes "fused" and
        "scan_local" the local heads share a launch with the sparse heads or
        with the scan, and side_stream is not used.  Otherwise, with
        side_stream, the local heads run there concurrently with the
        retrieval chain (the two share no buffer); the current stream waits
        for them before returning."""
        if self.mode == "layer":
            if k_r.dtype != torch.float32:
                raise ValueError("mode 'layer' takes an fp32 indexer key cache")
            rtp_decode_layer(q_r, k_r, q, K, V, self.N, self.H_r, self.n_sink, self.window, p,
                             scale, out, self.idx, self.count, self.ws_layer,
                             scores=self.scores)
            return
        if self.mode == "topp_attend":
            self.scan(q_r, k_r)
            rtp_topp_attend(self.scores, q, K, V, self.n_sink, self.window, p, scale, out,
                            self.idx, self.count, self.ws_ta)
            return
        if self.mode == "scan_local" and self.H_r > 0 and self.H_l > 0:
            if k_r.dtype != torch.float32:
                raise ValueError("mode 'scan_local' takes an fp32 indexer key cache "
                                 "(rtp_scan_local has no bf16 key path)")
            rtp_scan_local(q_r, k_r, self.scores, q, K, V, self.N, self.H_r, self.H_l,
                           self.n_sink, self.window, scale, out, self.ws_local)
            rtp_topp_select(self.scores, p, self.idx, self.count, self.ws_sel)
            rtp_decode_attend(q, K, V, self.idx, self.count, self.N, 0, self.H_r, 0, 0, 1,
                              scale, out, self.ws_attend)
            return
        if self.mode == "fused" and self.H_r > 0 and self.H_l > 0:
            self.scan(q_r, k_r)
            rtp_topp_select(self.scores, p, self.idx, self.count, self.ws_sel)
            self.attend(q, K, V, scale, out)
            return
        if side_stream is not None and self.H_r > 0 and self.H_l > 0:
            main = torch.cuda.current_stream(out.device)
            side_stream.wait_stream(main)
            with torch.cuda.stream(side_stream):
                self.local(q, K, V, scale, out)
            self.retrieval(q_r, k_r, q, K, V, p, scale, out)
            main.wait_stream(side_stream)
            return
        if self.H_r > 0:
            self.retrieval(q_r, k_r, q, K, V, p, scale, out)
        if self.H_l > 0:
            self.local(q, K, V, scale, out)
