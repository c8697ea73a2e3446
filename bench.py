"""Decode-step benchmark of the RTPurbo sparse decode path on one MI355X.

One step = one decode step through a 48-layer attention stack at N = 2^20
cached tokens (batch 1, 32 query / 4 KV heads, d = 128, bf16 K/V ~ 96 GiB
resident): per layer, the indexer scan, top-p selection and sparse
attention for the 8 retrieval query heads of KV head 0, and sink + window
attention for the 24 local query heads.  Layers run in sequence.  The step is
captured once in a HIP graph and replayed.

Prints ONE JSON line (rank 0) with steps/s, the dominant kernel's roofline
and the CPU oracle's baseline on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--p", type=float, default=0.9)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-side-stream", action="store_true")
    ap.add_argument("--sparse-mode", choices=["fused", "scan_local", "union", "per_head"],
                    default="fused",
                    help="scan_local: scan and local heads in one rtp_scan_local launch, sparse "
                         "heads in rtp_decode_attend; fused: sparse and local heads in one "
                         "rtp_decode_attend launch; per_head: separate calls, local heads on "
                         "a side stream; union: each kept row read once per KV head for all "
                         "its query heads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="end with a 256 MiB device-to-device copy, whose known size "
                         "calibrates the HBM byte counters of a --pmc profile")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import sparse_long_context_indexer_amd as rtp
    from sparse_long_context_indexer_amd.runner import DecodeLayer

    rtp.lib()  # fails loudly if librtp.so is missing
    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    B, L, N, Hq, Hkv, H_r, d = cfg.B, cfg.L, cfg.N, cfg.Hq, cfg.Hkv, cfg.H_r, cfg.d
    G_r = cfg.G_r
    p = args.p if args.p else cfg.p_list[0]

    # ---------------------------------------------------------- inputs
    t0 = time.time()
    log(f"allocating {cfg.name}: L={L} B={B} N={N} Hq={Hq} Hkv={Hkv} H_r={H_r}")
    K_all = torch.empty((L, B, Hkv, N, d), dtype=torch.int16, device=dev)
    V_all = torch.empty((L, B, Hkv, N, d), dtype=torch.int16, device=dev)
    kr_all = torch.empty((L, B, G_r, N, cfg.r), dtype=torch.float32, device=dev)
    qr_all = torch.empty((L, B, H_r, cfg.r), dtype=torch.float32, device=dev)
    q_all = torch.empty((L, B, Hq, d), dtype=torch.int16, device=dev)
    out_all = torch.zeros((L, B, Hq, d), dtype=torch.float32, device=dev)
    stage = [torch.empty((B, Hkv, N, d), dtype=torch.int16, pin_memory=True) for _ in range(2)]
    copy_stream = torch.cuda.Stream(device=dev)
    evs = [None, None]
    n = 0
    for l in range(L):
        for which, dst in (("K", K_all), ("V", V_all)):
            buf = n % 2
            if evs[buf] is not None:
                evs[buf].synchronize()
            synth.layer_kv(cfg, l, which, out=stage[buf].numpy().view(np.uint16))
            with torch.cuda.stream(copy_stream):
                dst[l].copy_(stage[buf], non_blocking=True)
                evs[buf] = torch.cuda.Event()
                evs[buf].record(copy_stream)
            n += 1
        kr_all[l].copy_(torch.from_numpy(synth.layer_kr(cfg, l)))
        qr_all[l].copy_(torch.from_numpy(synth.layer_qr(cfg, l)))
        q_all[l].copy_(torch.from_numpy(synth.layer_q(cfg, l).view(np.int16)))
        if l % 8 == 7:
            log(f"  uploaded layers 0..{l} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    del stage
    log(f"inputs resident ({time.time() - t0:.1f}s)")

    step_layer = DecodeLayer(B, Hq, Hkv, N, H_r, cfg.n_sink, cfg.window, dev,
                             mode=args.sparse_mode)
    scale = cfg.scale

    # Local heads of a layer run on a side stream, overlapping the retrieval
    # chain of the same layer; each layer joins both before the next starts.
    side = (None if args.no_side_stream or args.sparse_mode in ("fused", "scan_local")
            else torch.cuda.Stream(device=dev))

    def step():
        for l in range(L):
            step_layer(qr_all[l], kr_all[l], q_all[l], K_all[l], V_all[l], p, scale, out_all[l],
                       side_stream=side)

    stream = torch.cuda.current_stream(dev)
    if args.no_graph:
        run = step
    else:
        step()  # warm the caching allocator outside capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay

    # ---------------------------------------------------------- timing
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall / args.steps * 1e3:.3f})")

    # ------------------------------------------ per-call timing
    # Each C-ABI call of the step, for every layer with that layer's own
    # inputs (scores, kept sets), captured as one HIP graph of L launches so
    # that no host launch gap separates them, and replayed between HIP
    # events on the stream the launches run on: the time per launch is the
    # kernels' own duration back to back.
    sl = step_layer
    scores_l = torch.empty((L, B, H_r, N), dtype=torch.float32, device=dev)
    idx_l = torch.empty((L, B, H_r, N), dtype=torch.int32, device=dev)
    count_l = torch.empty((L, B, H_r), dtype=torch.int32, device=dev)
    keep_l = (torch.empty((L,) + tuple(sl.keep_bits.shape), dtype=torch.int32, device=dev)
              if sl.keep_bits is not None else None)
    for l in range(L):
        rtp.rtp_index_scores(qr_all[l], kr_all[l], scores_l[l])
        rtp.rtp_topp_select(scores_l[l], p, idx_l[l], count_l[l], sl.ws_sel,
                            keep_bits=None if keep_l is None else keep_l[l])
    torch.cuda.synchronize()

    def time_call(issue, reps=5):
        issue()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            issue()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / reps / L * 1e3  # us per launch (one layer)

    us = {
        "rtp_index_scores": time_call(lambda: [rtp.rtp_index_scores(qr_all[l], kr_all[l],
                                                                    scores_l[l])
                                               for l in range(L)]),
        "rtp_topp_select": time_call(lambda: [rtp.rtp_topp_select(
            scores_l[l], p, idx_l[l], count_l[l], sl.ws_sel,
            keep_bits=None if keep_l is None else keep_l[l]) for l in range(L)]),
        "rtp_topp_hist": time_call(lambda: [rtp.rtp_topp_hist(scores_l[l], sl.ws_sel)
                                            for l in range(L)]),
    }
    # Static top-k, the fixed budget that dynamic top-p replaces, timed on the
    # same scores at the workload's mean top-p budget: a reference call, not
    # part of the step (sel_fused_kernel<true>, the same launch shape).
    k_budget = max(1, int(round(float(count_l.float().mean().item()))))
    idx_k = torch.empty_like(idx_l[0])
    count_k = torch.empty_like(count_l[0])
    us["rtp_topk_select"] = time_call(lambda: [rtp.rtp_topk_select(
        scores_l[l], k_budget, idx_k, count_k, sl.ws_sel) for l in range(L)])
    # The scan over a bf16 copy of the indexer key cache (32 B per token
    # instead of 64), a reference call: the step scans the fp32 cache.
    kr_b = kr_all.to(torch.bfloat16).view(torch.int16)
    us["rtp_index_scores_bf16"] = time_call(lambda: [rtp.rtp_index_scores_bf16(
        qr_all[l], kr_b[l % kr_b.shape[0]], scores_l[l]) for l in range(L)])
    # The whole step with the bf16 key caches (the runner scans them with
    # rtp_index_scores_bf16), captured and replayed like the step above: a
    # reference figure for that variant, not the headline.
    def step_bf16():
        for l in range(L):
            step_layer(qr_all[l], kr_b[l], q_all[l], K_all[l], V_all[l], p, scale, out_all[l],
                       side_stream=side)
    step_bf16()
    torch.cuda.synchronize()
    g16 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g16):
        step_bf16()
    g16.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        g16.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step_bf16 = e0.elapsed_time(e1) / 5
    del g16, kr_b
    # Indexer projections (reference calls, not part of the step, whose q_r
    # and k_r are given): the prefill k_r build of one retrieval KV head
    # over all N tokens (256 B of bf16 features read, 64 B of k_r written
    # per token, on the matrix cores), and one decode token's q_r for the
    # H_r retrieval heads plus its k_r row appended at row N - 1.
    def bf16_bits(*shape):  # N(0,1) values as bf16 bit patterns
        return torch.randn(shape, dtype=torch.bfloat16, device=dev).view(torch.int16)
    xp = bf16_bits(1, 1, N, d)
    Wp = bf16_bits(G_r, 16, d)
    kr_out = torch.empty((1, 1, N, 16), dtype=torch.float32, device=dev)
    us["rtp_index_project_prefill"] = time_call(lambda: [rtp.rtp_index_project(
        xp, Wp[:1], kr_out) for l in range(L)])
    qp = bf16_bits(B, Hq, 1, d)
    Wq = bf16_bits(H_r, 16, d)
    qr_out = torch.empty((B, H_r, 1, 16), dtype=torch.float32, device=dev)
    kp = bf16_bits(B, Hkv, 1, d)
    kr_cache = torch.empty((B, G_r, N, 16), dtype=torch.float32, device=dev)
    us["rtp_index_project_decode"] = time_call(lambda: [
        (rtp.rtp_index_project(qp, Wq, qr_out),
         rtp.rtp_index_project(kp, Wp, kr_cache, out_pos=N - 1)) for l in range(L)])
    proj_gbps = N * (d * 2 + 16 * 4) / (us["rtp_index_project_prefill"] * 1e-6) / 1e9
    # Prefill attention of a 16384-token prompt on layer 0's cache, a
    # reference call: the retrieval heads dense, the local heads sinks +
    # window, one launch each.  Flops: 4 * d per (query, key) pair.
    T_pf = 16384
    q_pf = bf16_bits(B, Hq, T_pf, d)
    out_pf = torch.empty((B, Hq, T_pf, d), dtype=torch.float32, device=dev)
    us["rtp_prefill_attend_16k"] = time_call(lambda: [(
        rtp.rtp_prefill_attend(q_pf, K_all[0], V_all[0], 0, H_r, 0, 0, scale, out_pf),
        rtp.rtp_prefill_attend(q_pf, K_all[0], V_all[0], H_r, Hq - H_r, cfg.n_sink, cfg.window,
                               scale, out_pf)) for _ in range(4)]) * L / 4
    t_idx = np.arange(T_pf, dtype=np.float64)
    w0 = np.maximum(0, t_idx + 1 - cfg.window)
    local_pairs = float(np.sum(np.minimum(cfg.n_sink, w0) + (t_idx + 1 - w0)))
    pf_flops = B * 4 * d * (H_r * T_pf * (T_pf + 1) / 2 + (Hq - H_r) * local_pairs)
    pf_tflops = pf_flops / (us["rtp_prefill_attend_16k"] * 1e-6) / 1e12
    del q_pf, out_pf
    del xp, kr_out, kr_cache
    # rtp_topp_select runs both passes in one launch (sel_fused_kernel) when
    # its histogram and emit block rows fit one grid (2 * B * H_r <= 65535);
    # rtp_topp_hist, the histogram pass alone, is then timed for reference
    # only.  Otherwise it launches the hist kernel then the emit kernel, and
    # the emit kernel's duration is the difference.
    fused_select = 2 * B * H_r <= 65535
    if not fused_select:
        us["sel_emit_kernel"] = us["rtp_topp_select"] - us["rtp_topp_hist"]
    if sl.mode == "scan_local":
        us["rtp_scan_local"] = time_call(lambda: [rtp.rtp_scan_local(
            qr_all[l], kr_all[l], scores_l[l], q_all[l], K_all[l], V_all[l], N, H_r, Hq - H_r,
            cfg.n_sink, cfg.window, scale, out_all[l], sl.ws_local) for l in range(L)])
        us["rtp_decode_attend"] = time_call(lambda: [rtp.rtp_decode_attend(
            q_all[l], K_all[l], V_all[l], idx_l[l], count_l[l], N, 0, H_r, 0, 0, 1, scale,
            out_all[l], sl.ws_attend) for l in range(L)])
    elif sl.mode == "fused":
        us["rtp_decode_attend"] = time_call(lambda: [rtp.rtp_decode_attend(
            q_all[l], K_all[l], V_all[l], idx_l[l], count_l[l], N, 0, H_r, Hq - H_r,
            cfg.n_sink, cfg.window, scale, out_all[l], sl.ws_attend) for l in range(L)])
    elif sl.mode == "union":
        us["rtp_sparse_decode_union"] = time_call(lambda: [rtp.rtp_sparse_decode_union(
            q_all[l], K_all[l], V_all[l], keep_l[l], N, 0, scale, out_all[l], sl.ws_sparse)
            for l in range(L)])
    else:
        us["rtp_sparse_decode"] = time_call(lambda: [rtp.rtp_sparse_decode(
            q_all[l], K_all[l], V_all[l], idx_l[l], count_l[l], 0, scale, out_all[l],
            sl.ws_sparse) for l in range(L)])
    if sl.mode not in ("fused", "scan_local"):
        us["rtp_local_decode"] = time_call(lambda: [rtp.rtp_local_decode(
            q_all[l], K_all[l], V_all[l], N, H_r, Hq - H_r, cfg.n_sink, cfg.window, scale,
            out_all[l], sl.ws_local) for l in range(L)])
    log("per-call us/layer: " + ", ".join(f"{k}={v:.2f}" for k, v in us.items()))

    # --------------------------------------------- algorithmic bytes
    # Per layer: the k_r scan (N * 16 fp32 per retrieval KV head), the union
    # of the retrieval heads' kept rows (K + V, 512 B each), and the local
    # heads' sink + window rows (512 B each, once per local KV head).
    w_start = max(0, N - cfg.window)
    w_rows = min(cfg.n_sink, w_start) + (N - w_start)
    local_kv = Hkv - G_r
    n_sel = []
    union = []
    counts = count_l.cpu().numpy()
    for l in range(L):
        cnt = counts[l]
        u = 0
        for b in range(B):
            for g in range(G_r):
                mark = torch.zeros(N, dtype=torch.bool, device=dev)
                for h in range(g * cfg.G, min(H_r, (g + 1) * cfg.G)):
                    mark[idx_l[l, b, h, :int(cnt[b, h])].long()] = True
                u += int(mark.sum().item())
        union.append(u)
        n_sel.append(cnt.reshape(-1).tolist())
    del scores_l, idx_l, keep_l
    torch.cuda.synchronize()
    kr_bytes = B * G_r * N * cfg.r * 4
    gather_bytes = np.array(union) * 2 * d * 2
    window_bytes = B * local_kv * w_rows * 2 * d * 2
    B_alg = float(L * kr_bytes + gather_bytes.sum() + L * window_bytes)
    B_ns = float(sum(B * G_r * N * cfg.r * 2 + u * 2 * d * 2 + B * local_kv * w_rows * 2 * d * 2
                     for u in union))
    steps_per_s = 1e3 / ms_step
    achieved_gbps = B_alg / (ms_step * 1e-3) / 1e9

    # Roofline of the dominant kernel: the kernel with the largest time per
    # layer.  Calls that launch one kernel are timed directly.  Algorithmic
    # bytes per launch (one layer):
    #   select  4 B per score read + 4 B per kept index written (one launch:
    #           its histogram and emit blocks each read the scores; the
    #           second read earns no credit);
    #   emit    the same, for the emit kernel of the two-launch selection;
    #   hist    4 B per score read;
    #   scan    64 B of k_r read + 4 B of score written per query head, per
    #           token and retrieval KV head;
    #   sparse  512 B (K + V row) per row of the union of the group's kept
    #           sets (re-reads by several heads earn no credit) + the 4-B
    #           indices read;
    #   local   512 B per sink/window row per local KV head;
    #   attend  sparse (+ local in mode "fused"), one launch;
    #   scan + local, one launch (mode "scan_local").
    csrc = os.path.join(ROOT, "sparse_long_context_indexer_amd", "csrc")
    sel_total = float(np.mean([sum(x) for x in n_sel]))
    sparse_bytes = float(np.mean(union)) * 2 * d * 2 + sel_total * 4
    sel_bytes = B * H_r * N * 4 + sel_total * 4
    cands = {
        "sel_emit_kernel": ("sel_emit_kernel<false>", sel_bytes, "select.hip"),
        "rtp_topp_hist": ("sel_hist_kernel<false>", B * H_r * N * 4, "select.hip"),
        "rtp_index_scores": ("index_scores_kernel<8, false>", B * G_r * N * (cfg.r * 4 + cfg.G * 4),
                             "scan.hip"),
        "rtp_decode_attend": ("attend_kernel",
                              sparse_bytes + (window_bytes if sl.mode == "fused" else 0),
                              "attend.hip"),
        "rtp_scan_local": ("scan_local_kernel<8>",
                           B * G_r * N * (cfg.r * 4 + cfg.G * 4) + window_bytes, "attend.hip"),
        "rtp_sparse_decode": ("attend_kernel", sparse_bytes, "attend.hip"),
        "rtp_sparse_decode_union": ("union_attn_kernel",
                                    float(np.mean(union)) * 2 * d * 2 + B * H_r * ((N + 31) // 32) * 4,
                                    "attend.hip"),
        "rtp_local_decode": ("attend_kernel", window_bytes, "attend.hip"),
    }
    if fused_select:
        cands["rtp_topp_select"] = ("sel_fused_kernel<false>", sel_bytes, "select.hip")
    # Calls timed for reference only, outside the step: rtp_index_scores in
    # mode "scan_local" (the step runs the scan inside rtp_scan_local) and
    # rtp_topp_hist when the selection is one launch.
    in_step = [c for c in cands if c in us
               and not (sl.mode == "scan_local" and c == "rtp_index_scores")
               and not (fused_select and c == "rtp_topp_hist")]
    call = max(in_step, key=lambda c: us[c])
    kname, kbytes, ksrc = cands[call]
    roof = {"kernel": kname, "bound": "hbm",
            "achieved": kbytes / (us[call] * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(os.path.join(ROOT, "profiles", "hbm_traffic_ctx1m.md"),
                                       kname, os.path.join(csrc, ksrc))

    # ---------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, p, args.cpu_seconds)

    tokens_scanned = B * G_r * N * L
    rec = {
        "metric": "sparse-decode steps/s at 128K-1M ctx; achieved HBM GB/s vs MI355X peak",
        "value": round(steps_per_s, 3), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": L, "batch": B, "ctx_tokens": N,
                   "q_heads": Hq, "kv_heads": Hkv, "retrieval_q_heads": H_r,
                   "head_dim": d, "indexer_dim": cfg.r, "p": p, "sinks": cfg.n_sink,
                   "window": cfg.window, "kv_dtype": "bf16", "graph": not args.no_graph,
                   "sparse_mode": args.sparse_mode,
                   "local_side_stream": side is not None},
        "B_alg_bytes": B_alg, "B_ns_bytes": B_ns,
        "achieved_GBps": round(achieved_gbps, 1),
        "frac_of_hbm_peak": round(achieved_gbps / HBM_PEAK_GBPS, 4),
        "tokens_scanned_per_s": tokens_scanned * steps_per_s,
        "selected_per_head_mean": float(np.mean(n_sel)),
        "union_rows_per_layer_mean": float(np.mean(union)),
        "per_call_us_per_layer": {k: round(v, 2) for k, v in us.items()},
        "topk_budget": k_budget,
        "ms_per_step_bf16_kr": round(ms_step_bf16, 4),
        "project_prefill_GBps": round(proj_gbps, 1),
        "prefill_16k_TFLOPs": round(pf_tflops, 1),
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()


def measured_traffic(summary, kernel, source):
    """HBM bytes per launch of `kernel` from the committed PMC summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a
    copy of known size), or None when that kernel's source file has changed
    since the counters were taken.  The summary holds lines
    `traffic <kernel> <bytes per launch> <sha256 of its source file>`."""
    import hashlib
    try:
        lines = open(summary).read().splitlines()
    except OSError:
        return None
    sha = hashlib.sha256(open(source, "rb").read()).hexdigest()
    for line in lines:
        f = line.split()
        if len(f) == 4 and f[0] == "traffic" and f[1] == kernel:
            return float(f[2]) if f[3] == sha else None
    return None


def cpu_baseline(cfg, p, target_s):
    """The CPU oracle on whole layers of the same workload (same generator,
    same inputs): scores, full-sort top-p and fp64 attention for every
    retrieval head, fp64 sink + window attention for every local head.
    Only oracle calls are timed; input generation is not."""
    import oracle
    import synth
    layers = 0
    spent = 0.0
    while spent < target_s and layers < cfg.L:
        l = layers
        q_r, k_r, q = synth.layer_qr(cfg, l), synth.layer_kr(cfg, l), synth.layer_q(cfg, l)
        for b in range(cfg.B):
            sets = []
            t = time.perf_counter()
            for h in range(cfg.H_r):
                s = oracle.scores(q_r[b, h], k_r[b, min(h // cfg.G, cfg.G_r - 1)])
                sets.append(oracle.topp(s, p).sel)
            spent += time.perf_counter() - t
            for h in range(cfg.Hq):
                g = h // cfg.G
                rows = np.sort(sets[h]) if h < cfg.H_r else oracle.local_rows(cfg.N, cfg.n_sink, cfg.window)
                Kr = synth.kv_rows(cfg, l, "K", b, g, rows)
                Vr = synth.kv_rows(cfg, l, "V", b, g, rows)
                t = time.perf_counter()
                oracle.attention(q[b, h], Kr, Vr, cfg.scale)
                spent += time.perf_counter() - t
        layers += 1
        log(f"  cpu oracle: {layers} layer(s), {spent:.1f}s")
    return {"value": round(layers / cfg.L / spent, 5), "unit": "steps/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{layers} of {cfg.L} layers of {cfg.name} (all 32 heads), "
                      f"{spent:.1f}s single-threaded; value = layers/{cfg.L}/seconds"}


if __name__ == "__main__":
    main()
