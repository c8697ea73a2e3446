"""Decode-step benchmark of the RTPurbo sparse decode path on one MI355X.

One step = one decode step through a 48-layer attention stack at N = 2^20
cached tokens (batch 1, 32 query / 4 KV heads, d = 128, bf16 K/V ~ 96 GiB
resident): per layer, the indexer scan, top-p selection and sparse
attention for the 8 retrieval query heads of KV head 0, and sink + window
attention for the 24 local query heads.  Layers run in sequence; by default
each layer is one rtp_decode_layer launch.  The step is captured once in a
HIP graph and replayed.

Prints ONE JSON line (rank 0) with steps/s, the dominant kernel's roofline,
the CPU oracle's baseline on a bounded sample, the four-call path timed
beside it, and one record per smaller workload (configs 1-3, each p).
"""
from __future__ import annotations

import argparse
import json
import math
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
    ap.add_argument("--sparse-mode", choices=["layer", "fused", "topp_attend", "scan_local",
                                              "union", "per_head"],
                    default="fused",
                    help="layer: the whole layer in one rtp_decode_layer launch; topp_attend: "
                         "the scan, then selection and attention in one rtp_topp_attend "
                         "launch; scan_local: "
                         "scan and local heads in one rtp_scan_local launch, sparse "
                         "heads in rtp_decode_attend; fused: sparse and local heads in one "
                         "rtp_decode_attend launch; per_head: separate calls, local heads on "
                         "a side stream; union: each kept row read once per KV head for all "
                         "its query heads")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the records of the smaller workloads (configs 1-3)")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the reference calls (four-call path, top-k, bf16 keys, "
                         "projections, prefill)")
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
                             mode=args.sparse_mode, keep_scores=False)
    scale = cfg.scale

    # Local heads of a layer run on a side stream, overlapping the retrieval
    # chain of the same layer; each layer joins both before the next starts.
    side = (None if args.no_side_stream
            or args.sparse_mode in ("layer", "fused", "topp_attend", "scan_local")
            else torch.cuda.Stream(device=dev))
    stream = torch.cuda.current_stream(dev)

    def timed_step(layer_call, steps, warmup):
        """ms per step of layer_call(l) for l < L, captured once as a HIP
        graph (unless --no-graph) and replayed between HIP events."""
        def step():
            for l in range(L):
                layer_call(l)
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
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w) / steps * 1e3
        return e0.elapsed_time(e1) / steps, wall

    ms_step, wall_step = timed_step(
        lambda l: step_layer(qr_all[l], kr_all[l], q_all[l], K_all[l], V_all[l], p, scale,
                             out_all[l], side_stream=side), args.steps, args.warmup)
    log(f"timed {args.steps} steps ({args.sparse_mode}): {ms_step:.3f} ms/step "
        f"(wall {wall_step:.3f})")

    # ------------------------------------------ per-call timing
    # Each C-ABI call, for every layer with that layer's own inputs, captured
    # as one HIP graph of L launches so that no host launch gap separates
    # them, and replayed between HIP events on the stream the launches run
    # on: the time per launch is the kernels' own duration back to back.
    idx_l = torch.empty((L, B, H_r, N), dtype=torch.int32, device=dev)
    count_l = torch.empty((L, B, H_r), dtype=torch.int32, device=dev)
    ws_layer = torch.empty(rtp.decode_layer_workspace_size(B, Hq, Hkv, N, H_r, cfg.n_sink,
                                                           cfg.window),
                           dtype=torch.uint8, device=dev)

    def layer_call(l):
        rtp.rtp_decode_layer(qr_all[l], kr_all[l], q_all[l], K_all[l], V_all[l], N, H_r,
                             cfg.n_sink, cfg.window, p, scale, out_all[l], idx_l[l], count_l[l],
                             ws_layer)

    for l in range(L):
        layer_call(l)
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

    us = {"rtp_decode_layer": time_call(lambda: [layer_call(l) for l in range(L)])}
    ref = {}
    if not args.no_reference or args.sparse_mode != "layer":
        ref = reference_calls(args, cfg, p, dev, stream, L, qr_all, kr_all, q_all, K_all, V_all,
                              out_all, time_call, timed_step, us)
    log("per-call us/layer: " + ", ".join(f"{k}={v:.2f}" for k, v in us.items()))

    # --------------------------------------------- algorithmic bytes
    # Per layer: the k_r scan (N * 16 fp32 per retrieval KV head), the union
    # of the retrieval heads' kept rows (K + V, 512 B each), and the local
    # heads' sink + window rows (512 B each, once per local KV head).  The
    # kept sets are the layer call's own.
    w_start = max(0, N - cfg.window)
    w_rows = min(cfg.n_sink, w_start) + (N - w_start)
    local_kv = Hkv - G_r
    n_sel, union = kept_stats(idx_l, count_l, cfg, dev)
    del idx_l
    torch.cuda.synchronize()
    kr_bytes = B * G_r * N * cfg.r * 4
    gather_bytes = np.array(union) * 2 * d * 2
    window_bytes = B * local_kv * w_rows * 2 * d * 2
    B_alg = float(L * kr_bytes + gather_bytes.sum() + L * window_bytes)
    B_ns = float(sum(B * G_r * N * cfg.r * 2 + u * 2 * d * 2 + B * local_kv * w_rows * 2 * d * 2
                     for u in union))
    steps_per_s = 1e3 / ms_step
    achieved_gbps = B_alg / (ms_step * 1e-3) / 1e9

    # Roofline of the dominant kernel of the step.  In mode "layer" that is
    # the layer kernel itself (one launch per layer): its algorithmic bytes
    # per launch are the layer's B_alg (k_r + union rows + window rows; score,
    # histogram and workspace traffic earns no credit).
    csrc = os.path.join(ROOT, "sparse_long_context_indexer_amd", "csrc")
    if args.sparse_mode == "layer":
        kname, kbytes, ksrc, kus = "layer_kernel<8>", B_alg / L, "layer.hip", us["rtp_decode_layer"]
    else:
        kname, kbytes, ksrc, kus = ref["roof"]
    roof = {"kernel": kname, "bound": "hbm", "achieved": kbytes / (kus * 1e-6) / 1e9,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
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
    }
    rec.update({k: v for k, v in ref.items() if k != "roof"})
    rec["roofline"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()}
    rec["cpu_baseline"] = cpu

    # ------------------------------------------- the smaller workloads
    if not args.no_configs:
        del K_all, V_all, kr_all, qr_all, q_all, out_all, ws_layer, step_layer
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        rec["configs"] = [r for ci in (0, 1, 2, 3) for r in config_records(ci, dev, stream)]
    print(json.dumps(rec), flush=True)

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()


def kept_stats(idx, count, cfg, dev):
    """Per layer: the kept-set sizes of every retrieval head and the size of
    the union of each KV group's kept sets (summed over rows and groups)."""
    import torch
    L, B, H_r, N = idx.shape
    counts = count.cpu().numpy()
    n_sel, union = [], []
    for l in range(L):
        u = 0
        for b in range(B):
            for g in range(cfg.G_r):
                mark = torch.zeros(N, dtype=torch.bool, device=dev)
                for h in range(g * cfg.G, min(H_r, (g + 1) * cfg.G)):
                    mark[idx[l, b, h, :int(counts[l, b, h])].long()] = True
                u += int(mark.sum().item())
        union.append(u)
        n_sel.append(counts[l].reshape(-1).tolist())
    return n_sel, union


def reference_calls(args, cfg, p, dev, stream, L, qr_all, kr_all, q_all, K_all, V_all, out_all,
                    time_call, timed_step, us):
    """Calls timed beside the step for reference: the four-call layer
    (scan, select, attend: its launches one by one and as a whole step), the
    static top-k selector, the scan over bf16 keys, the indexer projections
    and a 16K-token prefill.  Adds their microseconds per launch to `us`
    and returns the extra record keys."""
    import torch
    import sparse_long_context_indexer_amd as rtp
    from sparse_long_context_indexer_amd.runner import DecodeLayer
    B, N, Hq, Hkv, H_r, d, G_r = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.H_r, cfg.d, cfg.G_r
    scale = cfg.scale
    four = DecodeLayer(B, Hq, Hkv, N, H_r, cfg.n_sink, cfg.window, dev, mode="fused")
    scores_l = torch.empty((L, B, H_r, N), dtype=torch.float32, device=dev)
    idx_l = torch.empty((L, B, H_r, N), dtype=torch.int32, device=dev)
    count_l = torch.empty((L, B, H_r), dtype=torch.int32, device=dev)
    for l in range(L):
        rtp.rtp_index_scores(qr_all[l], kr_all[l], scores_l[l])
        rtp.rtp_topp_select(scores_l[l], p, idx_l[l], count_l[l], four.ws_sel)
    torch.cuda.synchronize()
    us["rtp_index_scores"] = time_call(lambda: [rtp.rtp_index_scores(qr_all[l], kr_all[l],
                                                                     scores_l[l])
                                                for l in range(L)])
    us["rtp_topp_select"] = time_call(lambda: [rtp.rtp_topp_select(
        scores_l[l], p, idx_l[l], count_l[l], four.ws_sel) for l in range(L)])
    us["rtp_topp_hist"] = time_call(lambda: [rtp.rtp_topp_hist(scores_l[l], four.ws_sel)
                                             for l in range(L)])
    us["rtp_decode_attend"] = time_call(lambda: [rtp.rtp_decode_attend(
        q_all[l], K_all[l], V_all[l], idx_l[l], count_l[l], N, 0, H_r, Hq - H_r,
        cfg.n_sink, cfg.window, scale, out_all[l], four.ws_attend) for l in range(L)])
    ms_four, _ = timed_step(lambda l: four(qr_all[l], kr_all[l], q_all[l], K_all[l], V_all[l],
                                           p, scale, out_all[l]), 5, 1)
    # Selection and attention in one launch (rtp_topp_attend), on the same
    # per-layer scores, and the step with it (scan + one launch per layer).
    ws_ta = torch.empty(rtp.topp_attend_workspace_size(B, Hq, Hkv, N, H_r, cfg.n_sink,
                                                       cfg.window),
                        dtype=torch.uint8, device=dev)
    idx_t = torch.empty_like(idx_l[0])
    count_t = torch.empty_like(count_l[0])
    us["rtp_topp_attend"] = time_call(lambda: [rtp.rtp_topp_attend(
        scores_l[l], q_all[l], K_all[l], V_all[l], cfg.n_sink, cfg.window, p, scale, out_all[l],
        idx_t, count_t, ws_ta) for l in range(L)])
    del ws_ta, idx_t, count_t
    ta = DecodeLayer(B, Hq, Hkv, N, H_r, cfg.n_sink, cfg.window, dev, mode="topp_attend")
    ms_ta, _ = timed_step(lambda l: ta(qr_all[l], kr_all[l], q_all[l], K_all[l], V_all[l],
                                       p, scale, out_all[l]), 5, 1)
    del ta
    # Static top-k at the workload's mean top-p budget (sel_fused_kernel<true>).
    k_budget = max(1, int(round(float(count_l.float().mean().item()))))
    idx_k = torch.empty_like(idx_l[0])
    count_k = torch.empty_like(count_l[0])
    us["rtp_topk_select"] = time_call(lambda: [rtp.rtp_topk_select(
        scores_l[l], k_budget, idx_k, count_k, four.ws_sel) for l in range(L)])
    # The scan over a bf16 copy of the indexer key cache, and the four-call
    # step with it.
    kr_b = kr_all.to(torch.bfloat16).view(torch.int16)
    us["rtp_index_scores_bf16"] = time_call(lambda: [rtp.rtp_index_scores_bf16(
        qr_all[l], kr_b[l], scores_l[l]) for l in range(L)])
    ms_bf16, _ = timed_step(lambda l: four(qr_all[l], kr_b[l], q_all[l], K_all[l], V_all[l], p,
                                           scale, out_all[l]), 5, 1)
    del kr_b, scores_l, idx_l, idx_k, count_k
    # Indexer projections: the prefill k_r build of one retrieval KV head over
    # all N tokens, and one decode token's q_r for the H_r heads plus its k_r
    # row appended at row N - 1.
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
    del xp, kr_out, kr_cache
    # Prefill attention of a 16384-token prompt on layer 0's cache: the
    # retrieval heads dense, the local heads sinks + window, one launch
    # each.  Flops: 4 * d per (query, key) pair.
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
    sel_bytes = B * H_r * N * 4 + float(count_l.float().sum().item()) / L * 4
    out = {"ms_per_step_four_call": round(ms_four, 4),
           "ms_per_step_topp_attend": round(ms_ta, 4),
           "ms_per_step_four_call_bf16_kr": round(ms_bf16, 4),
           "topk_budget": k_budget,
           "project_prefill_GBps": round(proj_gbps, 1),
           "prefill_16k_TFLOPs": round(pf_tflops, 1),
           "roof": ("sel_fused_kernel<false>", sel_bytes, "select.hip", us["rtp_topp_select"])}
    del four
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def config_records(ci, dev, stream, reps=10):
    """Records of one smaller workload at each of its p: the one-launch layer
    over R input replicas at distinct addresses (R * B_alg >= 1 GiB, so the
    caches hold none of a step's inputs: cold), and on one replica (hot);
    kept-set sizes and unions; boundary exemptions and output errors against
    the oracle; and the oracle's own time for the whole step (every head:
    scores, full-sort top-p and fp64 attention over its set; local heads
    over sinks + window), single-threaded, oracle calls only."""
    import torch
    import oracle
    import synth
    import sparse_long_context_indexer_amd as rtp
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import judge_out, judge_set
    cfg = synth.CONFIGS[ci]
    B, N, Hq, Hkv, H_r, d, G_r = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.H_r, cfg.d, cfg.G_r
    t0 = time.time()
    q_r, k_r, q = synth.layer_qr(cfg, 0), synth.layer_kr(cfg, 0), synth.layer_q(cfg, 0)
    K, V = synth.layer_kv(cfg, 0, "K"), synth.layer_kv(cfg, 0, "V")
    d_in = [torch.from_numpy(x).to(dev) for x in
            (q_r, k_r, q.view(np.int16), K.view(np.int16), V.view(np.int16))]
    w_start = max(0, N - cfg.window)
    w_rows = min(cfg.n_sink, w_start) + (N - w_start)
    local_kv = Hkv - G_r
    ws = torch.empty(rtp.decode_layer_workspace_size(B, Hq, Hkv, N, H_r, cfg.n_sink, cfg.window),
                     dtype=torch.uint8, device=dev)
    recs = []
    for p in cfg.p_list:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        idx = torch.empty((B, H_r, N), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, H_r), dtype=torch.int32, device=dev)

        def call(x, o=out, i=idx, c=cnt):
            rtp.rtp_decode_layer(x[0], x[1], x[2], x[3], x[4], N, H_r, cfg.n_sink, cfg.window,
                                 p, cfg.scale, o, i, c, ws)
        call(d_in)
        torch.cuda.synchronize()
        n_sel, union = kept_stats(idx[None], cnt[None], cfg, dev)
        B_alg = float(B * G_r * N * cfg.r * 4 + union[0] * 2 * d * 2
                      + B * local_kv * w_rows * 2 * d * 2)
        R = max(1, math.ceil((1 << 30) / B_alg))
        reps_in = [d_in] + [[x.clone() for x in d_in] for _ in range(R - 1)]

        def timed(inputs):
            g = torch.cuda.CUDAGraph()
            for x in inputs:
                call(x)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for x in inputs:
                    call(x)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / (reps * len(inputs))
        ms_cold = timed(reps_in)
        ms_hot = timed([d_in] * 8)
        del reps_in
        # Against the oracle: exempt boundary tokens and output errors.
        c = cnt.cpu().numpy()
        ix = idx.cpu().numpy()
        o = out.cpu().numpy()
        exempt, bad, err, rel = 0, 0, 0.0, 0.0
        for b in range(B):
            for h in range(Hq):
                g = h // cfg.G
                if h < H_r:
                    s = oracle.scores(q_r[b, h], k_r[b, g])
                    v = judge_set(s, p, ix[b, h, :c[b, h]])
                    exempt += len(v.exempt)
                    bad += len(v.bad) + (0 if v.ok else 1)
                    rows = np.sort(ix[b, h, :c[b, h]])
                else:
                    rows = oracle.local_rows(N, cfg.n_sink, cfg.window)
                ok, e_abs, e_rel = judge_out(o[b, h], oracle.attention(q[b, h], K[b, g, rows],
                                                                       V[b, g, rows], cfg.scale))
                bad += 0 if ok else 1
                err, rel = max(err, e_abs), max(rel, e_rel)
        # The oracle's whole step, timed.
        t_or = 0.0
        for b in range(B):
            for h in range(Hq):
                g = h // cfg.G
                t = time.perf_counter()
                if h < H_r:
                    sel = oracle.topp(oracle.scores(q_r[b, h], k_r[b, g]), p).sel
                t_or += time.perf_counter() - t
                rows = (np.sort(sel) if h < H_r
                        else oracle.local_rows(N, cfg.n_sink, cfg.window))
                Kr, Vr = K[b, g, rows], V[b, g, rows]
                t = time.perf_counter()
                oracle.attention(q[b, h], Kr, Vr, cfg.scale)
                t_or += time.perf_counter() - t
        ns = np.array(n_sel[0]).reshape(B, H_r)
        rec = {"workload": cfg.name, "p": p, "batch": B, "ctx_tokens": N,
               "steps_per_s": round(1e3 / ms_cold, 1), "ms_per_step": round(ms_cold, 5),
               "ms_per_step_hot": round(ms_hot, 5), "replicas": R,
               "tokens_scanned_per_s": B * G_r * N / (ms_cold * 1e-3),
               "B_alg_bytes": B_alg, "GBps": round(B_alg / (ms_cold * 1e-3) / 1e9, 1),
               "frac_of_hbm_peak": round(B_alg / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               "n_S_per_row_head": ns.tolist(), "union_rows": union[0],
               "exempt_tokens": exempt, "parity_failures": bad,
               "max_abs_err": err, "max_rel_err": rel,
               "oracle_s_per_step": round(t_or, 4), "oracle_threads": 1}
        log(f"config {ci} p={p}: {ms_cold * 1e3:.1f} us/step cold ({R} replicas), "
            f"{ms_hot * 1e3:.1f} hot, {rec['GBps']} GB/s, union {union[0]}, exempt {exempt}, "
            f"failures {bad}")
        recs.append(rec)
    log(f"config {ci} done ({time.time() - t0:.1f}s)")
    del d_in, ws
    torch.cuda.empty_cache()
    return recs


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
                      f"{spent:.1f}s single-threaded; value = layers/{cfg.L}/seconds"
                      + (" (extrapolated from the layers timed)" if layers < cfg.L
                         else " (the whole step timed)"),
            "layers_timed": layers, "extrapolated": layers < cfg.L}


if __name__ == "__main__":
    main()
