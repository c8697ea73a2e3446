"""GPU parity: every kernel of the HIP path against the CPU oracle on the same
seeded inputs, through the C ABI (via the thin Python binding)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (MASS_SLACK, check_layer, dev, judge_out, judge_set, load_layer,
                     run_layer, to_dev)

pytestmark = pytest.mark.gpu

rtp = pytest.importorskip("sparse_long_context_indexer_amd")


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------ full configs

@pytest.mark.parametrize("mode", ["fused", "scan_local", "union", "per_head"])
@pytest.mark.parametrize("ci", [0, 1, 3])
def test_config_layer(ci, mode):
    cfg = synth.CONFIGS[ci]
    _print(f"config {ci} {cfg.name} ({mode})")
    L = load_layer(cfg)
    rep = {}
    res = run_layer(L, cfg.p_list[0], mode=mode)
    fails = check_layer(L, cfg.p_list[0], res, report=rep)
    _print(f"  k per head {rep['k']} exempt {rep['exempt']}")
    assert not fails, "\n".join(fails[:20])


def test_config2_budget_mix_all_p():
    cfg = synth.CONFIGS[2]
    L = load_layer(cfg)
    for p in cfg.p_list:
        rep = {}
        res = run_layer(L, p, mode="fused")
        fails = check_layer(L, p, res, report=rep)
        ks = np.array(rep["k"]).reshape(cfg.B, cfg.H_r)
        _print(f"config 2 p={p}: n_S per (row, head)\n{ks}\n  exempt {rep['exempt']}")
        assert not fails, "\n".join(fails[:20])


def test_config4_sampled_layers():
    # Full-size layers of the 48-layer 1M-context stack (same kernels and
    # launch shapes as the benchmark), judged in full for every head.
    cfg = synth.CONFIGS[4]
    for layer, mode in ((0, "fused"), (0, "union"), (47, "per_head"), (47, "fused"),
                        (21, "scan_local")):
        _print(f"config 4 layer {layer} ({mode})")
        L = load_layer(cfg, layer, keep_host_kv=False)
        rep = {}
        res = run_layer(L, 0.9, mode=mode)
        fails = check_layer(L, 0.9, res, report=rep)
        _print(f"  k per head {rep['k']} exempt {rep['exempt']}")
        del L
        torch.cuda.empty_cache()
        assert not fails, "\n".join(fails[:20])


# ------------------------------------------------------------ scan shapes

@pytest.mark.parametrize("B,Hq_r,Hkv_r,N,cap", [
    (1, 1, 1, 1, 1), (1, 8, 1, 1000, 1000), (2, 12, 1, 4097, 5000),
    (3, 6, 2, 3333, 3333), (1, 3, 3, 70000, 70001), (2, 16, 2, 1025, 1040)])
def test_scores_bit_exact_shapes(B, Hq_r, Hkv_r, N, cap):
    k = synth.key(77, synth.KR, N, B, Hq_r)
    q_r = synth.normal_f32(k, 0, B * Hq_r * 16).reshape(B, Hq_r, 16) * 3
    k_r = synth.normal_f32(k, 10**9, B * Hkv_r * cap * 16).reshape(B, Hkv_r, cap, 16)
    k_r[..., ::7, 3] = 0.0  # exact zeros, a zero score or two
    q_r[0, 0, :] = 0.0      # an all-zero query: every score +0
    s = torch.full((B, Hq_r, N), float("nan"), device=dev())
    rtp.rtp_index_scores(to_dev(q_r.astype(np.float32)), to_dev(k_r), s)
    got = s.cpu().numpy()
    G = Hq_r // Hkv_r
    for b in range(B):
        for h in range(Hq_r):
            ref = oracle.scores(q_r[b, h].astype(np.float32), k_r[b, h // G, :N])
            assert np.array_equal(got[b, h].view(np.uint32), ref.view(np.uint32)), (b, h)


# ---------------------------------------------------------- select stress

def _select(scores: np.ndarray, p: float):
    B, H, N = scores.shape
    sd = to_dev(scores.astype(np.float32))
    idx = torch.full((B, H, N), -7, dtype=torch.int32, device=dev())
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=dev())
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, B, H, N), dtype=torch.uint8,
                     device=dev())
    rtp.rtp_topp_select(sd, p, idx, cnt, ws)
    c = cnt.cpu().numpy()
    ix = idx.cpu().numpy()
    return [[ix[b, h, :c[b, h]] for h in range(H)] for b in range(B)], c


def _assert_select(scores, p, exact=False):
    sets, c = _select(scores, p)
    B, H, N = scores.shape
    for b in range(B):
        for h in range(H):
            v = judge_set(scores[b, h].astype(np.float32), p, sets[b][h])
            assert v.ok, (b, h, p, v.k_gpu, v.k_oracle, v.bad[:5], v.mass, v.note)
            if exact:
                assert not v.exempt, (b, h, v.exempt[:5])


def test_select_all_ties():
    # q_r = 0: every score is +0; the first ceil(p*N) indices are kept.
    for N in (4096, 100_003):
        s = np.zeros((1, 1, N), np.float32)
        sets, c = _select(s, 0.9)
        k = math.ceil(float(np.float32(0.9)) * N)
        assert c[0, 0] == k
        assert np.array_equal(np.sort(sets[0][0]), np.arange(k))


def test_select_many_duplicates():
    rng = np.random.default_rng(1)
    s = np.round(rng.standard_normal((2, 3, 50_000)) * 2).astype(np.float32)
    s[0, 0, ::3] = -0.0
    for p in (0.3, 0.9, 0.999):
        _assert_select(s, p, exact=True)


def test_select_tiny_rows_and_extremes():
    rng = np.random.default_rng(2)
    for N in range(1, 13):
        s = (rng.standard_normal((1, 4, N)) * rng.choice([0.1, 1, 10])).astype(np.float32)
        for p in (1e-6, 0.5, 0.9, 1.0):
            _assert_select(s, p, exact=True)
    s = (rng.standard_normal((1, 2, 20_000)) * 1000).astype(np.float32)   # one-hot-like
    _assert_select(s, 0.9, exact=True)
    s = (rng.standard_normal((1, 2, 20_000)) * 1e-3 - 50).astype(np.float32)  # flat, negative
    _assert_select(s, 0.95, exact=True)


@pytest.mark.parametrize("k", [2, 17, 63, 64, 65, 300])
@pytest.mark.parametrize("level", [6.0, 2.5])
def test_select_boundary_tie_group(k, level):
    # k tokens share one score; p puts the crossing inside that group, so
    # the kept set holds the group's lowest indices.  At level 6.0 the group
    # tops the row; at 2.5 distinct scores around it share its bins.  Sizes
    # straddle one wave of boundary candidates.
    rng = np.random.default_rng(17 + k)
    N = 50_000
    s = rng.standard_normal((1, 2, N)).astype(np.float32)
    for h in range(2):
        pos = rng.choice(N, k, replace=False)
        s[0, h, pos] = np.float32(level)
        x = s[0, h].astype(np.float64)
        w = np.exp(x - x.max())
        above = w[x > level].sum()
        group = w[x == level].sum()
        frac = 0.37 if h == 0 else 0.81
        pv = np.float32((above + frac * group) / w.sum())
        _assert_select(s[:, h:h + 1], float(pv), exact=True)


def test_select_p_one_keeps_all():
    s = np.random.default_rng(3).standard_normal((2, 2, 9000)).astype(np.float32)
    sets, c = _select(s, 1.0)
    assert np.all(c == 9000)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(np.sort(sets[b][h]), np.arange(9000))


def test_topp_hist_alone_then_select():
    # The histogram pass alone writes no output, and a select after one or
    # two of them still finds the oracle's sets.
    rng = np.random.default_rng(5)
    s = (rng.standard_normal((2, 3, 70_001)) * 3).astype(np.float32)
    sd = torch.from_numpy(s).to(dev())
    B, H, N = s.shape
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, B, H, N), dtype=torch.uint8,
                     device=dev())
    idx = torch.full((B, H, N), -7, dtype=torch.int32, device=dev())
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=dev())
    rtp.rtp_topp_hist(sd, ws)
    torch.cuda.synchronize()
    assert torch.all(idx == -7) and torch.all(cnt == -7)
    rtp.rtp_topp_hist(sd, ws)
    rtp.rtp_topp_select(sd, 0.9, idx, cnt, ws)
    c = cnt.cpu().numpy()
    ix = idx.cpu().numpy()
    for b in range(B):
        for h in range(H):
            v = judge_set(s[b, h], 0.9, ix[b, h, :c[b, h]])
            assert v.ok, (b, h, v.k_gpu, v.k_oracle)


def test_select_repeatable():
    cfg = synth.CONFIGS[2].with_(N=65536)
    q_r, k_r = synth.layer_qr(cfg, 0), synth.layer_kr(cfg, 0)
    s = np.stack([[oracle.scores(q_r[b, h], k_r[b, 0]) for h in range(8)] for b in range(4)])
    a, _ = _select(s, 0.9)
    b_, _ = _select(s, 0.9)
    for r in range(4):
        for h in range(8):
            assert set(a[r][h].tolist()) == set(b_[r][h].tolist())


def test_select_many_chunks():
    # 280 chunks of 32768 scores (more blocks than compute units), then the
    # same rows cut to 8 chunks each, against the oracle, on rows with
    # heavy-tailed, clustered and duplicated scores.
    rng = np.random.default_rng(23)
    B, H, N = 2, 5, 900_000
    s = rng.standard_normal((B, H, N)).astype(np.float32) * np.float32(2.0)
    s[:, :, ::97] += np.float32(6.0)                       # a heavy tail
    s[0, 1, :] = np.round(s[0, 1, :] * 4) / 4              # many exact duplicates
    s[1, 3, rng.integers(0, N, 2000)] = np.float32(9.5)    # a tie block at the top
    for n in (N, 8 * 32768 - 123):
        sub = np.ascontiguousarray(s[:, :, :n])
        for p in (0.5, 0.9):
            _assert_select(sub, p)


def test_select_two_launch_path():
    # 40000 score rows: more than one launch holds as histogram rows plus
    # emit rows, so the selection runs as a histogram launch then an emit
    # launch.
    rng = np.random.default_rng(29)
    s = (rng.standard_normal((1, 40000, 96)) * 3).astype(np.float32)
    s[0, ::3, ::5] = np.float32(1.25)  # ties
    sets, c = _select(s, 0.8)
    for h in range(0, 40000, 7):
        v = judge_set(s[0, h], 0.8, sets[0][h])
        assert v.ok, (h, v.k_gpu, v.k_oracle, v.note)


@pytest.mark.parametrize("B, Hq_r, Hkv_r, N, cap", [(1, 1, 1, 1, 1), (2, 8, 1, 70_001, 70_005),
                                                   (1, 12, 3, 4099, 4099), (1, 8, 1, 1 << 20, 1 << 20)])
def test_scores_bf16_keys_bit_exact(B, Hq_r, Hkv_r, N, cap):
    rng = np.random.default_rng(N + Hq_r)
    q = rng.standard_normal((B, Hq_r, 16)).astype(np.float32)
    kb = synth.f32_to_bf16(rng.standard_normal((B, Hkv_r, cap, 16)).astype(np.float32) * 2)
    sc = torch.full((B, Hq_r, N), 7.0, dtype=torch.float32, device=dev())
    rtp.rtp_index_scores_bf16(to_dev(q), torch.from_numpy(kb.view(np.int16)).to(dev()), sc)
    got = sc.cpu().numpy()
    G = Hq_r // Hkv_r
    heads = range(Hq_r) if N < (1 << 20) else (0, Hq_r - 1)
    for b in range(B):
        for h in heads:
            want = oracle.scores_bf16(q[b, h], kb[b, h // G, :N])
            assert np.array_equal(got[b, h].view(np.uint32), want.view(np.uint32)), (b, h)


def test_layer_with_bf16_key_cache():
    # The runner takes a bf16 k_r cache through rtp_index_scores_bf16: its
    # scores are the oracle's over the widened keys, bit for bit, and the
    # kept sets are the oracle's top-p sets of those scores.
    from sparse_long_context_indexer_amd.runner import DecodeLayer
    cfg = synth.CONFIGS[1]
    L = load_layer(cfg)
    kb = synth.f32_to_bf16(L.k_r)
    step = DecodeLayer(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.H_r, cfg.n_sink, cfg.window, dev())
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.float32, device=dev())
    step(L.d["q_r"], torch.from_numpy(kb.view(np.int16)).to(dev()), L.d["q"], L.d["K"],
         L.d["V"], 0.9, cfg.scale, out)
    torch.cuda.synchronize()
    sc, c, ix = step.scores.cpu().numpy(), step.count.cpu().numpy(), step.idx.cpu().numpy()
    G = cfg.H_r // cfg.G_r
    for b in range(cfg.B):
        for h in range(cfg.H_r):
            want = oracle.scores_bf16(L.q_r[b, h], kb[b, h // G, :cfg.N])
            assert np.array_equal(sc[b, h].view(np.uint32), want.view(np.uint32)), (b, h)
            v = judge_set(want, 0.9, ix[b, h, :c[b, h]])
            assert v.ok, (b, h, v.k_gpu, v.k_oracle)
    # The outputs: sparse heads against the oracle's attention over the
    # GPU's set, local heads over the sinks and window.
    got = out.cpu().numpy()
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            kv = h // cfg.G
            if h < cfg.H_r:
                rows = np.sort(ix[b, h, :c[b, h]])
            else:
                rows = oracle.local_rows(cfg.N, cfg.n_sink, cfg.window)
            ref = oracle.attention(L.q[b, h], L.kv_rows("K", b, kv, rows),
                                   L.kv_rows("V", b, kv, rows), cfg.scale)
            ok, err, rel = judge_out(got[b, h], ref)
            assert ok, (b, h, err, rel)
    # scan_local has no bf16 key path: the runner says so instead of
    # reading the keys as fp32.
    sl = DecodeLayer(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.H_r, cfg.n_sink, cfg.window, dev(),
                     mode="scan_local")
    with pytest.raises(ValueError, match="fp32"):
        sl(L.d["q_r"], torch.from_numpy(kb.view(np.int16)).to(dev()), L.d["q"], L.d["K"],
           L.d["V"], 0.9, cfg.scale, out)


# ----------------------------------------------------------------- prefill

@pytest.mark.parametrize("T,n_sink,window,hb,nh", [
    (1, 0, 0, 0, 8), (37, 0, 0, 2, 3), (300, 0, 0, 0, 8), (1000, 4, 64, 1, 6),
    (1000, 0, 1, 0, 8), (2000, 4, 300, 3, 5), (130, 17, 16, 0, 8)])
def test_prefill_attend_against_oracle(T, n_sink, window, hb, nh):
    # Dense (window 0) and sinks + window heads, GQA with 4 query heads per
    # KV head, a cache wider than T; sampled queries against the oracle's
    # attention over each query's rows, heads outside the range untouched.
    B, Hq, Hkv, cap = 2, 8, 2, T + 5
    q = synth.normal_bf16(synth.key(80 + T, 1), 0, B * Hq * T * 128).reshape(B, Hq, T, 128)
    K = synth.normal_bf16(synth.key(80 + T, 2), 0, B * Hkv * cap * 128).reshape(B, Hkv, cap, 128)
    V = synth.normal_bf16(synth.key(80 + T, 3), 0, B * Hkv * cap * 128).reshape(B, Hkv, cap, 128)
    scale = 1.0 / math.sqrt(128.0)
    out = torch.full((B, Hq, T, 128), float("nan"), dtype=torch.float32, device=dev())
    rtp.rtp_prefill_attend(torch.from_numpy(q.view(np.int16)).to(dev()),
                           torch.from_numpy(K.view(np.int16)).to(dev()),
                           torch.from_numpy(V.view(np.int16)).to(dev()), hb, nh, n_sink, window,
                           scale, out)
    got = out.cpu().numpy()
    rng = np.random.default_rng(T)
    ts = np.unique(np.concatenate([np.arange(min(T, 20)), np.arange(max(0, T - 20), T),
                                   rng.integers(0, T, 40)]))
    for b in range(B):
        for h in range(hb, hb + nh):
            for t in ts:
                rows = np.arange(t + 1) if window <= 0 else oracle.local_rows(t + 1, n_sink, window)
                ref = oracle.attention(q[b, h, t], K[b, h // 4, rows], V[b, h // 4, rows], scale)
                ok, err, rel = judge_out(got[b, h, t], ref)
                assert ok, (b, h, t, err, rel)
        outside = [h for h in range(Hq) if not hb <= h < hb + nh]
        assert np.all(np.isnan(got[b, outside]))


@pytest.mark.parametrize("scale_kind", ["negative", "zero"])
def test_prefill_attend_scale_sign(scale_kind):
    # A negative scale (the kernel flips Q's signs and uses |scale|) and a
    # zero scale (uniform weights over each query's keys), dense and sinks +
    # window heads, against the oracle.
    B, Hq, Hkv, T = 1, 8, 2, 300
    cap = T
    q = synth.normal_bf16(synth.key(91, 1), 0, B * Hq * T * 128).reshape(B, Hq, T, 128)
    K = synth.normal_bf16(synth.key(91, 2), 0, B * Hkv * cap * 128).reshape(B, Hkv, cap, 128)
    V = synth.normal_bf16(synth.key(91, 3), 0, B * Hkv * cap * 128).reshape(B, Hkv, cap, 128)
    scale = -1.0 / math.sqrt(128.0) if scale_kind == "negative" else 0.0
    out = torch.full((B, Hq, T, 128), float("nan"), dtype=torch.float32, device=dev())
    qd = torch.from_numpy(q.view(np.int16)).to(dev())
    Kd = torch.from_numpy(K.view(np.int16)).to(dev())
    Vd = torch.from_numpy(V.view(np.int16)).to(dev())
    rtp.rtp_prefill_attend(qd, Kd, Vd, 0, 4, 0, 0, scale, out)
    rtp.rtp_prefill_attend(qd, Kd, Vd, 4, 4, 3, 40, scale, out)
    got = out.cpu().numpy()
    for h in range(Hq):
        for t in (0, 1, 2, 39, 40, 41, 150, 299):
            rows = np.arange(t + 1) if h < 4 else oracle.local_rows(t + 1, 3, 40)
            ref = oracle.attention(q[0, h, t], K[0, h // 4, rows], V[0, h // 4, rows], scale)
            ok, err, rel = judge_out(got[0, h, t], ref)
            assert ok, (scale_kind, h, t, err, rel)


def test_prefill_attend_v_beyond_fp16():
    # V values of 2^16 and more (beyond fp16, in which the kernel stages V):
    # their dimension tiles are staged scaled by a power of two.  A tiny value
    # beside a large one in the same tile, dense and sinks + window heads,
    # every third query against the oracle: |err| <= 2e-3 + (2^-9 + 1e-5) *
    # sum_i w_i |v_i|.  The kernel rounds P to fp16 and normalises by the sum
    # of the rounded weights, so each output is an average of V rows under
    # weights within 2^-10 (relative) of the exact ones: the error scales with
    # the magnitude of V (the 1e-5 covers fp32 accumulation).
    B, Hq, Hkv, T = 1, 8, 2, 700
    q = synth.normal_bf16(synth.key(91, 1), 0, B * Hq * T * 128).reshape(B, Hq, T, 128)
    K = synth.normal_bf16(synth.key(91, 2), 0, B * Hkv * T * 128).reshape(B, Hkv, T, 128)
    V = synth.normal_bf16(synth.key(91, 3), 0, B * Hkv * T * 128).reshape(B, Hkv, T, 128)

    def bf(x):
        return np.uint16(np.array([x], np.float32).view(np.uint32)[0] >> 16)
    for g in range(Hkv):
        V[0, g, 70, 5] = bf(327680.0)        # 1.25 * 2^18
        V[0, g, 71, 6] = bf(2.0 ** -16)      # below fp16's normal range once scaled
        V[0, g, 300, 100] = bf(-2621440.0)   # -1.25 * 2^21
        V[0, g, 650, 40] = bf(69632.0)       # 1.0625 * 2^16
        V[0, g, 651, 41] = bf(65280.0)       # the largest bf16 below 2^16 (no scaling)
    scale = 1.0 / math.sqrt(128.0)
    out = torch.full((B, Hq, T, 128), float("nan"), dtype=torch.float32, device=dev())
    qd = torch.from_numpy(q.view(np.int16)).to(dev())
    Kd = torch.from_numpy(K.view(np.int16)).to(dev())
    Vd = torch.from_numpy(V.view(np.int16)).to(dev())
    rtp.rtp_prefill_attend(qd, Kd, Vd, 0, 4, 0, 0, scale, out)
    rtp.rtp_prefill_attend(qd, Kd, Vd, 4, 4, 4, 200, scale, out)
    got = out.cpu().numpy()
    Vabs = V & np.uint16(0x7FFF)
    worst = 0.0
    for h in range(Hq):
        g = h // 4
        for t in range(0, T, 3):
            rows = np.arange(t + 1) if h < 4 else oracle.local_rows(t + 1, 4, 200)
            ref = oracle.attention(q[0, h, t], K[0, g, rows], V[0, g, rows], scale)
            mag = oracle.attention(q[0, h, t], K[0, g, rows], Vabs[0, g, rows], scale)
            err = np.abs(got[0, h, t].astype(np.float64) - ref)
            bound = 2e-3 + (2.0 ** -9 + 1e-5) * mag
            assert np.all(err <= bound), (h, t, float(np.max(err - bound)))
            worst = max(worst, float(np.max(err / bound)))
    print(f"worst error / bound: {worst:.3g}")


def test_prefill_attend_v_tiny():
    # Every V value near 2^-20 (below fp16's normal range): the kernel stages
    # such dimension tiles scaled up by a power of two, so outputs keep their
    # relative precision.  Peaked softmax (scale 1), dense and sinks + window
    # heads, every fourth query against the oracle (max-abs 2e-3 and max-rel
    # 1e-2 of the row's largest output).
    B, Hq, Hkv, T = 1, 8, 2, 300
    q = synth.normal_bf16(synth.key(93, 1), 0, B * Hq * T * 128).reshape(B, Hq, T, 128)
    K = synth.normal_bf16(synth.key(93, 2), 0, B * Hkv * T * 128).reshape(B, Hkv, T, 128)
    V = synth.normal_bf16(synth.key(93, 3), 0, B * Hkv * T * 128).reshape(B, Hkv, T, 128)
    nz = (V & 0x7FFF) != 0
    V = np.where(nz, V - np.uint16(20 << 7), V).astype(np.uint16)  # exact scaling by 2^-20
    scale = 1.0
    out = torch.full((B, Hq, T, 128), float("nan"), dtype=torch.float32, device=dev())
    qd = torch.from_numpy(q.view(np.int16)).to(dev())
    Kd = torch.from_numpy(K.view(np.int16)).to(dev())
    Vd = torch.from_numpy(V.view(np.int16)).to(dev())
    rtp.rtp_prefill_attend(qd, Kd, Vd, 0, 4, 0, 0, scale, out)
    rtp.rtp_prefill_attend(qd, Kd, Vd, 4, 4, 4, 64, scale, out)
    got = out.cpu().numpy()
    worst = 0.0
    for h in range(Hq):
        for t in range(0, T, 4):
            rows = np.arange(t + 1) if h < 4 else oracle.local_rows(t + 1, 4, 64)
            ref = oracle.attention(q[0, h, t], K[0, h // 4, rows], V[0, h // 4, rows], scale)
            ok, err, rel = judge_out(got[0, h, t], ref)
            assert ok, (h, t, err, rel)
            worst = max(worst, rel)
    print(f"largest relative error: {worst:.3g} (bound 1e-2)")


def test_prefill_attend_benched_size():
    # The size the benchmark times: a 16384-token prompt, 32 query heads on
    # 4 KV heads, heads 0-7 dense and heads 8-31 on 4 sinks + a 4096-token
    # window, one launch each.  Sampled queries (the first ones, both sides
    # of the window edge, random ones, the last ones) against the oracle.
    B, Hq, Hkv, T = 1, 32, 4, 16384
    H_r, n_sink, window = 8, 4, 4096
    cap = T + 3
    q = synth.normal_bf16(synth.key(86, 1), 0, B * Hq * T * 128).reshape(B, Hq, T, 128)
    K = synth.normal_bf16(synth.key(86, 2), 0, B * Hkv * cap * 128).reshape(B, Hkv, cap, 128)
    V = synth.normal_bf16(synth.key(86, 3), 0, B * Hkv * cap * 128).reshape(B, Hkv, cap, 128)
    scale = 1.0 / math.sqrt(128.0)
    out = torch.full((B, Hq, T, 128), float("nan"), dtype=torch.float32, device=dev())
    qd = torch.from_numpy(q.view(np.int16)).to(dev())
    Kd = torch.from_numpy(K.view(np.int16)).to(dev())
    Vd = torch.from_numpy(V.view(np.int16)).to(dev())
    rtp.rtp_prefill_attend(qd, Kd, Vd, 0, H_r, 0, 0, scale, out)
    rtp.rtp_prefill_attend(qd, Kd, Vd, H_r, Hq - H_r, n_sink, window, scale, out)
    rng = np.random.default_rng(16384)
    ts = np.unique(np.concatenate([np.arange(5), np.arange(window - 3, window + 3),
                                   rng.integers(0, T, 8), np.arange(T - 4, T)]))
    heads = [0, 3, 7, 8, 19, 31]
    worst = 0.0
    got = out[:, heads][:, :, torch.from_numpy(ts).to(dev())].cpu().numpy()
    assert not torch.isnan(out).any().item()
    del out
    for b in range(B):
        for hi, h in enumerate(heads):
            for ti, t in enumerate(ts):
                rows = (np.arange(t + 1) if h < H_r
                        else oracle.local_rows(t + 1, n_sink, window))
                ref = oracle.attention(q[b, h, t], K[b, h // 8, rows], V[b, h // 8, rows], scale)
                ok, err, rel = judge_out(got[b, hi, ti], ref)
                assert ok, (b, h, t, err, rel)
                worst = max(worst, err)
    print(f"largest abs error: {worst:.3g} (bound 2e-3)")


# -------------------------------------------------------------- projection

# fp32 accumulation of d exact products in any order: the error stays within
# d * 2u * sum |terms| (u = 2^-24; 2u also covers a truncating adder).
PROJ_REL = 2 * 128 * 2.0 ** -24


def _proj_inputs(B, Hx, x_cap, H, seed):
    x = synth.normal_bf16(synth.key(seed, 1), 0, B * Hx * x_cap * 128).reshape(B, Hx, x_cap, 128)
    W = synth.bf16_to_f32(synth.normal_bf16(synth.key(seed, 2), 0, H * 16 * 128)) / 16.0
    return x, synth.f32_to_bf16(W).reshape(H, 16, 128)   # W / 16 is exact in bf16


def _proj_gpu(x, W, out_cap, hb, T, pos, sentinel=-3.5):
    B, Hx, x_cap, _ = x.shape
    H = W.shape[0]
    out = torch.full((B, H, out_cap, 16), sentinel, dtype=torch.float32, device=dev())
    rtp.rtp_index_project(torch.from_numpy(x.view(np.int16)).to(dev()),
                          torch.from_numpy(W.view(np.int16)).to(dev()), out,
                          head_begin=hb, T=T, out_pos=pos)
    return out.cpu().numpy()


def _assert_proj(x, W, got, hb, T, pos, sentinel=-3.5):
    B, H = got.shape[:2]
    xf = synth.bf16_to_f32(x).astype(np.float64)
    Wf = synth.bf16_to_f32(W).astype(np.float64)
    for b in range(B):
        for h in range(H):
            want = oracle.project(x[b, hb + h, :T], W[h])
            bound = PROJ_REL * (np.abs(xf[b, hb + h, :T]) @ np.abs(Wf[h]).T) + 1e-30
            rows = got[b, h, pos:pos + T].astype(np.float64)
            assert np.all(np.abs(rows - want) <= bound), (b, h, np.max(np.abs(rows - want) / bound))
            assert np.all(got[b, h, :pos] == sentinel) and np.all(got[b, h, pos + T:] == sentinel)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 255, 256, 257, 4097])
def test_project_shapes(T):
    # Heads 1..3 of 5, caches wider than T, rows written at an offset.
    x, W = _proj_inputs(2, 5, T + 3, 3, 60 + T)
    for pos in (0, 7):
        got = _proj_gpu(x, W, T + 9, 1, T, pos)
        _assert_proj(x, W, got, 1, T, pos)


def test_project_append_matches_prefill_bits():
    # The k_r row of token n is the same whether it is projected within a
    # prefill of n + 1 tokens or appended alone at row n, and q_r of decode
    # heads takes the same path with one-row caches.
    n = 1000
    x, W = _proj_inputs(2, 4, n + 1, 2, 70)
    full = _proj_gpu(x, W, n + 1, 2, n + 1, 0)
    head = _proj_gpu(np.ascontiguousarray(x[:, :, :n]), W, n + 1, 2, n, 0, sentinel=0.0)
    last = _proj_gpu(np.ascontiguousarray(x[:, :, n:n + 1]), W, n + 1, 2, 1, n, sentinel=0.0)
    assert np.array_equal(full[:, :, :n], head[:, :, :n])
    assert np.array_equal(full[:, :, n], last[:, :, n])
    _assert_proj(x, W, full, 2, n + 1, 0)
    q, Wq = _proj_inputs(1, 32, 1, 8, 71)            # 8 retrieval query heads of 32
    _assert_proj(q, Wq, _proj_gpu(q, Wq, 1, 0, 1, 0), 0, 1, 0)


def test_project_prefill_1m_sampled():
    # The prefill k_r build at 2^20 tokens (one KV head), checked on sampled
    # rows; the whole output is checked finite and the rows past T untouched.
    N = 1 << 20
    x, W = _proj_inputs(1, 1, N, 1, 72)
    got = _proj_gpu(x, W, N + 5, 0, N, 0)
    assert np.all(got[0, 0, N:] == -3.5) and np.all(np.isfinite(got[0, 0, :N]))
    rows = np.concatenate([np.arange(32), np.random.default_rng(73).choice(N, 4000), N - 32 + np.arange(32)])
    want = oracle.project(x[0, 0, rows], W[0])
    bound = PROJ_REL * (np.abs(synth.bf16_to_f32(x[0, 0, rows]).astype(np.float64))
                        @ np.abs(synth.bf16_to_f32(W[0]).astype(np.float64)).T) + 1e-30
    assert np.all(np.abs(got[0, 0, rows].astype(np.float64) - want) <= bound)


# ------------------------------------------------------------------ top-k

def _select_k(scores: np.ndarray, k: int, keep_bits=False):
    B, H, N = scores.shape
    sd = to_dev(scores.astype(np.float32))
    idx = torch.full((B, H, N), -7, dtype=torch.int32, device=dev())
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=dev())
    kb = (torch.full((B, H, rtp.keep_words(N)), -1, dtype=torch.int32, device=dev())
          if keep_bits else None)
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, B, H, N), dtype=torch.uint8,
                     device=dev())
    rtp.rtp_topk_select(sd, k, idx, cnt, ws, keep_bits=kb)
    c = cnt.cpu().numpy()
    ix = idx.cpu().numpy()
    sets = [[ix[b, h, :c[b, h]] for h in range(H)] for b in range(B)]
    return sets, c, (kb.cpu().numpy() if keep_bits else None)


def _assert_topk(scores, k, keep_bits=False):
    sets, c, kb = _select_k(scores, k, keep_bits)
    B, H, N = scores.shape
    for b in range(B):
        for h in range(H):
            want = oracle.topk(scores[b, h], k)
            got = sets[b][h]
            assert c[b, h] == min(k, N), (b, h, k, c[b, h])
            assert np.array_equal(np.sort(got), np.sort(want)), (b, h, k)
            if kb is not None:
                bits = np.unpackbits(kb[b, h].view(np.uint8), bitorder="little")[:N]
                assert np.array_equal(np.flatnonzero(bits), np.sort(want)), (b, h, k)


@pytest.mark.parametrize("N", [1, 13, 4096, 70_001])
def test_topk_random_rows(N):
    rng = np.random.default_rng(31 + N)
    s = (rng.standard_normal((2, 3, N)) * rng.choice([0.5, 3.0])).astype(np.float32)
    for k in sorted({1, 2, max(1, N // 7), max(1, N - 1), N, N + 3}):
        _assert_topk(s, k, keep_bits=(k == 2))


def test_topk_ties_and_signed_zeros():
    rng = np.random.default_rng(37)
    s = np.round(rng.standard_normal((2, 3, 50_000)) * 2).astype(np.float32)
    s[0, 0, ::3] = -0.0
    s[1, 2, :] = 0.0                       # one score everywhere
    s[0, 1, rng.integers(0, 50_000, 300)] = np.float32(9.0)
    for k in (1, 17, 64, 65, 300, 4099, 49_999):
        _assert_topk(s, k)


def test_topk_many_chunks_and_boundary_groups():
    # 28 chunks of 32768 scores per row, and k falling inside groups of
    # equal scores of either side of one wave.
    rng = np.random.default_rng(41)
    B, H, N = 1, 4, 900_000
    s = (rng.standard_normal((B, H, N)) * 2).astype(np.float32)
    s[0, 1, :] = np.round(s[0, 1, :] * 4) / 4
    s[0, 2, rng.choice(N, 100, replace=False)] = np.float32(7.0)
    s[0, 3, rng.choice(N, 3000, replace=False)] = np.float32(7.0)
    for k in (50, 2048, 12_345, 123_456):
        _assert_topk(s, k)


def test_topk_two_launch_path():
    rng = np.random.default_rng(43)
    s = (rng.standard_normal((1, 40000, 96)) * 3).astype(np.float32)
    s[0, ::3, ::5] = np.float32(1.25)
    sets, c, _ = _select_k(s, 30)
    assert np.all(c == 30)
    for h in range(0, 40000, 7):
        assert np.array_equal(np.sort(sets[0][h]), np.sort(oracle.topk(s[0, h], 30))), h


def test_topk_at_the_top_p_budget_keeps_the_top_p_set():
    # With k set to each row's top-p count, the two selectors keep the same
    # tokens (top-p keeps a prefix of the same order).
    cfg = synth.CONFIGS[2].with_(N=65536)
    q_r, k_r = synth.layer_qr(cfg, 0), synth.layer_kr(cfg, 0)
    s = np.stack([[oracle.scores(q_r[b, h], k_r[b, 0]) for h in range(2)] for b in range(2)])
    sets_p, c_p = _select(s, 0.9)
    for b in range(2):
        for h in range(2):
            row = np.ascontiguousarray(s[b:b + 1, h:h + 1])
            sets_k, c_k, _ = _select_k(row, int(c_p[b, h]))
            assert np.array_equal(np.sort(sets_k[0][0]), np.sort(sets_p[b][h])), (b, h)
            assert np.array_equal(np.sort(sets_k[0][0]),
                                  np.sort(oracle.topk(s[b, h], int(c_p[b, h]))))


# -------------------------------------------------------- attention edges

def test_sparse_single_row_is_value_row():
    cfg = synth.CONFIGS[0].with_(N=300)
    L = load_layer(cfg)
    for t in (0, 299):
        idx = torch.full((1, 1, 300), t, dtype=torch.int32, device=dev())
        cnt = torch.ones((1, 1), dtype=torch.int32, device=dev())
        out = torch.zeros((1, 1, 128), dtype=torch.float32, device=dev())
        ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_SPARSE_DECODE, 1, 1, 300),
                         dtype=torch.uint8, device=dev())
        rtp.rtp_sparse_decode(L.d["q"], L.d["K"], L.d["V"], idx, cnt, 0, cfg.scale, out, ws)
        want = synth.bf16_to_f32(L.V[0, 0, t])
        assert np.array_equal(out.cpu().numpy()[0, 0], want)


def test_sparse_p_one_equals_dense():
    cfg = synth.CONFIGS[1].with_(N=5000)
    L = load_layer(cfg)
    res = run_layer(L, 1.0)
    for h in range(cfg.H_r):
        assert res["count"][0, h] == cfg.N
        ref = oracle.attention(L.q[0, h], L.K[0, 0], L.V[0, 0], cfg.scale)
        ok, err, rel = judge_out(res["out"][0, h], ref)
        assert ok, (h, err, rel)


@pytest.mark.parametrize("N,n_sink,window", [
    (1, 4, 4096), (3, 4, 4096), (4100, 4, 4096), (4101, 4, 4096), (9000, 0, 4096),
    (9000, 4, 1), (20000, 17, 333)])
def test_local_edges(N, n_sink, window):
    cfg = synth.CONFIGS[1].with_(N=N, n_sink=n_sink, window=window, B=2, needles_per_head=0)
    L = load_layer(cfg)
    out = torch.full((2, 32, 128), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, 2, 24, N), dtype=torch.uint8,
                     device=dev())
    rtp.rtp_local_decode(L.d["q"], L.d["K"], L.d["V"], N, 8, 24, n_sink, window, cfg.scale,
                         out, ws)
    got = out.cpu().numpy()
    rows = oracle.local_rows(N, n_sink, window)
    for b in range(2):
        for h in range(8, 32):
            ref = oracle.attention(L.q[b, h], L.K[b, h // 8, rows], L.V[b, h // 8, rows],
                                   cfg.scale)
            ok, err, rel = judge_out(got[b, h], ref)
            assert ok, (b, h, err, rel)
        assert np.all(np.isnan(got[b, :8]))  # heads outside the range untouched


@pytest.mark.parametrize("N,n_sink,window", [
    (3, 4, 4096), (4100, 4, 4096), (4101, 4, 4096), (9000, 0, 4096), (9000, 4, 1),
    (20000, 17, 333)])
def test_local_ring_cache_matches_linear(N, n_sink, window):
    # A ring cache holding the tokens a local head can still see (every
    # other token's slot has been overwritten by a newer one) gives the
    # linear cache's result bit for bit, and the oracle's.
    cfg = synth.CONFIGS[1].with_(N=N, n_sink=n_sink, window=window, B=2, needles_per_head=0)
    L = load_layer(cfg)
    ring = min(N, n_sink + window)
    live = oracle.local_rows(N, n_sink, window)
    slot = np.where(live < n_sink, live, n_sink + (live - n_sink) % window)
    assert len(np.unique(slot)) == len(live) and slot.max() < ring
    Kr = np.zeros((2, L.K.shape[1], ring, 128), np.uint16)
    Vr = np.zeros_like(Kr)
    Kr[:, :, slot] = L.K[:, :, live]
    Vr[:, :, slot] = L.V[:, :, live]
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, 2, 24, N), dtype=torch.uint8,
                     device=dev())
    lin = torch.full((2, 32, 128), float("nan"), dtype=torch.float32, device=dev())
    rtp.rtp_local_decode(L.d["q"], L.d["K"], L.d["V"], N, 8, 24, n_sink, window, cfg.scale,
                         lin, ws)
    out = torch.full((2, 32, 128), float("nan"), dtype=torch.float32, device=dev())
    rtp.rtp_local_decode_ring(L.d["q"], torch.from_numpy(Kr.view(np.int16)).to(dev()),
                              torch.from_numpy(Vr.view(np.int16)).to(dev()), N, 8, 24, n_sink,
                              window, cfg.scale, out, ws)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), lin.cpu().numpy().view(np.uint32))
    rows = oracle.local_rows(N, n_sink, window)
    for h in (8, 31):
        ref = oracle.attention(L.q[1, h], L.K[1, h // 8, rows], L.V[1, h // 8, rows], cfg.scale)
        ok, err, rel = judge_out(got[1, h], ref)
        assert ok, (h, err, rel)


def test_local_unaligned_head_range():
    # Heads 5..13 with 4 query heads per KV head: partial groups at both ends.
    cfg = synth.CONFIGS[1].with_(N=6000, Hq=16, Hkv=4, H_r=0, needles_per_head=0)
    L = load_layer(cfg)
    out = torch.full((1, 16, 128), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, 1, 9, 6000), dtype=torch.uint8,
                     device=dev())
    rtp.rtp_local_decode(L.d["q"], L.d["K"], L.d["V"], 6000, 5, 9, 4, 4096, cfg.scale, out, ws)
    got = out.cpu().numpy()
    rows = oracle.local_rows(6000, 4, 4096)
    for h in range(16):
        if 5 <= h < 14:
            ref = oracle.attention(L.q[0, h], L.K[0, h // 4, rows], L.V[0, h // 4, rows],
                                   cfg.scale)
            ok, err, rel = judge_out(got[0, h], ref)
            assert ok, (h, err, rel)
        else:
            assert np.all(np.isnan(got[0, h]))


@pytest.mark.parametrize("sets", ["local_only", "sparse_only", "both_unaligned"])
def test_decode_attend_head_sets(sets):
    # rtp_decode_attend with one set empty, and with head ranges that cut
    # KV groups (4 query heads per KV head: heads 1..6 sparse, 7..14 local).
    cfg = synth.CONFIGS[1].with_(N=9000, Hq=16, Hkv=4, H_r=0, needles_per_head=0)
    L = load_layer(cfg)
    N = cfg.N
    sb, ns, lb, nl = {"local_only": (0, 0, 3, 11), "sparse_only": (2, 9, 0, 0),
                      "both_unaligned": (1, 6, 7, 8)}[sets]
    rng = np.random.default_rng(11)
    idx = torch.zeros((1, max(ns, 1), N), dtype=torch.int32)
    count = torch.zeros((1, max(ns, 1)), dtype=torch.int32)
    picks = []
    for k in range(ns):
        c = int(rng.integers(1, 3000))
        sel = np.sort(rng.choice(N, c, replace=False))
        idx[0, k, :c] = torch.from_numpy(sel.astype(np.int32))
        count[0, k] = c
        picks.append(sel)
    out = torch.full((1, 16, 128), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_DECODE_ATTEND, 1, 16, N), dtype=torch.uint8,
                     device=dev())
    rtp.rtp_decode_attend(L.d["q"], L.d["K"], L.d["V"],
                          idx.to(dev()) if ns else None, count.to(dev()) if ns else None, N,
                          sb, lb, nl, 4, 4096, cfg.scale, out, ws)
    got = out.cpu().numpy()
    rows = oracle.local_rows(N, 4, 4096)
    for h in range(16):
        if sb <= h < sb + ns:
            sel = picks[h - sb]
            ref = oracle.attention(L.q[0, h], L.K[0, h // 4, sel], L.V[0, h // 4, sel], cfg.scale)
        elif lb <= h < lb + nl:
            ref = oracle.attention(L.q[0, h], L.K[0, h // 4, rows], L.V[0, h // 4, rows],
                                   cfg.scale)
        else:
            assert np.all(np.isnan(got[0, h])), h
            continue
        ok, err, rel = judge_out(got[0, h], ref)
        assert ok, (sets, h, err, rel)


@pytest.mark.parametrize("N,Hq_r,Hkv_r,Hq,Hkv,lb,nl,n_sink,window", [
    (1, 8, 1, 32, 4, 8, 24, 4, 4096),        # one token
    (4101, 8, 1, 32, 4, 8, 24, 4, 4096),     # window + sinks + 1
    (9000, 12, 1, 16, 4, 5, 9, 0, 333),      # 12 heads per KV group; cut KV groups
    (70001, 3, 3, 8, 2, 1, 7, 17, 20000),    # 1 head per group, ragged tiles
    (2049, 16, 2, 8, 8, 0, 8, 2, 1)])        # 8 heads per group; window of one row
def test_scan_local_shapes(N, Hq_r, Hkv_r, Hq, Hkv, lb, nl, n_sink, window):
    # The scan and the local heads in one launch: scores bit-exact, local
    # outputs against the oracle's attention, heads outside the range untouched.
    B = 2
    cfg = synth.CONFIGS[1].with_(N=N, B=B, Hq=Hq, Hkv=Hkv, H_r=0, needles_per_head=0,
                                 n_sink=n_sink, window=window)
    L = load_layer(cfg)
    k = synth.key(91, synth.KR, N, B, Hq_r)
    q_r = synth.normal_f32(k, 0, B * Hq_r * 16).reshape(B, Hq_r, 16) * 3
    cap = N + 5
    k_r = synth.normal_f32(k, 10**9, B * Hkv_r * cap * 16).reshape(B, Hkv_r, cap, 16)
    k_r[..., ::5, 7] = 0.0
    s = torch.full((B, Hq_r, N), float("nan"), device=dev())
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, B, nl, N), dtype=torch.uint8,
                     device=dev())
    ws.fill_(0xA5)
    rtp.rtp_scan_local(to_dev(q_r.astype(np.float32)), to_dev(k_r), s, L.d["q"], L.d["K"],
                       L.d["V"], N, lb, nl, n_sink, window, cfg.scale, out, ws)
    got = s.cpu().numpy()
    G = Hq_r // Hkv_r
    for b in range(B):
        for h in range(Hq_r):
            ref = oracle.scores(q_r[b, h].astype(np.float32), k_r[b, h // G, :N])
            assert np.array_equal(got[b, h].view(np.uint32), ref.view(np.uint32)), (b, h)
    o = out.cpu().numpy()
    rows = oracle.local_rows(N, n_sink, window)
    Gq = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            if lb <= h < lb + nl:
                ref = oracle.attention(L.q[b, h], L.K[b, h // Gq, rows], L.V[b, h // Gq, rows],
                                       cfg.scale)
                ok, err, rel = judge_out(o[b, h], ref)
                assert ok, (b, h, err, rel)
            else:
                assert np.all(np.isnan(o[b, h])), (b, h)


# ---------------------------------------------------------------- graphs

@pytest.mark.parametrize("mode", ["fused", "union"])
def test_graph_replays_match_eager(mode):
    # One decode layer (and a top-k select, and a projection) captured as a
    # HIP graph and replayed several times, with eager work on other inputs
    # and host synchronisations between replays: every replay gives the
    # eager run's scores and counts bit for bit, the same kept sets, and the
    # same outputs up to the order of the kept rows.
    from sparse_long_context_indexer_amd.runner import DecodeLayer
    cfg = synth.CONFIGS[1]
    L = load_layer(cfg)
    step = DecodeLayer(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.H_r, cfg.n_sink, cfg.window, dev(),
                       mode=mode)
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.float32, device=dev())
    tk_idx = torch.empty_like(step.idx)
    tk_cnt = torch.empty_like(step.count)
    x = torch.from_numpy(synth.normal_bf16(synth.key(90, 1), 0, 4 * 300 * 128)
                         .reshape(1, 4, 300, 128).view(np.int16)).to(dev())
    Wp = torch.from_numpy(synth.normal_bf16(synth.key(90, 2), 0, 4 * 16 * 128)
                          .reshape(4, 16, 128).view(np.int16)).to(dev())
    pr = torch.empty((1, 4, 300, 16), dtype=torch.float32, device=dev())

    def issue():
        step(L.d["q_r"], L.d["k_r"], L.d["q"], L.d["K"], L.d["V"], 0.9, cfg.scale, out)
        rtp.rtp_topk_select(step.scores, 777, tk_idx, tk_cnt, step.ws_sel)
        rtp.rtp_index_project(x, Wp, pr)

    def snap():
        torch.cuda.synchronize()
        c, ix = step.count.cpu().numpy(), step.idx.cpu().numpy()
        tc, tix = tk_cnt.cpu().numpy(), tk_idx.cpu().numpy()
        return (out.cpu().numpy(), step.scores.cpu().numpy(), c,
                [np.sort(ix[b, h, :c[b, h]]) for b in range(cfg.B) for h in range(cfg.H_r)],
                [np.sort(tix[b, h, :tc[b, h]]) for b in range(cfg.B) for h in range(cfg.H_r)],
                pr.cpu().numpy())

    issue()
    ref = snap()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        issue()
    other = torch.empty((2, 3, 50_000), dtype=torch.float32, device=dev())
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        got = snap()
        assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2]), rep
        assert all(np.array_equal(a_, b_) for a_, b_ in zip(got[3], ref[3])), rep
        assert all(np.array_equal(a_, b_) for a_, b_ in zip(got[4], ref[4])), rep
        assert np.array_equal(got[5], ref[5]), rep
        assert np.allclose(got[0], ref[0], rtol=1e-5, atol=1e-6), rep
        # eager work between replays: a selection on other scores (another
        # shape) in the graph's own select workspace, judged against the
        # oracle; the next replay must not care
        other.normal_()
        o_np = other.cpu().numpy()
        e_idx = torch.full((2, 3, 50_000), -7, dtype=torch.int32, device=dev())
        e_cnt = torch.full((2, 3), -7, dtype=torch.int32, device=dev())
        rtp.rtp_topp_select(other, 0.5, e_idx, e_cnt, step.ws_sel)
        torch.cuda.synchronize()
        ec, eix = e_cnt.cpu().numpy(), e_idx.cpu().numpy()
        for b in range(2):
            for h in range(3):
                v = judge_set(o_np[b, h], 0.5, eix[b, h, :ec[b, h]])
                assert v.ok, (rep, b, h, v.k_gpu, v.k_oracle, v.bad[:5], v.note)


# ------------------------------------------------------------ workspaces
# ------------------------------------------------------------ workspaces

@pytest.mark.parametrize("mode", ["fused", "scan_local", "per_head", "union"])
def test_workspace_garbage_and_reuse(mode):
    # Workspaces start as arbitrary bytes (no initialisation is required),
    # are reused by the next call, and are then reused for a smaller call
    # whose layout differs.
    from sparse_long_context_indexer_amd.runner import DecodeLayer
    cfg = synth.CONFIGS[1]
    L = load_layer(cfg)
    step = DecodeLayer(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.H_r, cfg.n_sink, cfg.window, dev(),
                       mode=mode)
    g = torch.Generator(device="cpu").manual_seed(7)
    if step.keep_bits is not None:
        step.keep_bits.copy_(torch.randint(-2**31, 2**31 - 1, step.keep_bits.shape,
                                           dtype=torch.int32, generator=g))
    wss = [step.ws_sel, step.ws_sparse, step.ws_local]
    if mode in ("fused", "scan_local"):
        wss.append(step.ws_attend)
    for ws in wss:
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=g))
    for rep in range(2):
        _print(f"full-size call {rep}")
        res = run_layer(L, 0.9, step=step)
        fails = check_layer(L, 0.9, res)
        assert not fails, "\n".join(fails[:20])
    small = cfg.with_(N=20000, B=1)
    Ls = load_layer(small)
    s2 = DecodeLayer(1, cfg.Hq, cfg.Hkv, 20000, cfg.H_r, cfg.n_sink, cfg.window, dev(),
                     mode=mode)
    s2.ws_sparse, s2.ws_local, s2.ws_sel = step.ws_sparse, step.ws_local, step.ws_sel
    if mode in ("fused", "scan_local"):
        s2.ws_attend = step.ws_attend
    for ws in wss[1:]:
        ws[ws.numel() // 3:].fill_(0xFF)
    for rep in range(2):
        _print(f"smaller call {rep} on the same workspaces")
        res = run_layer(Ls, 0.9, step=s2)
        fails = check_layer(Ls, 0.9, res)
        assert not fails, "\n".join(fails[:20])


# ------------------------------------------------------------- union mode

@pytest.mark.parametrize("N,n_sink,window", [(5000, 4, 4096), (70_001, 4, 4096),
                                              (70_001, 0, 31), (100, 7, 50)])
def test_retrieval_heads_with_sinks_and_window(N, n_sink, window):
    # The variant where retrieval heads attend their top-p set plus the local
    # rows: the bitmap after the local bits are added is exactly S u local,
    # and union attention over it matches the oracle over that set.
    cfg = synth.CONFIGS[1].with_(N=N, needles_per_head=0)
    L = load_layer(cfg)
    H_r = 8
    sc = torch.empty((1, H_r, N), dtype=torch.float32, device=dev())
    rtp.rtp_index_scores(L.d["q_r"], L.d["k_r"], sc)
    idx = torch.empty((1, H_r, N), dtype=torch.int32, device=dev())
    cnt = torch.empty((1, H_r), dtype=torch.int32, device=dev())
    kb = torch.empty((1, H_r, rtp.keep_words(N)), dtype=torch.int32, device=dev())
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, 1, H_r, N), dtype=torch.uint8,
                     device=dev())
    rtp.rtp_topp_select(sc, 0.9, idx, cnt, ws, keep_bits=kb)
    rtp.rtp_keep_bits_add_local(kb, N, n_sink, window)
    out = torch.full((1, cfg.Hq, 128), float("nan"), dtype=torch.float32, device=dev())
    wsu = torch.empty(rtp.workspace_size(rtp.RTP_WS_SPARSE_UNION, 1, H_r, N), dtype=torch.uint8,
                      device=dev())
    rtp.rtp_sparse_decode_union(L.d["q"], L.d["K"], L.d["V"], kb, N, 0, cfg.scale, out, wsu)
    got, bits = out.cpu().numpy(), kb.cpu().numpy()
    c, ix = cnt.cpu().numpy(), idx.cpu().numpy()
    local = oracle.local_rows(N, n_sink, window)
    for h in range(H_r):
        rows = np.union1d(ix[0, h, :c[0, h]], local)
        have = np.flatnonzero(np.unpackbits(bits[0, h].view(np.uint8), bitorder="little")[:N])
        assert np.array_equal(have, rows), h
        ref = oracle.attention(L.q[0, h], L.K[0, h // 8, rows], L.V[0, h // 8, rows], cfg.scale)
        ok, err, rel = judge_out(got[0, h], ref)
        assert ok, (h, err, rel)


@pytest.mark.parametrize("N,hb,nq", [(70001, 0, 8), (5000, 3, 8), (33, 0, 8), (100000, 4, 12)])
def test_union_decode_random_sets(N, hb, nq):
    # Keep bitmaps built on the host (random densities per head, stray bits
    # past N in the last word, head ranges across KV heads), against the
    # oracle's attention over each head's set.
    cfg = synth.CONFIGS[1].with_(N=N, needles_per_head=0)
    L = load_layer(cfg)
    rng = np.random.default_rng(N + hb)
    words = (N + 31) // 32
    kb = np.zeros((1, nq, words), dtype=np.uint32)
    sets = []
    for i in range(nq):
        dens = [0.001, 0.05, 0.5, 1.0][i % 4]
        sel = np.flatnonzero(rng.random(N) < dens)
        if len(sel) == 0:
            sel = np.array([rng.integers(N)])
        bits = np.zeros(words * 32, dtype=np.uint8)
        bits[sel] = 1
        bits[N:] = 1  # past the end: must be ignored
        kb[0, i] = np.packbits(bits, bitorder="little").view("<u4")
        sets.append(sel)
    out = torch.full((1, cfg.Hq, 128), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_SPARSE_UNION, 1, nq, N), dtype=torch.uint8,
                     device=dev())
    ws.fill_(0xA5)
    kbt = torch.from_numpy(kb.view(np.int32)).to(dev())
    for rep in range(2):
        rtp.rtp_sparse_decode_union(L.d["q"], L.d["K"], L.d["V"], kbt, N, hb, cfg.scale, out, ws)
        got = out.cpu().numpy()
        for i in range(nq):
            h = hb + i
            ref = oracle.attention(L.q[0, h], L.K[0, h // 8, sets[i]], L.V[0, h // 8, sets[i]],
                                   cfg.scale)
            ok, err, rel = judge_out(got[0, h], ref)
            assert ok, (rep, h, len(sets[i]), err, rel)
        outside = [h for h in range(cfg.Hq) if not hb <= h < hb + nq]
        assert np.all(np.isnan(got[0, outside]))


def test_union_single_row_is_value_row():
    cfg = synth.CONFIGS[1].with_(N=300, needles_per_head=0)
    L = load_layer(cfg)
    for t in (0, 31, 32, 299):
        kb = np.zeros((1, 8, 10), dtype=np.uint32)
        kb[0, :, t // 32] = np.uint32(1) << np.uint32(t % 32)
        out = torch.zeros((1, 32, 128), dtype=torch.float32, device=dev())
        ws = torch.empty(rtp.workspace_size(rtp.RTP_WS_SPARSE_UNION, 1, 8, 300),
                         dtype=torch.uint8, device=dev())
        rtp.rtp_sparse_decode_union(L.d["q"], L.d["K"], L.d["V"],
                                    torch.from_numpy(kb.view(np.int32)).to(dev()), 300, 0,
                                    cfg.scale, out, ws)
        got = out.cpu().numpy()
        want = synth.bf16_to_f32(L.V[0, 0, t])
        for h in range(8):
            assert np.array_equal(got[0, h], want), (t, h)
