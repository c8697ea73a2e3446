"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks the oracle against one of: a hand-derived closed form
(tests/golden/closed_forms.json), brute force over all subsets on tiny
inputs, a library routine it reduces to (torch's scaled-dot-product attention
in fp64), or an invariant of the definition (nesting in p, permutation
equivariance, mass bounds).  Chosen so that a dropped term, a wrong sign or
index, a wrong tie rule or a transposed operand fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _f(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


# ------------------------------------------------------------------ scores

def test_scores_closed_forms(golden):
    for case in golden["scores"]:
        q = np.array([_f(x) for x in case["q"]], np.float32)
        k = np.array([_f(x) for x in case["k"]], np.float32).reshape(1, 16)
        s = oracle.scores(q, k)[0]
        want = np.float32(_f(case["expected"]))
        assert s.view(np.uint32) == want.view(np.uint32), case["name"]


def test_scores_exact_integer_dots_match_float64():
    # Small integer operands: every fp32 fma is exact, so the score equals
    # the exact dot product computed by numpy in float64.
    rng = np.random.default_rng(11)
    q = rng.integers(-50, 51, size=16).astype(np.float32)
    k = rng.integers(-50, 51, size=(257, 16)).astype(np.float32)
    s = oracle.scores(q, k)
    exact = k.astype(np.float64) @ q.astype(np.float64)
    assert np.array_equal(s.astype(np.float64), exact)


def test_scores_rows_are_independent_and_zero_is_positive():
    q = np.zeros(16, np.float32)
    k = np.random.default_rng(0).standard_normal((33, 16)).astype(np.float32)
    s = oracle.scores(q, k)
    assert np.all(s.view(np.uint32) == 0)  # +0, never -0
    q = np.eye(16, dtype=np.float32)[3] * 2.0
    s = oracle.scores(q, k)
    assert np.array_equal(s, (2.0 * k[:, 3]).astype(np.float32))


# ------------------------------------------------------------------ top-p

def _golden_scores(spec):
    if "fill" in spec:
        return np.full(spec["n"], spec["fill"], np.float32)
    return np.array([_f(v) for v in spec["values"]], np.float32)


def test_topp_closed_forms(golden):
    for case in golden["topp"]:
        s = _golden_scores(case["scores"])
        r = oracle.topp(s, case["p"])
        assert r.k == case["expected_k"], case["name"]
        es = case["expected_set"]
        want = (np.arange(*es["range"]) if "range" in es else np.array(es["values"]))
        assert np.array_equal(np.sort(r.sel), np.sort(want)), case["name"]


def _brute_force_min_k(s, p):
    """Smallest subset size whose exact mass reaches p*Z, by enumeration."""
    n = len(s)
    m = max(float(x) for x in s)
    e = [math.exp(float(x) - m) for x in s]
    Z = math.fsum(e)
    target = float(np.float32(p)) * Z
    best_mass = {}
    for size in range(1, n + 1):
        best = max(math.fsum(e[i] for i in c)
                   for c in itertools.combinations(range(n), size))
        best_mass[size] = best
        if best >= target:
            return size, best_mass, e, Z
    return n, best_mass, e, Z


@pytest.mark.parametrize("seed", range(12))
def test_topp_minimal_by_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 13))
    s = (rng.standard_normal(n) * rng.choice([0.3, 1.0, 3.0])).astype(np.float32)
    for p in (0.5, 0.8, 0.9, 0.95, 0.99):
        r = oracle.topp(s, p)
        k_bf, best, e, Z = _brute_force_min_k(s, p)
        assert r.k == k_bf, (seed, p)
        target = float(np.float32(p)) * Z
        # the oracle's set reaches p and is a heaviest set of its size
        mass = math.fsum(e[i] for i in r.sel)
        assert mass >= target * (1 - 1e-15)
        assert math.isclose(mass, best[r.k], rel_tol=1e-14)
        # no set one smaller reaches p
        if r.k > 1:
            assert best[r.k - 1] < target * (1 + 1e-15)


def test_topp_ties_go_to_lower_index():
    # Three equal top scores; p needs exactly two of them.
    s = np.array([0.0, 9.0, 1.0, 9.0, 9.0, 0.0], np.float32)
    e = np.exp(s.astype(np.float64) - 9.0)
    p = float(np.float32(0.6))
    assert 2 / e.sum() >= p > 1 / e.sum()
    r = oracle.topp(s, p)
    assert list(r.sel) == [1, 3]


def test_topp_two_token_closed_form():
    rng = np.random.default_rng(5)
    for _ in range(200):
        a, b = sorted(rng.standard_normal(2) * 2, reverse=True)
        s = np.array([a, b], np.float32)
        if s[0] == s[1]:
            continue
        p = float(np.float32(rng.uniform(0.5, 0.99)))
        first = 1.0 / (1.0 + math.exp(float(s[1]) - float(s[0])))
        r = oracle.topp(s, p)
        if abs(first - p) < 1e-12:
            continue
        assert r.k == (1 if first >= p else 2)
        assert r.sel[0] == 0


def test_topp_one_hot_query_selects_one_token():
    # One key carries a large component along a coordinate axis and the
    # query points along that axis: its score beats every other by > 30,
    # so it alone holds more than 0.9 of the mass.
    cfg = synth.CONFIGS[0].with_(N=4096)
    for i_star, axis in ((0, 3), (17, 0), (4095, 15)):
        kr = synth.layer_kr(cfg, 0)[0, 0].copy()
        kr[i_star, axis] = 10.0
        q = np.zeros(16, np.float32)
        q[axis] = 5.0
        s = oracle.scores(q, kr)
        assert np.sort(s)[-2] < s[i_star] - 30
        r = oracle.topp(s, 0.9)
        assert r.k == 1 and r.sel[0] == i_star


def test_topp_nested_in_p_and_mass_bounds():
    cfg = synth.CONFIGS[2].with_(N=8192)
    kr = synth.layer_kr(cfg, 0)
    qr = synth.layer_qr(cfg, 0)
    for b in range(cfg.B):
        s = oracle.scores(qr[b, 0], kr[b, 0])
        prev = set()
        for p in (0.5, 0.8, 0.9, 0.95, 0.99):
            r = oracle.topp(s, p)
            cur = set(r.sel.tolist())
            assert prev <= cur
            prev = cur
            pf = float(np.float32(p))
            assert r.mass >= pf - 1e-12
            assert r.slack < pf
            assert abs(oracle.set_mass(s, r.sel) - r.mass) < 1e-12
            # descending order with ties by index
            ss = s[r.sel]
            assert np.all(ss[:-1] >= ss[1:])


def test_set_mass_closed_forms():
    # Scores [1, 0]: mass({0}) = e / (e + 1) = 1 / (1 + e^-1), and the other
    # token takes the rest.
    s = np.array([1.0, 0.0], dtype=np.float32)
    assert abs(oracle.set_mass(s, [0]) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(oracle.set_mass(s, [1]) - 1.0 / (1.0 + math.e)) < 1e-15
    # A row of N equal scores: any k of them hold k / N, whatever the value.
    for val in (-3.5, 0.0, 40.0):
        t = np.full(1000, val, dtype=np.float32)
        for k in (1, 7, 500, 1000):
            assert abs(oracle.set_mass(t, np.arange(k) * (1000 // k)) - k / 1000.0) < 1e-13
    # Scores a + ln w_i for integer weights: mass(S) = sum_S w / sum w; the
    # shift a is exact in fp32 and must cancel.
    w = np.array([1, 2, 3, 4, 6], dtype=np.float64)
    for a in (0.0, -20.0, 30.0):
        sw = (a + np.log(w)).astype(np.float32)
        # the fp32 rounding of each score moves its weight by < 2^-23 relative
        ws = np.exp(sw.astype(np.float64) - float(np.max(sw)))
        for members in ([0], [4], [1, 3], [0, 1, 2, 3, 4]):
            want = ws[members].sum() / ws.sum()
            assert abs(oracle.set_mass(sw, members) - want) < 1e-14
            approx = w[members].sum() / w.sum()
            assert abs(oracle.set_mass(sw, members) - approx) < 1e-6
    # The empty set holds nothing.
    assert oracle.set_mass(s, np.zeros(0, dtype=np.int64)) == 0.0


def test_topp_p_one_selects_all():
    s = np.random.default_rng(3).standard_normal(1000).astype(np.float32)
    r = oracle.topp(s, 1.0)
    assert r.k == 1000 and np.array_equal(np.sort(r.sel), np.arange(1000))


def test_topp_permutation_equivariance():
    rng = np.random.default_rng(9)
    s = (rng.standard_normal(5000) * 3).astype(np.float32)
    perm = rng.permutation(5000)
    r1 = oracle.topp(s, 0.9)
    r2 = oracle.topp(s[perm], 0.9)
    assert set(perm[r2.sel].tolist()) == set(r1.sel.tolist())


def test_scores_bf16_keys_widen_exactly():
    # bf16 keys give the fp32 scores of their exact fp32 widening, and a key
    # row of exact small integers gives the integer dot product.
    cfg = synth.CONFIGS[0].with_(N=3000)
    q = synth.layer_qr(cfg, 0)[0, 0]
    kb = synth.f32_to_bf16(synth.layer_kr(cfg, 0)[0, 0])
    assert np.array_equal(oracle.scores_bf16(q, kb),
                          oracle.scores(q, synth.bf16_to_f32(kb)))
    qi = np.arange(16, dtype=np.float32) - 8
    ki = (np.arange(5 * 16, dtype=np.float32).reshape(5, 16) % 7) - 3
    want = (ki.astype(np.int64) @ qi.astype(np.int64)).astype(np.float32)
    assert np.array_equal(oracle.scores_bf16(qi, synth.f32_to_bf16(ki)), want)


# -------------------------------------------------------------- projection

def _bf16_of(v):
    return synth.f32_to_bf16(np.asarray(v, np.float32))


def test_project_selector_rows_copy_dims():
    # A projector whose row j is the unit vector e_{perm[j]} copies those
    # dims of every token row.
    rng = np.random.default_rng(50)
    x = synth.normal_bf16(synth.key(50, 1), 0, 37 * 128).reshape(37, 128)
    perm = rng.choice(128, 16, replace=False)
    W = np.zeros((16, 128), np.float32)
    W[np.arange(16), perm] = 1.0
    out = oracle.project(x, _bf16_of(W))
    assert np.array_equal(out, synth.bf16_to_f32(x)[:, perm].astype(np.float64))


def test_project_closed_form_and_transposition():
    # x all ones, W[j][c] = (j - 7) / 8 (exact in bf16): out[t][j] = 16 (j - 7).
    x = _bf16_of(np.ones((5, 128)))
    W = _bf16_of(np.repeat(((np.arange(16) - 7) / 8.0)[:, None], 128, axis=1))
    assert np.array_equal(oracle.project(x, W), np.tile(16.0 * (np.arange(16) - 7), (5, 1)))
    # W[j][c] = c-dependent, x[t] = e_t: out[t][j] = W[j][t] (catches a
    # transposed operand).
    Wv = _bf16_of((np.arange(16 * 128).reshape(16, 128) % 29) - 14)
    e = np.zeros((128, 128), np.float32)
    e[np.arange(128), np.arange(128)] = 1.0
    assert np.array_equal(oracle.project(_bf16_of(e), Wv), synth.bf16_to_f32(Wv).T.astype(np.float64))


def test_project_matches_numpy_matmul_fp64():
    x = synth.normal_bf16(synth.key(51, 1), 0, 300 * 128).reshape(300, 128)
    W = synth.normal_bf16(synth.key(51, 2), 0, 16 * 128).reshape(16, 128)
    ref = synth.bf16_to_f32(x).astype(np.float64) @ synth.bf16_to_f32(W).astype(np.float64).T
    got = oracle.project(x, W)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ top-k

@pytest.mark.parametrize("seed", range(8))
def test_topk_unique_dominating_subset_by_brute_force(seed):
    # The top-k set is the one subset of size min(k, n) in which every member
    # beats every non-member (a larger score, or an equal score and a lower
    # index).  Scores are rounded so that ties are common.
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 10))
    s = np.round(rng.standard_normal(n) * 2).astype(np.float32)
    s[rng.random(n) < 0.2] = -0.0

    def beats(i, j):
        return s[i] > s[j] or (s[i] == s[j] and i < j)

    for k in range(0, n + 2):
        m = min(k, n)
        winners = [set(c) for c in itertools.combinations(range(n), m)
                   if all(beats(i, j) for i in c for j in range(n) if j not in c)]
        assert len(winners) == 1, (seed, k)
        sel = oracle.topk(s, k)
        assert set(sel.tolist()) == winners[0]
        assert all(beats(sel[t], sel[t + 1]) for t in range(len(sel) - 1))


def test_topk_matches_numpy_lexsort():
    rng = np.random.default_rng(11)
    for n in (1, 7, 1000, 20_000):
        s = (np.round(rng.standard_normal(n) * 8) / 4).astype(np.float32)
        order = np.lexsort((np.arange(n), -s.astype(np.float64)))
        for k in (1, 2, n // 3, n - 1, n, n + 5):
            if k < 1:
                continue
            assert np.array_equal(oracle.topk(s, k), order[:min(k, n)]), (n, k)


def test_topk_one_is_first_argmax_and_ties_take_low_indices():
    rng = np.random.default_rng(12)
    for _ in range(50):
        s = np.round(rng.standard_normal(300)).astype(np.float32)
        assert oracle.topk(s, 1)[0] == int(np.argmax(s))
    z = np.zeros(100, np.float32)
    z[::2] = -0.0
    assert np.array_equal(np.sort(oracle.topk(z, 37)), np.arange(37))
    assert oracle.topk(z, 0).size == 0


def test_topk_agrees_with_topp_prefix_and_nests():
    cfg = synth.CONFIGS[2].with_(N=8192)
    s = oracle.scores(synth.layer_qr(cfg, 0)[0, 0], synth.layer_kr(cfg, 0)[0, 0])
    for p in (0.5, 0.9, 0.99):
        r = oracle.topp(s, p)
        assert np.array_equal(oracle.topk(s, r.k), r.sel)
    prev = set()
    for k in (1, 10, 100, 1000, 8192):
        cur = set(oracle.topk(s, k).tolist())
        assert prev <= cur and len(cur) == k
        prev = cur


# -------------------------------------------------------------- attention

def _bf16(x):
    return synth.f32_to_bf16(np.asarray(x, np.float32))


def _sdpa64(q, K, V, scale, mask=None):
    import torch
    qt = torch.from_numpy(synth.bf16_to_f32(q).astype(np.float64)).view(1, 1, -1)
    Kt = torch.from_numpy(synth.bf16_to_f32(K).astype(np.float64)).unsqueeze(0)
    Vt = torch.from_numpy(synth.bf16_to_f32(V).astype(np.float64)).unsqueeze(0)
    m = None if mask is None else torch.from_numpy(mask).view(1, 1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m,
                                                         scale=scale)
    return o.view(-1).numpy()


def test_attention_single_row_is_that_value_row():
    rng = np.random.default_rng(1)
    q, K, V = (_bf16(rng.standard_normal(s)) for s in ((128,), (1, 128), (1, 128)))
    out = oracle.attention(q, K, V, 0.0883883461356163)
    assert np.array_equal(out, synth.bf16_to_f32(V[0]).astype(np.float64))


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(2)
    q = _bf16(rng.standard_normal(128))
    K = np.repeat(_bf16(rng.standard_normal((1, 128))), 37, axis=0)
    V = _bf16(rng.standard_normal((37, 128)))
    out = oracle.attention(q, K, V, 0.0883883461356163)
    want = synth.bf16_to_f32(V).astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out - want)) < 1e-14


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(3)
    for n in (1, 5, 300):
        q = _bf16(rng.standard_normal(128))
        K = _bf16(rng.standard_normal((n, 128)) * 2)
        V = _bf16(rng.standard_normal((n, 128)))
        scale = float(np.float32(1 / math.sqrt(128)))
        out = oracle.attention(q, K, V, scale)
        assert np.max(np.abs(out - _sdpa64(q, K, V, scale))) < 1e-12


def test_local_rows_closed_forms(golden):
    for case in golden["local_rows"]:
        rows = oracle.local_rows(case["N"], case["n_sink"], case["window"])
        if "expected" in case:
            assert rows.tolist() == case["expected"]
        else:
            assert len(rows) == case["expected_count"]
            assert len(set(rows.tolist())) == len(rows)


def test_local_attention_equals_masked_dense():
    rng = np.random.default_rng(4)
    N, n_sink, W = 300, 4, 64
    q = _bf16(rng.standard_normal(128))
    K = _bf16(rng.standard_normal((N, 128)))
    V = _bf16(rng.standard_normal((N, 128)))
    scale = float(np.float32(1 / math.sqrt(128)))
    rows = oracle.local_rows(N, n_sink, W)
    out = oracle.attention(q, K[rows], V[rows], scale)
    mask = np.full(N, -np.inf)
    mask[:n_sink] = 0.0
    mask[N - W:] = 0.0
    assert np.max(np.abs(out - _sdpa64(q, K, V, scale, mask))) < 1e-12
    # a cache no longer than sinks + window: local == dense
    rows = oracle.local_rows(60, n_sink, W)
    assert np.array_equal(rows, np.arange(60))


def test_sparse_with_p_one_equals_dense_attention():
    cfg = synth.CONFIGS[0].with_(N=512)
    kr = synth.layer_kr(cfg, 0)[0, 0]
    qr = synth.layer_qr(cfg, 0)[0, 0]
    q = synth.layer_q(cfg, 0)[0, 0]
    K = synth.kv_rows(cfg, 0, "K", 0, 0, np.arange(cfg.N))
    V = synth.kv_rows(cfg, 0, "V", 0, 0, np.arange(cfg.N))
    r = oracle.topp(oracle.scores(qr, kr), 1.0)
    out = oracle.attention(q, K[r.sel], V[r.sel], cfg.scale)
    assert np.max(np.abs(out - _sdpa64(q, K, V, cfg.scale))) < 1e-12


def test_whole_head_permutation_equivariance():
    # Jointly shuffling the cached rows permutes the set and leaves the
    # output unchanged.
    cfg = synth.CONFIGS[1].with_(N=4096)
    rng = np.random.default_rng(8)
    kr = synth.layer_kr(cfg, 0)[0, 0]
    qr = synth.layer_qr(cfg, 0)[0, 2]
    q = synth.layer_q(cfg, 0)[0, 2]
    K = synth.kv_rows(cfg, 0, "K", 0, 0, np.arange(cfg.N))
    V = synth.kv_rows(cfg, 0, "V", 0, 0, np.arange(cfg.N))
    perm = rng.permutation(cfg.N)
    s1 = oracle.scores(qr, kr)
    assert len(np.unique(s1)) == cfg.N  # no ties, so the set is unique
    r1 = oracle.topp(s1, 0.9)
    r2 = oracle.topp(oracle.scores(qr, kr[perm]), 0.9)
    assert set(perm[r2.sel].tolist()) == set(r1.sel.tolist())
    o1 = oracle.attention(q, K[r1.sel], V[r1.sel], cfg.scale)
    o2 = oracle.attention(q, K[perm][r2.sel], V[perm][r2.sel], cfg.scale)
    assert np.max(np.abs(o1 - o2)) < 1e-12
