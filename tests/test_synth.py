"""The seeded input generator: determinism, random access, distributions."""
import numpy as np

import synth


def test_random_access_matches_bulk():
    cfg = synth.CONFIGS[1].with_(N=3000)
    K = synth.layer_kv(cfg, 0, "K")
    rows = np.array([0, 1, 2999, 1234])
    for g in range(cfg.Hkv):
        assert np.array_equal(synth.kv_rows(cfg, 0, "K", 0, g, rows), K[0, g, rows])
    a = synth.normal_f32(synth.key(1, synth.KR), 0, 1000, nthreads=1)
    b = synth.normal_f32(synth.key(1, synth.KR), 0, 1000, nthreads=4)
    assert np.array_equal(a, b)
    c = synth.normal_f32(synth.key(1, synth.KR), 500, 500)
    assert np.array_equal(a[500:], c)


def test_streams_are_distinct_and_deterministic():
    k1 = synth.key(3, synth.K, 0, 0, 0)
    assert k1 == synth.key(3, synth.K, 0, 0, 0)
    keys = {synth.key(3, s, l, b, h) for s in (synth.K, synth.V) for l in (0, 1)
            for b in (0, 1) for h in (0, 1)}
    assert len(keys) == 16
    u = synth.uniform(k1, range(1000))
    assert np.array_equal(u, synth._uniform_block(k1, 1000))
    assert np.all((u > 0) & (u < 1))


def test_distributions():
    x = synth.normal_f32(synth.key(0, synth.KR), 0, 1 << 20)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    t = synth.bf16_to_f32(synth.bf16_table())
    assert np.all(np.diff(t) >= 0)                 # monotone quantiles
    assert np.array_equal(t, -t[::-1])             # symmetric
    assert abs(t.mean()) < 1e-6 and abs(t.std() - 1) < 0.01
    y = synth.bf16_to_f32(synth.normal_bf16(synth.key(0, synth.K), 0, 1 << 20))
    assert abs(y.mean()) < 0.01 and abs(y.std() - 1) < 0.01


def test_needles_and_clusters():
    cfg = synth.CONFIGS[1].with_(N=8192)
    pos = synth.needle_positions(cfg, 0, 0)
    assert len(pos) == 256 and len(np.unique(pos)) == 256
    assert pos.min() >= 0 and pos.max() < cfg.N
    kr = synth.layer_kr(cfg, 0)
    qr = synth.layer_qr(cfg, 0)
    for h in range(cfg.H_r):
        qhat = qr[0, h] / np.linalg.norm(qr[0, h])
        for i in pos[h * 32:(h + 1) * 32]:
            assert np.linalg.norm(kr[0, 0, i] - 4 * qhat) < 1.0
    c3 = synth.CONFIGS[3].with_(N=4096)
    q3 = synth.layer_qr(c3, 0)
    assert np.allclose(np.linalg.norm(q3[0], axis=1), 8.0, rtol=1e-6)


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3], np.float32)
    b = synth.f32_to_bf16(x)
    back = synth.bf16_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0          # tie to even
    assert back[2] == np.float32(1.0078125)           # above the tie: up
    assert back[3] == -2.5
