"""Seeded synthetic inputs for the RTPurbo decode path.

Shared by the GPU path's tests and benchmark (which upload what this module
generates) and by the CPU oracle (which regenerates only the rows it reads).
Holds no step of the attention method: only pseudo-random draws and the input
recipes (planted needles, Gaussian key clusters) that stand in for the pages'
long-context workloads, which no synthetic run can reproduce.

Layouts (row-major, C order):
    q_r  float32 [B][H_r][16]        indexer query of each retrieval head
    k_r  float32 [B][G_r][N][16]     indexer keys of each retrieval KV head
    q    uint16  [B][Hq][d]          bf16 bit patterns, full-dim query
    K, V uint16  [B][Hkv][N][d]      bf16 bit patterns, KV cache
Retrieval query heads are 0..H_r-1 (KV heads 0..G_r-1); local heads are
H_r..Hq-1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "_synth.so")

# Stream ids: one independent counter space per kind of value.
Q, QR, KR, K, V, NEEDLE_POS, NEEDLE_NOISE, CENTRES, ASSIGN, CLUSTER_NOISE, \
    QUERY_CLUSTERS = range(1, 12)


def build() -> str:
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11",
                           "-Wall", "-pthread", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        U64, U32, I64, P = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p
        lib.synth_key.argtypes = [U64, U32, U32, U32, U32]
        lib.synth_key.restype = U64
        lib.synth_uniform.argtypes = [U64, U64]
        lib.synth_uniform.restype = ctypes.c_double
        lib.synth_normal_f32.argtypes = [U64, I64, I64, P, ctypes.c_int]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_bf16.argtypes = [U64, I64, I64, P, ctypes.c_int]
        lib.synth_normal_bf16.restype = None
        lib.synth_bf16_rows.argtypes = [U64, P, I64, I64, P]
        lib.synth_bf16_rows.restype = None
        lib.synth_f32_rows.argtypes = [U64, P, I64, I64, P]
        lib.synth_f32_rows.restype = None
        lib.synth_bf16_table.argtypes = []
        lib.synth_bf16_table.restype = ctypes.POINTER(ctypes.c_uint16)
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ------------------------------------------------------------- primitives

def key(seed: int, stream: int, layer: int = 0, b: int = 0, head: int = 0) -> int:
    return int(_load().synth_key(seed, stream, layer, b, head))


def uniform(k: int, counters) -> np.ndarray:
    lib = _load()
    c = np.asarray(counters, dtype=np.uint64).reshape(-1)
    return np.array([lib.synth_uniform(k, int(x)) for x in c], dtype=np.float64)


def normal_f32(k: int, start: int, count: int, out=None, nthreads=None) -> np.ndarray:
    out = np.empty(count, np.float32) if out is None else out
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == count
    _load().synth_normal_f32(k, start, count, out.ctypes.data,
                             nthreads or default_threads())
    return out


def normal_bf16(k: int, start: int, count: int, out=None, nthreads=None) -> np.ndarray:
    out = np.empty(count, np.uint16) if out is None else out
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == count
    _load().synth_normal_bf16(k, start, count, out.ctypes.data,
                              nthreads or default_threads())
    return out


def bf16_table() -> np.ndarray:
    ptr = _load().synth_bf16_table()
    return np.ctypeslib.as_array(ptr, shape=(65536,)).copy()


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def partial_shuffle(k: int, n_pool: int, m: int) -> np.ndarray:
    """First m entries of a Fisher-Yates shuffle of range(n_pool), drawn
    with uniform(k, t) at step t: distinct values, uniformly chosen."""
    if m > n_pool:
        raise ValueError("more draws than pool entries")
    u = uniform(k, range(m))
    swap: dict = {}
    out = np.empty(m, dtype=np.int64)
    for t in range(m):
        j = t + int(u[t] * (n_pool - t))
        j = min(j, n_pool - 1)
        vt, vj = swap.get(t, t), swap.get(j, j)
        swap[t], swap[j] = vj, vt
        out[t] = vj
    return out


# ---------------------------------------------------------------- configs

@dataclass(frozen=True)
class Config:
    """One synthetic decode workload (all sizes per decode step)."""
    index: int
    name: str
    seed: int
    B: int
    L: int
    N: int
    Hq: int
    Hkv: int
    H_r: int                     # retrieval query heads (0..H_r-1)
    keys: str                    # "needle" or "cluster"
    needles_per_head: int = 0
    q_scale: tuple = (1.0,)      # indexer-query scale per batch row
    p_list: tuple = (0.9,)
    n_sink: int = 4
    window: int = 4096
    d: int = 128
    r: int = 16
    clusters: int = 64
    desc: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def G_r(self) -> int:
        return max(1, self.H_r // self.G)

    @property
    def H_l(self) -> int:
        return self.Hq - self.H_r

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = [
    Config(0, "toy_single_head_4k", seed=0, B=1, L=1, N=4096, Hq=1, Hkv=1, H_r=1,
           keys="needle", needles_per_head=8, n_sink=0, window=0,
           desc="1 q head / 1 kv head, N=4096, 8 planted needles, p=0.9, no local heads"),
    Config(1, "gqa_64k", seed=1, B=1, L=1, N=65536, Hq=32, Hkv=4, H_r=8,
           keys="needle", needles_per_head=32,
           desc="32 q / 4 kv heads, N=65536; q heads 0-7 retrieval (kv 0), 32 needles each; "
                "q heads 8-31 local (4 sinks + 4096 window)"),
    Config(2, "budget_mix_128k", seed=2, B=4, L=1, N=131072, Hq=32, Hkv=4, H_r=8,
           keys="needle", needles_per_head=32, q_scale=(0.1, 0.5, 2.0, 8.0),
           p_list=(0.8, 0.9, 0.95),
           desc="as gqa_64k at N=131072, batch 4, indexer-query scale 0.1/0.5/2/8 per row, "
                "p in {0.8, 0.9, 0.95}"),
    Config(3, "clusters_512k", seed=3, B=1, L=1, N=524288, Hq=32, Hkv=4, H_r=8,
           keys="cluster", q_scale=(8.0,),
           desc="as gqa_64k at N=524288; keys in 64 Gaussian clusters (width 0.3, centres x3), "
                "each query aligned with 1-3 clusters"),
    Config(4, "ctx1m_48layers", seed=4, B=1, L=48, N=1 << 20, Hq=32, Hkv=4, H_r=8,
           keys="needle", needles_per_head=32,
           desc="48 layers of gqa_64k at N=1048576 (bf16 K/V 2 GiB per layer)"),
]


# ------------------------------------------------------------ layer inputs

def layer_qr(cfg: Config, layer: int) -> np.ndarray:
    """Indexer queries q_r, float32 [B][H_r][16]."""
    out = np.empty((cfg.B, cfg.H_r, cfg.r), np.float32)
    for b in range(cfg.B):
        c = cfg.q_scale[b % len(cfg.q_scale)]
        for h in range(cfg.H_r):
            if cfg.keys == "cluster":
                out[b, h] = _cluster_query(cfg, layer, b, h)
            else:
                z = normal_f32(key(cfg.seed, QR, layer, b, h), 0, cfg.r)
                out[b, h] = (c * z.astype(np.float64)).astype(np.float32)
    return out


def _unit(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True))


def cluster_centres(cfg: Config, layer: int) -> np.ndarray:
    k = key(cfg.seed, CENTRES, layer, 0, 0)
    raw = normal_f32(k, 0, cfg.clusters * cfg.r).reshape(cfg.clusters, cfg.r)
    return _unit(raw)


def _cluster_query(cfg: Config, layer: int, b: int, h: int) -> np.ndarray:
    k = key(cfg.seed, QUERY_CLUSTERS, layer, b, h)
    n_pick = 1 + int(uniform(k, [0])[0] * 3)
    picks = partial_shuffle(key(cfg.seed, QUERY_CLUSTERS, layer, b, 1000 + h),
                            cfg.clusters, n_pick)
    u = cluster_centres(cfg, layer)[picks].sum(axis=0)
    c = cfg.q_scale[b % len(cfg.q_scale)]
    return (c * _unit(u)).astype(np.float32)


def needle_positions(cfg: Config, layer: int, b: int) -> np.ndarray:
    """Distinct needle positions, needles_per_head per retrieval query head:
    head h owns entries [h*m, (h+1)*m)."""
    m = cfg.needles_per_head * cfg.H_r
    return partial_shuffle(key(cfg.seed, NEEDLE_POS, layer, b, 0), cfg.N, m)


def layer_kr(cfg: Config, layer: int, nthreads=None) -> np.ndarray:
    """Indexer keys k_r, float32 [B][G_r][N][16]."""
    out = np.empty((cfg.B, cfg.G_r, cfg.N, cfg.r), np.float32)
    qr = layer_qr(cfg, layer) if cfg.keys == "needle" else None
    for b in range(cfg.B):
        for g in range(cfg.G_r):
            flat = out[b, g].reshape(-1)
            if cfg.keys == "cluster":
                centres = cluster_centres(cfg, layer)
                ka = key(cfg.seed, ASSIGN, layer, b, g)
                assign = np.minimum((_uniform_block(ka, cfg.N) * cfg.clusters)
                                    .astype(np.int64), cfg.clusters - 1)
                noise = normal_f32(key(cfg.seed, CLUSTER_NOISE, layer, b, g), 0,
                                   cfg.N * cfg.r, nthreads=nthreads)
                val = 3.0 * centres[assign] + 0.3 * noise.reshape(cfg.N, cfg.r).astype(np.float64)
                out[b, g] = val.astype(np.float32)
            else:
                normal_f32(key(cfg.seed, KR, layer, b, g), 0, cfg.N * cfg.r,
                           out=flat, nthreads=nthreads)
        if cfg.keys == "needle" and cfg.needles_per_head:
            pos = needle_positions(cfg, layer, b)
            m = cfg.needles_per_head
            nk = key(cfg.seed, NEEDLE_NOISE, layer, b, 0)
            for h in range(cfg.H_r):
                g = min(h // cfg.G, cfg.G_r - 1)
                qhat = _unit(qr[b, h])
                for t in range(m):
                    i = int(pos[h * m + t])
                    noise = normal_f32(nk, i * cfg.r, cfg.r).astype(np.float64)
                    out[b, g, i] = (4.0 * qhat + 0.1 * noise).astype(np.float32)
    return out


def _uniform_block(k: int, n: int) -> np.ndarray:
    """uniform(k, 0..n-1) computed in bulk (same values as uniform())."""
    c = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(k) + c * np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def layer_q(cfg: Config, layer: int) -> np.ndarray:
    """Full-dim queries, bf16 bits [B][Hq][d]."""
    out = np.empty((cfg.B, cfg.Hq, cfg.d), np.uint16)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            normal_bf16(key(cfg.seed, Q, layer, b, h), 0, cfg.d, out=out[b, h])
    return out


def layer_kv(cfg: Config, layer: int, which: str, out=None, nthreads=None) -> np.ndarray:
    """K or V cache, bf16 bits [B][Hkv][N][d]."""
    stream = K if which == "K" else V
    shape = (cfg.B, cfg.Hkv, cfg.N, cfg.d)
    out = np.empty(shape, np.uint16) if out is None else out
    assert out.shape == shape and out.dtype == np.uint16
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            normal_bf16(key(cfg.seed, stream, layer, b, g), 0, cfg.N * cfg.d,
                        out=out[b, g].reshape(-1), nthreads=nthreads)
    return out


def kv_rows(cfg: Config, layer: int, which: str, b: int, g: int, rows) -> np.ndarray:
    """Selected rows of K or V for (b, kv head g), bf16 bits [n][d]."""
    stream = K if which == "K" else V
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((r.shape[0], cfg.d), np.uint16)
    _load().synth_bf16_rows(key(cfg.seed, stream, layer, b, g), r.ctypes.data,
                            r.shape[0], cfg.d, out.ctypes.data)
    return out
