"""CPU oracle for the RTPurbo sparse decode path (arXiv 2605.16928).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product library never imports it.

This module is argument marshalling around ``oracle.c`` (plain C, fp32 scores
by a fixed fmaf chain, fp64 masses and attention; see the header of that file
for the definition each function follows).  Tests apply these per-head
definitions to every head of a decode layer themselves.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "_oracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall"]


def build() -> str:
    """Compile oracle.c into _oracle.so with gcc; returns the library path."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_scores.argtypes = [P, P, I64, P]
        lib.orc_scores.restype = None
        lib.orc_scores_bf16.argtypes = [P, P, I64, P]
        lib.orc_scores_bf16.restype = None
        lib.orc_topp.argtypes = [P, I64, ctypes.c_float, P, P]
        lib.orc_topp.restype = I64
        lib.orc_project.argtypes = [P, I64, I64, P, I64, P]
        lib.orc_project.restype = None
        lib.orc_topk.argtypes = [P, I64, I64, P]
        lib.orc_topk.restype = I64
        lib.orc_set_mass.argtypes = [P, I64, P, I64]
        lib.orc_set_mass.restype = ctypes.c_double
        lib.orc_attention.argtypes = [P, P, P, I64, P, I64, ctypes.c_float, P]
        lib.orc_attention.restype = None
        lib.orc_local_rows.argtypes = [I64, I64, I64, P]
        lib.orc_local_rows.restype = I64
        _lib = lib
    return _lib


class _Report(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int64), ("tau", ctypes.c_float),
                ("max_score", ctypes.c_double), ("Z", ctypes.c_double),
                ("mass", ctypes.c_double), ("last_mass", ctypes.c_double),
                ("slack", ctypes.c_double)]


@dataclass
class TopP:
    sel: np.ndarray       # int64, selection order (largest score first)
    k: int
    tau: float            # score of the last selected token
    max_score: float
    Z: float
    mass: float           # selected mass / Z
    last_mass: float      # last selected token's mass / Z
    slack: float          # mass without the last token / Z


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def scores(q_r: np.ndarray, k_r: np.ndarray) -> np.ndarray:
    """Indexer scores of one query head over [N][16] keys (fp32)."""
    q = np.ascontiguousarray(q_r, dtype=np.float32).reshape(16)
    k = np.ascontiguousarray(k_r, dtype=np.float32).reshape(-1, 16)
    out = np.empty(k.shape[0], dtype=np.float32)
    _load().orc_scores(_ptr(q), _ptr(k), k.shape[0], _ptr(out))
    return out


def scores_bf16(q_r: np.ndarray, k_bits: np.ndarray) -> np.ndarray:
    """Indexer scores of one query head over [N][16] bf16 keys (uint16 bit
    patterns, widened to fp32)."""
    q = np.ascontiguousarray(q_r, dtype=np.float32).reshape(16)
    k = np.ascontiguousarray(k_bits, dtype=np.uint16).reshape(-1, 16)
    out = np.empty(k.shape[0], dtype=np.float32)
    _load().orc_scores_bf16(_ptr(q), _ptr(k), k.shape[0], _ptr(out))
    return out


def topp(s: np.ndarray, p: float) -> TopP:
    """Top-p set of one head's scores; p is rounded to fp32 first."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    n = s.shape[0]
    sel = np.empty(max(n, 1), dtype=np.int64)
    rep = _Report()
    k = _load().orc_topp(_ptr(s), n, ctypes.c_float(p), _ptr(sel), ctypes.byref(rep))
    if k < 0:
        raise MemoryError("oracle top-p: out of memory")
    return TopP(sel=sel[:k].copy(), k=int(k), tau=float(rep.tau),
                max_score=rep.max_score, Z=rep.Z, mass=rep.mass,
                last_mass=rep.last_mass, slack=rep.slack)


def topk(s: np.ndarray, k: int) -> np.ndarray:
    """Top-k set of one head's scores (int64 indices, largest score first,
    ties to the lower index); k >= N keeps all."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    n = s.shape[0]
    sel = np.empty(max(n, 1), dtype=np.int64)
    c = _load().orc_topk(_ptr(s), n, int(k), _ptr(sel))
    if c < 0:
        raise MemoryError("oracle top-k: out of memory")
    return sel[:c].copy()


def project(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """fp64 projection of bf16 rows: x uint16 [T][d], W uint16 [r][d] (bf16
    bit patterns) -> float64 [T][r] with out[t][j] = sum_c W[j][c] x[t][c]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    T, d = x.shape
    r, dw = W.shape
    if dw != d:
        raise ValueError("x and W disagree in d")
    out = np.empty((T, r), np.float64)
    _load().orc_project(_ptr(x), T, d, _ptr(W), r, _ptr(out))
    return out


def set_mass(s: np.ndarray, members) -> float:
    """Mass fraction of an arbitrary token set under the scores s."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    m = np.ascontiguousarray(np.asarray(members, dtype=np.int64))
    return float(_load().orc_set_mass(_ptr(s), s.shape[0], _ptr(m), m.shape[0]))


def attention(q: np.ndarray, K_rows: np.ndarray, V_rows: np.ndarray,
              scale: float) -> np.ndarray:
    """fp64 softmax attention of one bf16 query over the given bf16 rows.

    q: uint16 [d]; K_rows, V_rows: uint16 [n][d] (bf16 bit patterns).
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    K = np.ascontiguousarray(K_rows, dtype=np.uint16)
    V = np.ascontiguousarray(V_rows, dtype=np.uint16)
    n, d = K.shape
    if n < 1:
        raise ValueError("attention over an empty set")
    rows = np.arange(n, dtype=np.int64)
    out = np.empty(d, dtype=np.float64)
    _load().orc_attention(_ptr(q), _ptr(K), _ptr(V), d, _ptr(rows), n,
                          ctypes.c_float(scale), _ptr(out))
    return out


def local_rows(N: int, n_sink: int, window: int) -> np.ndarray:
    """Rows a local head attends: the first n_sink plus the newest window."""
    rows = np.empty(max(N, 1), dtype=np.int64)
    n = _load().orc_local_rows(N, n_sink, window, _ptr(rows))
    return rows[:n].copy()
