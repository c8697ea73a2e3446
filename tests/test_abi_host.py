"""The C-ABI library on the host: it loads, exports every symbol that
include/rtp.h declares, sizes workspaces, and rejects bad arguments before
launching anything (so these calls never reach a GPU)."""
import ctypes
import os
import re

import pytest

import sparse_long_context_indexer_amd as rtp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtp.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rtp.LIB_PATH):
        from sparse_long_context_indexer_amd import _build
        _build.build()
    return rtp.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:rtp_status|const char \*|int32_t)\s*(rtp_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 24
    assert sorted(rtp.SYMBOLS) == names
    for n in names:
        assert hasattr(lib, n), n
    dyn = os.popen(f"nm -D --defined-only {rtp.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", dyn), n


def test_status_strings(lib):
    for code in range(9):
        assert rtp.status_string(code)
    assert rtp.status_string(99) == "unknown status"
    assert lib.rtp_last_hip_error() == 0


def test_workspace_sizes(lib):
    a = rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, 1, 8, 1 << 20)
    assert a >= 8 * (1 << 20) * 8          # candidate list capacity
    assert a % 256 == 0
    assert rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, 1, 8, 4096) < a
    for which in (rtp.RTP_WS_SPARSE_DECODE, rtp.RTP_WS_LOCAL_DECODE, rtp.RTP_WS_SPARSE_UNION,
                  rtp.RTP_WS_DECODE_ATTEND):
        s = rtp.workspace_size(which, 2, 8, 65536)
        assert s > 0 and s % 256 == 0
    # The combined attention workspace holds both sets' workspaces.
    assert rtp.workspace_size(rtp.RTP_WS_DECODE_ATTEND, 2, 32, 65536) >= (
        rtp.workspace_size(rtp.RTP_WS_SPARSE_DECODE, 2, 32, 65536)
        + rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, 2, 32, 65536))
    with pytest.raises(rtp.RtpError) as e:
        rtp.workspace_size(9, 1, 1, 1)
    assert e.value.status == 4
    with pytest.raises(rtp.RtpError) as e:
        rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, 0, 1, 1)
    assert e.value.status == 2
    assert lib.rtp_workspace_size(1, 1, 1, 1, None) == 1


# Fake device addresses: never dereferenced, since every call below fails
# validation before anything is launched.
A = 0x7f0000000000
A4 = A + 4


def test_index_scores_validation(lib):
    f = lib.rtp_index_scores
    assert f(None, A, A, 1, 8, 1, 100, 100, 16, None) == 1
    assert f(A, A, A, 1, 8, 1, 100, 100, 8, None) == 3          # r != 16
    assert f(A, A, A, 1, 8, 3, 100, 100, 16, None) == 2         # 8 % 3
    assert f(A, A, A, 1, 8, 1, 0, 100, 16, None) == 2           # N < 1
    assert f(A, A, A, 1, 8, 1, 101, 100, 16, None) == 2         # N > cap
    assert f(A, A, A, 0, 8, 1, 100, 100, 16, None) == 2         # B < 1
    assert f(A4, A, A, 1, 8, 1, 100, 100, 16, None) == 5        # q_r alignment
    assert f(A, A4, A, 1, 8, 1, 100, 100, 16, None) == 5        # k_r alignment


def test_topp_select_validation(lib):
    f = lib.rtp_topp_select
    ws = rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, 1, 8, 1000)
    assert f(None, 1, 8, 1000, 0.9, A, A, None, A, ws, None) == 1
    assert f(A, 1, 8, 1000, 0.9, A, A, None, None, ws, None) == 1
    for p in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        assert f(A, 1, 8, 1000, p, A, A, None, A, ws, None) == 4, p
    assert f(A, 1, 8, 0, 0.9, A, A, None, A, ws, None) == 2
    assert f(A, 1, 8, 1000, 0.9, A, A, None, A, ws - 1, None) == 6
    assert f(A, 1, 8, 1000, 0.9, A, A, None, A + 16, ws, None) == 5   # workspace alignment
    assert f(A + 2, 1, 8, 1000, 0.9, A, A, None, A, ws, None) == 5
    assert f(A, 1, 8, 1000, 0.9, A, A, A + 2, A, ws, None) == 5       # keep_bits alignment


def test_prefill_attend_validation(lib):
    # Every call below fails validation (the pointers are not device memory).
    f = lib.rtp_prefill_attend
    base = [A, A, A, 1, 32, 4, 1000, 1000, 128, 8, 24, 4, 4096, 0.088, A, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(0, None) == 1 and call(14, None) == 1
    assert call(8, 64) == 3
    assert call(5, 3) == 2 and call(6, 0) == 2 and call(7, 999) == 2
    assert call(9, 9) == 2 and call(10, 0) == 2 and call(3, 70000) == 2
    assert call(11, -1) == 4 and call(13, float("nan")) == 4
    assert call(1, A + 8) == 5 and call(14, A + 2) == 5


def test_keep_bits_add_local_validation(lib):
    # Every call below fails validation (the pointer is not device memory).
    f = lib.rtp_keep_bits_add_local
    assert f(None, 1, 8, 1000, 4, 64, None) == 1
    assert f(A, 0, 8, 1000, 4, 64, None) == 2 and f(A, 1, 8, 0, 4, 64, None) == 2
    assert f(A, 1, 65536, 1000, 4, 64, None) == 2
    assert f(A, 1, 8, 1000, -1, 64, None) == 4 and f(A, 1, 8, 1000, 4, 0, None) == 4
    assert f(A + 2, 1, 8, 1000, 4, 64, None) == 5


def test_local_decode_ring_validation(lib):
    # Every call below fails validation (the pointers are not device memory).
    f = lib.rtp_local_decode_ring
    ws = rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, 1, 8, 100000)
    base = [A, A, A, 1, 32, 4, 100000, 4100, 128, 8, 24, 4, 4096, 0.088, A, A, ws, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(0, None) == 1 and call(1, None) == 1
    assert call(7, 4099) == 2                   # kv_cap below n_sink + window
    assert call(6, 0) == 2                      # N < 1
    assert call(11, -1) == 4 and call(12, 0) == 4
    assert call(8, 64) == 3                     # d
    assert call(16, ws - 1) == 6
    assert call(1, A + 8) == 5


def test_index_scores_bf16_validation(lib):
    # Every call below fails validation (the pointers are not device memory).
    f = lib.rtp_index_scores_bf16
    assert f(None, A, A, 1, 8, 1, 100, 100, 16, None) == 1
    assert f(A, A, A, 1, 8, 1, 100, 100, 8, None) == 3          # r != 16
    assert f(A, A, A, 1, 8, 3, 100, 100, 16, None) == 2         # 8 % 3
    assert f(A, A, A, 1, 8, 1, 101, 100, 16, None) == 2         # N > cap
    assert f(A, A + 8, A, 1, 8, 1, 100, 100, 16, None) == 5     # k_r alignment


def test_index_project_validation(lib):
    # Every call below fails validation (the pointers are not device memory).
    f = lib.rtp_index_project
    base = [A, 2, 5, 100, 1, 3, 50, 128, A, 16, A, 200, 10, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(0, None) == 1 and call(8, None) == 1 and call(10, None) == 1
    assert call(7, 64) == 3 and call(9, 8) == 3        # d, r
    assert call(1, 0) == 2 and call(2, 0) == 2 and call(5, 0) == 2 and call(6, 0) == 2
    assert call(3, 49) == 2                              # x_cap < T
    assert call(4, -1) == 2 and call(4, 3) == 2          # head range outside Hx
    assert call(12, -1) == 2 and call(12, 151) == 2      # out rows past out_cap
    assert call(11, 49) == 2
    assert call(1, 30000) == 2                           # B*H above one grid
    assert call(0, A + 8) == 5 and call(8, A + 8) == 5 and call(10, A + 2) == 5


def test_topk_select_validation(lib):
    # Every call below fails validation (the pointers are not device memory).
    f = lib.rtp_topk_select
    ws = rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, 1, 8, 1000)
    assert f(None, 1, 8, 1000, 10, A, A, None, A, ws, None) == 1
    assert f(A, 1, 8, 1000, 10, None, A, None, A, ws, None) == 1
    assert f(A, 1, 8, 1000, 10, A, A, None, None, ws, None) == 1
    for k in (0, -1, -(2 ** 31)):
        assert f(A, 1, 8, 1000, k, A, A, None, A, ws, None) == 4, k
    assert f(A, 1, 8, 0, 10, A, A, None, A, ws, None) == 2
    assert f(A, 0, 8, 1000, 10, A, A, None, A, ws, None) == 2
    assert f(A, 1, 65536, 1000, 10, A, A, None, A, ws, None) == 2     # B*H above one grid
    assert f(A, 1, 8, 1000, 10, A, A, None, A, ws - 1, None) == 6
    assert f(A, 1, 8, 1000, 10, A, A, None, A + 16, ws, None) == 5    # workspace alignment
    assert f(A + 2, 1, 8, 1000, 10, A, A, None, A, ws, None) == 5
    assert f(A, 1, 8, 1000, 10, A, A, A + 2, A, ws, None) == 5        # keep_bits alignment


def test_sparse_decode_union_validation(lib):
    f = lib.rtp_sparse_decode_union
    ws = rtp.workspace_size(rtp.RTP_WS_SPARSE_UNION, 1, 8, 1000)
    base = [A, A, A, A, 1, 32, 4, 1000, 1000, 128, 0, 8, 0.088, A, A, ws, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert f(*base[:3], None, *base[4:]) == 1
    assert call(0, None) == 1
    assert call(3, A + 2) == 5                  # keep_bits alignment
    assert call(9, 64) == 3                     # d != 128
    assert call(6, 5) == 2                      # 32 % 5
    assert call(10, 30) == 2                    # 30 + 8 > 32
    assert call(12, float("inf")) == 4
    assert call(15, ws - 1) == 6


def test_sparse_decode_validation(lib):
    f = lib.rtp_sparse_decode
    ws = rtp.workspace_size(rtp.RTP_WS_SPARSE_DECODE, 1, 8, 1000)
    args = [A, A, A, A, A, 1, 32, 4, 1000, 1000, 128, 0, 8, 0.088, A, A, ws, None]

    def call(**kw):
        a = list(args)
        pos = {"q": 0, "idx": 3, "Hq": 6, "Hkv": 7, "N": 8, "cap": 9, "d": 10, "hb": 11,
               "nq": 12, "scale": 13, "out": 14, "ws": 15, "wsb": 16}
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    assert call(q=None) == 1
    assert call(idx=None) == 1
    assert call(d=64) == 3
    assert call(Hkv=5) == 2
    assert call(cap=999) == 2
    assert call(hb=30) == 2                     # 30 + 8 > 32
    assert call(nq=0) == 2
    assert call(scale=float("nan")) == 4
    assert call(q=A + 8) == 5
    assert call(wsb=ws - 1) == 6


def test_local_decode_validation(lib):
    f = lib.rtp_local_decode
    ws = rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, 1, 24, 1000)
    base = [A, A, A, 1, 32, 4, 1000, 1000, 128, 8, 24, 4, 4096, 0.088, A, A, ws, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(0, None) == 1
    assert call(8, 96) == 3
    assert call(11, -1) == 4                    # n_sink < 0
    assert call(12, 0) == 4                     # window < 1
    assert call(16, ws - 256) == 6
    assert call(15, A + 64) == 5


def test_one_hip_runtime_in_process(lib):
    # librtp must bind to the HIP runtime torch already loaded, not map a
    # second copy (two runtimes in one process report no device).
    maps = open("/proc/self/maps").read()
    hip = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(hip) == 1, hip


def test_decode_attend_validation(lib):
    f = lib.rtp_decode_attend
    ws = rtp.workspace_size(rtp.RTP_WS_DECODE_ATTEND, 1, 32, 1000)
    pos = {"q": 0, "idx": 3, "count": 4, "Hq": 6, "Hkv": 7, "N": 8, "d": 10, "sb": 11, "ns": 12,
           "lb": 13, "nl": 14, "sink": 15, "win": 16, "scale": 17, "ws": 19, "wsb": 20}
    args = [A, A, A, A, A, 1, 32, 4, 1000, 1000, 128, 0, 8, 8, 24, 4, 4096, 0.088, A, A, ws,
            None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    assert call(q=None) == 1
    assert call(idx=None) == 1                  # sparse heads need idx and count
    assert call(count=None) == 1
    assert call(ns=0, nl=0) == 2                # nothing to do
    assert call(ns=-1) == 2
    assert call(lb=4) == 2                      # ranges 0..7 and 4..27 overlap
    assert call(lb=9) == 2                      # 9 + 24 > 32
    assert call(sink=-1) == 4
    assert call(win=0) == 4
    assert call(d=64) == 3
    assert call(scale=float("nan")) == 4
    assert call(idx=A + 2) == 5
    assert call(wsb=0) == 6                     # (ws - 1 would still suffice: the size
    assert call(ws=A + 16) == 5                 #  query covers any head split)
    # With no sparse heads, idx and count are not needed (the call gets as
    # far as the workspace check); with no local heads, n_sink and window
    # are not checked.  Every call here fails before any launch.
    assert call(ns=0, idx=None, count=None, wsb=0) == 6
    assert call(nl=0, sink=-1, win=0, wsb=0) == 6


def test_scan_local_validation(lib):
    f = lib.rtp_scan_local
    ws = rtp.workspace_size(rtp.RTP_WS_LOCAL_DECODE, 1, 24, 1000)
    pos = {"q_r": 0, "k_r": 1, "scores": 2, "Hq_r": 3, "Hkv_r": 4, "kr_cap": 5, "r": 6, "q": 7,
           "B": 10, "Hq": 11, "Hkv": 12, "N": 13, "kv_cap": 14, "d": 15, "lb": 16, "nl": 17,
           "sink": 18, "win": 19, "scale": 20, "out": 21, "ws": 22, "wsb": 23}
    args = [A, A, A, 8, 1, 1000, 16, A, A, A, 1, 32, 4, 1000, 1000, 128, 8, 24, 4, 4096, 0.088,
            A, A, ws, None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    # Every call below breaks one rule, so none reaches a launch.
    for name in ("q_r", "k_r", "scores", "q", "out", "ws"):
        assert call(**{name: None}) == 1, name
    assert call(r=8) == 3
    assert call(d=64) == 3
    assert call(Hq_r=7, Hkv_r=2) == 2           # not a multiple
    assert call(Hkv_r=0) == 2
    assert call(kr_cap=999) == 2                # k_r holds fewer than N rows
    assert call(kv_cap=999) == 2
    assert call(N=0) == 2
    assert call(B=0) == 2
    assert call(nl=0) == 2                      # the local set may not be empty
    assert call(lb=9) == 2                      # 9 + 24 > 32
    assert call(sink=-1) == 4
    assert call(win=0) == 4
    assert call(scale=float("nan")) == 4
    assert call(q_r=A + 4) == 5
    assert call(k_r=A + 8) == 5
    assert call(scores=A + 2) == 5
    assert call(q=A + 2) == 5
    assert call(ws=A + 16) == 5
    assert call(wsb=0) == 6
    assert call(wsb=ws - 1) == 6                # sized for exactly these 24 heads


def test_topp_hist_validation(lib):
    f = lib.rtp_topp_hist
    ws = rtp.workspace_size(rtp.RTP_WS_TOPP_SELECT, 1, 8, 1000)
    assert f(None, 1, 8, 1000, A, ws, None) == 1
    assert f(A, 1, 8, 1000, None, ws, None) == 1
    assert f(A, 1, 8, 0, A, ws, None) == 2
    assert f(A, 0, 8, 1000, A, ws, None) == 2
    assert f(A + 2, 1, 8, 1000, A, ws, None) == 5
    assert f(A, 1, 8, 1000, A + 16, ws, None) == 5
    assert f(A, 1, 8, 1000, A, ws - 1, None) == 6


def test_decode_layer_validation(lib):
    # Host-side checks of rtp_decode_layer, in order: NULL, unsupported
    # dimensions, sizes, values, alignment; all before any device query.
    f = lib.rtp_decode_layer
    pos = {"q_r": 0, "k_r": 1, "kr_cap": 2, "q": 3, "K": 4, "V": 5, "kv_cap": 6, "B": 7,
           "Hq": 8, "Hkv": 9, "N": 10, "d": 11, "r": 12, "Hq_r": 13, "sink": 14, "win": 15,
           "p": 16, "scale": 17, "out": 18, "idx": 19, "count": 20, "scores": 21, "ws": 22,
           "wsb": 23}
    args = [A, A, 1000, A, A, A, 1000, 1, 32, 4, 1000, 128, 16, 8, 4, 4096, 0.9, 0.088, A, A, A,
            None, A, 1 << 30, None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    for name in ("q_r", "k_r", "q", "K", "V", "out", "idx", "count", "ws"):
        assert call(**{name: None}) == 1, name
    assert call(d=64) == 3 and call(r=8) == 3
    assert call(N=0) == 2 and call(kr_cap=999) == 2 and call(kv_cap=999) == 2
    assert call(B=0) == 2 and call(Hkv=3) == 2 and call(Hq_r=0) == 2 and call(Hq_r=33) == 2
    assert call(Hq_r=12) == 2                   # not whole KV heads (G = 8)
    assert call(sink=-1) == 4 and call(win=0) == 4
    for p in (0.0, -0.1, 1.01, float("nan")):
        assert call(p=p) == 4, p
    assert call(scale=float("inf")) == 4
    assert call(q_r=A + 4) == 5 and call(K=A + 8) == 5 and call(scores=A + 2) == 5
    assert call(ws=A + 16) == 5 and call(idx=A + 2) == 5
    # With every head a retrieval head, n_sink and window are not checked.
    assert call(Hq_r=32, sink=-1, win=0, q_r=A + 4) == 5
    with pytest.raises(rtp.RtpError) as e:
        rtp.decode_layer_workspace_size(1, 32, 4, 0, 8, 4, 4096)
    assert e.value.status == 2
    assert lib.rtp_decode_layer_workspace_size(1, 32, 4, 100, 8, 4, 4096, None) == 1


def test_topp_attend_validation(lib):
    # Host-side checks of rtp_topp_attend, in order: NULL, unsupported
    # dimensions, sizes, values, alignment; all before any device query.
    f = lib.rtp_topp_attend
    pos = {"scores": 0, "q": 1, "K": 2, "V": 3, "B": 4, "Hq": 5, "Hkv": 6, "N": 7,
           "kv_cap": 8, "d": 9, "Hq_r": 10, "sink": 11, "win": 12, "p": 13, "scale": 14,
           "out": 15, "idx": 16, "count": 17, "ws": 18, "wsb": 19}
    args = [A, A, A, A, 1, 32, 4, 1000, 1000, 128, 8, 4, 4096, 0.9, 0.088, A, A, A, A, 1 << 30,
            None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    for name in ("scores", "q", "K", "V", "out", "idx", "count", "ws"):
        assert call(**{name: None}) == 1, name
    assert call(d=64) == 3
    assert call(N=0) == 2 and call(kv_cap=999) == 2
    assert call(B=0) == 2 and call(Hkv=3) == 2 and call(Hq_r=0) == 2 and call(Hq_r=33) == 2
    assert call(Hq_r=12) == 2                   # not whole KV heads (G = 8)
    assert call(Hkv=2, Hq_r=16) == 3            # G = 16: more than 8 heads per KV head
    assert call(B=129) == 3                     # more than 1024 score rows
    assert call(N=1 << 30, kv_cap=1 << 30) == 3  # B * Hq_r * N beyond 32 bits
    assert call(sink=-1) == 4 and call(win=0) == 4
    for p in (0.0, -0.1, 1.01, float("nan")):
        assert call(p=p) == 4, p
    assert call(scale=float("nan")) == 4
    assert call(scores=A + 2) == 5 and call(K=A + 8) == 5 and call(ws=A + 16) == 5
    assert call(idx=A + 2) == 5
    # With every head a retrieval head, n_sink and window are not checked.
    assert call(Hq_r=32, sink=-1, win=0, q=A + 4) == 5
    with pytest.raises(rtp.RtpError) as e:
        rtp.topp_attend_workspace_size(1, 32, 4, 0, 8, 4, 4096)
    assert e.value.status == 2
    assert lib.rtp_topp_attend_workspace_size(1, 32, 4, 100, 8, 4, 4096, None) == 1


def test_wait_limit_and_status_entry_points(lib):
    assert lib.rtp_set_wait_limit(1 << 24) == 0
    assert lib.rtp_device_status(None, 0) == 1


def _cpu(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def test_binding_checks_every_shape():
    # Every tensor's full shape is checked against the sizes the C call will
    # read; a mismatch raises before anything reaches the library (these
    # tensors live on the host, so a call that passed the checks would stop
    # at the device check instead).
    import torch
    f32, i32, bf, u8 = torch.float32, torch.int32, torch.bfloat16, torch.uint8
    ws = _cpu((64,), u8)
    B, Hq, Hkv, N, cap = 2, 32, 4, 100, 120
    q, K, V = _cpu((B, Hq, 128), bf), _cpu((B, Hkv, cap, 128), bf), _cpu((B, Hkv, cap, 128), bf)
    out = _cpu((B, Hq, 128), f32)
    bad = [
        lambda: rtp.rtp_index_scores(_cpu((B, 8, 16), f32), _cpu((B + 1, 1, cap, 16), f32),
                                     _cpu((B, 8, N), f32)),
        lambda: rtp.rtp_index_scores(_cpu((B, 8, 16), f32), _cpu((B, 1, cap, 16), f32),
                                     _cpu((B, 7, N), f32)),
        lambda: rtp.rtp_topp_select(_cpu((B, 8, N), f32), 0.9, _cpu((B, 8, N - 1), i32),
                                    _cpu((B, 8), i32), ws),
        lambda: rtp.rtp_topp_select(_cpu((B, 8, N), f32), 0.9, _cpu((B, 8, N), i32),
                                    _cpu((B, 7), i32), ws),
        lambda: rtp.rtp_topk_select(_cpu((B, 8, N), f32), 5, _cpu((B, 8, N), i32),
                                    _cpu((B + 1, 8), i32), ws),
        lambda: rtp.rtp_sparse_decode(q, K, V, _cpu((B, 8, N), i32), _cpu((B, 8), i32), 0, 0.1,
                                      _cpu((B, Hq, 64), f32), ws),
        lambda: rtp.rtp_sparse_decode(q, K, _cpu((B, Hkv, cap - 1, 128), bf),
                                      _cpu((B, 8, N), i32), _cpu((B, 8), i32), 0, 0.1, out, ws),
        lambda: rtp.rtp_sparse_decode(q, K, V, _cpu((B, 8, N), i32), _cpu((B, 8), i32), 0, 0.1,
                                      out, ws, N=N + 1),
        lambda: rtp.rtp_sparse_decode(q, K, V, _cpu((1, 8, N), i32), _cpu((B, 8), i32), 0, 0.1,
                                      out, ws),
        lambda: rtp.rtp_sparse_decode_union(q, K, V, _cpu((B, 8, 3), i32), N, 0, 0.1, out, ws),
        lambda: rtp.rtp_decode_attend(q, K, V, _cpu((B, 8, N - 1), i32), _cpu((B, 8), i32), N,
                                      0, 8, 24, 4, 4096, 0.1, out, ws),
        lambda: rtp.rtp_local_decode(q, _cpu((B + 1, Hkv, cap, 128), bf), V, N, 8, 24, 4, 4096,
                                     0.1, out, ws),
        lambda: rtp.rtp_local_decode_ring(q, K, V, N, 8, 24, 4, 4096, 0.1,
                                          _cpu((B, Hq - 1, 128), f32), ws),
        lambda: rtp.rtp_scan_local(_cpu((B, 8, 16), f32), _cpu((B, 1, cap, 16), f32),
                                   _cpu((B, 8, N + 1), f32), q, K, V, N, 8, 24, 4, 4096, 0.1,
                                   out, ws),
        lambda: rtp.rtp_prefill_attend(_cpu((B, Hq, 50, 128), bf), K, V, 0, 8, 0, 0, 0.1,
                                       _cpu((B, Hq, 49, 128), f32)),
        lambda: rtp.rtp_decode_layer(_cpu((B, 8, 16), f32), _cpu((B, 2, cap, 16), f32), q, K, V,
                                     N, 8, 4, 4096, 0.9, 0.1, out, _cpu((B, 8, N), i32),
                                     _cpu((B, 8), i32), ws),
        lambda: rtp.rtp_decode_layer(_cpu((B, 8, 16), f32), _cpu((B, 1, cap, 16), f32), q, K, V,
                                     N, 8, 4, 4096, 0.9, 0.1, out, _cpu((B, 8, N + 1), i32),
                                     _cpu((B, 8), i32), ws),
        lambda: rtp.rtp_decode_layer(_cpu((B, 8, 16), f32), _cpu((B, 1, cap, 16), f32), q, K, V,
                                     N, 8, 4, 4096, 0.9, 0.1, out, _cpu((B, 8, N), i32),
                                     _cpu((B, 8), i32), ws, scores=_cpu((B, 8, N - 1), f32)),
        lambda: rtp.rtp_index_project(_cpu((B, 4, 50, 128), bf), _cpu((2, 16, 128), bf),
                                      _cpu((B, 3, 60, 16), f32)),
        lambda: rtp.rtp_keep_bits_add_local(_cpu((B, 8, 5), i32), N, 4, 64),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError) as e:
            call()
        assert "device tensor" not in str(e.value), (i, str(e.value))


def test_sparse_decode_noalloc_validation(lib):
    f = lib.rtp_sparse_decode_noalloc
    args = [A, A, A, A, A, 1, 32, 4, 1000, 1000, 128, 0, 8, 0.088, A, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)

    assert call(3, None) == 1 and call(4, None) == 1 and call(0, None) == 1
    assert call(10, 64) == 3
    assert call(8, 0) == 2 and call(12, 0) == 2
    assert call(13, float("nan")) == 4
    assert call(3, A + 2) == 5
    # 4 MiB of scratch holds 256 score rows of partials, not 65535.
    assert call(5, 65535) == 2 or call(5, 65535) == 8
    assert call(5, 300) == 8                     # 300 * 8 rows > the scratch
    assert rtp.status_string(8).startswith("the sizes exceed")
