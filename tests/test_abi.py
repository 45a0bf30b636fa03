"""C-ABI checks that run without a GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4moe.h")
# ABI checks can run against another build of the library (the host-sanitizer
# build of tests/test_sanitizers.py)
LIB = os.environ.get("Q4MOE_ABI_LIB") or os.path.join(ROOT, "moe_experts_amd", "libq4moe.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from moe_experts_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.q4_strerror.restype = ctypes.c_char_p
    L.q4_strerror.argtypes = [I]
    L.q4_0_gemv.argtypes = [P, P, P, I, I, I, P, Z, P]
    L.q4_0_gemv_workspace_bytes.restype = Z
    L.q4_0_gemv_workspace_bytes.argtypes = [I, I, I]
    L.q4_0_gemm.argtypes = [P, P, P, I, I, I, P]
    L.moe_q4_0_decode.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, Z, P]
    L.moe_q4_0_workspace_bytes.restype = Z
    L.moe_q4_0_workspace_bytes.argtypes = [I, I, I, I, I]
    L.moe_router_topk.argtypes = [P, P, P, P, P, I, I, I, I, I, P, Z, P]
    L.moe_router_workspace_bytes.restype = Z
    L.moe_router_workspace_bytes.argtypes = [I, I, I]
    L.moe_q4_0_layer.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, Z, P]
    L.moe_q4_0_layer_workspace_bytes.restype = Z
    L.moe_q4_0_layer_workspace_bytes.argtypes = [I, I, I, I, I, I]
    return L


PROBE_HEADER = os.path.join(ROOT, "include", "q4probe.h")
PROBE_LIB = os.path.join(ROOT, "moe_experts_amd", "libq4probe.so")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("_") and n != "sizeof"))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("q4_0_gemv", "q4_0_gemm", "moe_q4_0_decode", "q4_0_gemv_workspace_bytes",
              "moe_q4_0_workspace_bytes", "moe_router_topk", "moe_router_workspace_bytes",
              "moe_q4_0_layer", "moe_q4_0_layer_workspace_bytes", "q4_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in q4moe.h but not exported"


def test_every_header_has_its_library():
    """Each header under include/ belongs to one in-tree library, which loads
    and exports every function the header declares."""
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["q4moe.h", "q4probe.h"]
    if not os.path.exists(PROBE_LIB):
        from moe_experts_amd import build
        build.build()
    probe = ctypes.CDLL(PROBE_LIB)
    names = declared_functions(PROBE_HEADER)
    assert names == ["q4_probe_empty", "q4_probe_mfma_f16", "q4_probe_mfma_f32", "q4_probe_stream",
                     "q4_probe_tile"]
    for n in names:
        assert hasattr(probe, n), f"{n} declared in q4probe.h but not exported"


def test_probes_reject_bad_arguments():
    probe = ctypes.CDLL(PROBE_LIB)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    probe.q4_probe_stream.argtypes = [P, Z, I, P, P]
    probe.q4_probe_mfma_f16.argtypes = [I, I, P, P]
    probe.q4_probe_mfma_f32.argtypes = [I, I, P, P]
    assert probe.q4_probe_stream(None, 1024, 8, FAKE, None) == -1
    assert probe.q4_probe_stream(FAKE, 1000, 8, FAKE, None) == -1   # not a multiple of 16
    assert probe.q4_probe_stream(FAKE, 1 << 32, 8, FAKE, None) == -1
    assert probe.q4_probe_stream(FAKE, 1024, 0, FAKE, None) == -1
    assert probe.q4_probe_stream(FAKE + 4, 1024, 8, FAKE, None) == -3
    for f in (probe.q4_probe_mfma_f16, probe.q4_probe_mfma_f32):
        assert f(0, 8, FAKE, None) == -1
        assert f(8, 0, FAKE, None) == -1
        assert f(8, 8, None, None) == -1
    probe.q4_probe_tile.argtypes = [P, I, I, I, I, P, P]
    probe.q4_probe_empty.argtypes = [P, P]
    t = probe.q4_probe_tile
    assert t(None, 4096, 2304, 288, 128, FAKE, None) == -1
    assert t(FAKE, 4096, 2300, 288, 128, FAKE, None) == -1   # pitch not a multiple of 16
    assert t(FAKE, 4096, 2304, 280, 128, FAKE, None) == -1   # tile width not a multiple of 16
    assert t(FAKE, 4096, 2304, 288, 0, FAKE, None) == -1
    assert t(FAKE, 4096, 2304, 16, 1, FAKE, None) == -1      # 589824 workgroups
    assert t(FAKE, 1 << 20, 4096, 288, 128, FAKE, None) == -6  # 4 GiB matrix
    assert t(FAKE + 2, 4096, 2304, 288, 128, FAKE, None) == -3
    assert probe.q4_probe_empty(None, None) == -1


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        s = lib.q4_strerror(code)
        assert isinstance(s, bytes) and len(s) > 3


FAKE = 0x10000  # never dereferenced: every case below fails host validation


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, 1, 32, 1), -1),           # null x
    ((FAKE, FAKE, FAKE, 0, 32, 1), -1),           # M = 0
    ((FAKE, FAKE, FAKE, 1, 32, 0), -1),           # K = 0
    ((FAKE, FAKE, FAKE, 1, 48, 4), -2),           # N not a multiple of 32
    ((FAKE, FAKE, FAKE, 9, 32, 4), -2),           # M > 8
    ((FAKE + 2, FAKE, FAKE, 1, 32, 4), -3),       # misaligned x
    ((FAKE, FAKE + 1, FAKE, 1, 32, 4), -3),       # misaligned blocks
    ((FAKE, FAKE, FAKE, 1, 1 << 30, 1 << 30), -6),  # matrix larger than 2 GiB
    ((FAKE, FAKE, FAKE, 8, 32, 1 << 27), -6),       # activations larger than 2 GiB
])
def test_gemv_rejects_bad_arguments(lib, args, code):
    assert lib.q4_0_gemv(*args, None, 0, None) == code


def test_gemv_requires_workspace_when_split(lib):
    need = lib.q4_0_gemv_workspace_bytes(1, 4096, 4096)
    assert need > 0
    assert lib.q4_0_gemv(FAKE, FAKE, FAKE, 1, 4096, 4096, None, 0, None) == -4
    assert lib.q4_0_gemv(FAKE, FAKE, FAKE, 1, 4096, 4096, FAKE, need - 1, None) == -4
    assert lib.q4_0_gemv(FAKE, FAKE, FAKE, 1, 4096, 4096, FAKE + 16, need, None) == -3


def test_workspace_sizes(lib):
    assert lib.q4_0_gemv_workspace_bytes(0, 4096, 4096) == 0
    assert lib.q4_0_gemv_workspace_bytes(9, 4096, 4096) == 0
    assert lib.q4_0_gemv_workspace_bytes(1, 4096, 11008) > 0
    assert lib.moe_q4_0_workspace_bytes(1, 5120, 1536, 160, 6) > 0
    assert lib.moe_q4_0_workspace_bytes(65, 5120, 1536, 160, 6) == 0
    assert lib.moe_q4_0_workspace_bytes(1, 5120, 1536, 160, 9) == 0
    assert lib.moe_q4_0_workspace_bytes(1, 5120, 1530, 160, 6) == 0


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, 1, 32, 1), -1),
    ((FAKE, FAKE, FAKE, 1, 33, 1), -2),
    ((FAKE + 2, FAKE, FAKE, 1, 32, 1), -3),
    ((FAKE, FAKE, FAKE, 1, 1 << 20, 1 << 17), -6),
])
def test_gemm_rejects_bad_arguments(lib, args, code):
    assert lib.q4_0_gemm(*args, None) == code


def test_moe_rejects_bad_arguments(lib):
    f = lib.moe_q4_0_decode
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert f(None, *ok[1:], 1, 5120, 1536, 160, 6, None, 0, None) == -1
    assert f(*ok, 0, 5120, 1536, 160, 6, None, 0, None) == -1
    assert f(*ok, 65, 5120, 1536, 160, 6, None, 0, None) == -2
    assert f(*ok, 1, 5120, 1536, 160, 9, None, 0, None) == -2
    assert f(*ok, 1, 5120, 1536, 1025, 6, None, 0, None) == -2
    assert f(*ok, 1, 5121, 1536, 160, 6, None, 0, None) == -2
    assert f(*ok, 1, 5120, 1536, 160, 6, None, 0, None) == -4
    need = lib.moe_q4_0_workspace_bytes(1, 5120, 1536, 160, 6)
    assert f(*ok, 1, 5120, 1536, 160, 6, FAKE + 64, need, None) == -3


def test_moe_rejects_buffers_past_32_bit_offsets(lib):
    """h [T * topk][I] and the partial sums must stay below 2 GiB: a shape whose
    single expert matrix is small but whose per-pair buffers are not is
    refused before any launch, and has no workspace size."""
    f = lib.moe_q4_0_decode
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    T, H, I, E, topk = 64, 32, 1 << 20, 4, 8
    assert lib.moe_q4_0_workspace_bytes(T, H, I, E, topk) == 0
    assert f(*ok, T, H, I, E, topk, FAKE, 1 << 40, None) == -6
    assert lib.moe_q4_0_workspace_bytes(T, H, 1 << 14, E, topk) > 0


def test_gemv_noalloc_rejects_workspace_past_its_array(lib):
    """q4_0_gemv_noalloc serves the K-split partials from a fixed static
    array: a shape that needs more is refused before any HIP call, and bad
    arguments get q4_0_gemv's own errors."""
    P, I = ctypes.c_void_p, ctypes.c_int
    f = lib.q4_0_gemv_noalloc
    f.argtypes = [P, P, P, I, I, I, P]
    M, K, N = 8, 4096, 393216
    assert lib.q4_0_gemv_workspace_bytes(M, N, K) > (16 << 20)
    assert f(FAKE, FAKE, FAKE, M, N, K, None) == -6
    assert f(None, FAKE, FAKE, 1, 64, 64, None) == -1
    assert f(FAKE, FAKE, FAKE, 1, 48, 64, None) == -2
    assert f(FAKE, FAKE, FAKE, 9, 64, 64, None) == -2


def test_route_layout(lib):
    Z = ctypes.c_size_t
    lib.moe_q4_0_route_layout.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(Z)] * 3
    a, b, c = Z(), Z(), Z()
    assert lib.moe_q4_0_route_layout(32, 5120, 1536, 160, 6, ctypes.byref(a), ctypes.byref(b),
                                     ctypes.byref(c)) == 0
    need = lib.moe_q4_0_workspace_bytes(32, 5120, 1536, 160, 6)
    # items, counters and matrix-core items are disjoint, in order, inside the workspace
    assert a.value < b.value < c.value < need
    assert b.value - a.value >= 160 * 48 and c.value - b.value >= 8
    assert lib.moe_q4_0_route_layout(32, 5121, 1536, 160, 6, ctypes.byref(a), ctypes.byref(b),
                                     ctypes.byref(c)) == -2
    assert lib.moe_q4_0_route_layout(32, 5120, 1536, 160, 6, None, ctypes.byref(b),
                                     ctypes.byref(c)) == -1


def test_prefill_route_layout(lib):
    Z = ctypes.c_size_t
    lib.moe_q4_0_prefill_route_layout.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(Z)] * 4
    lib.moe_q4_0_prefill_workspace_bytes.restype = Z
    T, H, I, E, topk = 2048, 5120, 1536, 160, 6
    o = [Z() for _ in range(4)]
    refs = [ctypes.byref(v) for v in o]
    assert lib.moe_q4_0_prefill_route_layout(T, H, I, E, topk, *refs) == 0
    src, pos, tiles, counts = (v.value for v in o)
    need = lib.moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk)
    # src, pos, the tile list and the counters are disjoint, in order, inside the workspace
    assert src < pos < tiles < counts and counts + 8 <= need
    assert pos - src >= T * topk * 4 and tiles - pos >= T * topk * 4
    assert counts - tiles >= 16 * (T * topk // 128 + E)
    assert lib.moe_q4_0_prefill_route_layout(T, H + 1, I, E, topk, *refs) == -2
    assert lib.moe_q4_0_prefill_route_layout(T, H, I, E, topk, None, *refs[1:]) == -1
    assert lib.moe_q4_0_prefill_route_layout(T, H, I, E, topk, *refs[:3], None) == -1


def test_router_rejects_bad_arguments(lib):
    f = lib.moe_router_topk
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE)
    assert f(None, *ok[1:], 1, 5120, 160, 6, 2, None, 0, None) == -1
    assert f(*ok, 0, 5120, 160, 6, 2, None, 0, None) == -1
    assert f(*ok, 1, 5120, 160, 6, -1, None, 0, None) == -1
    assert f(*ok, 65, 5120, 160, 6, 2, None, 0, None) == -2     # T > 64
    assert f(*ok, 1, 5122, 160, 6, 2, None, 0, None) == -2     # H % 4
    assert f(*ok, 1, 5120, 1025, 6, 2, None, 0, None) == -2    # E > 1024
    assert f(*ok, 1, 5120, 5, 6, 0, None, 0, None) == -2       # topk > E
    assert f(*ok, 1, 5120, 160, 6, 3, None, 0, None) == -2     # 9 slots
    assert f(*ok, 1, 1 << 22, 160, 6, 2, None, 0, None) == -6  # router weights > 2 GiB
    assert f(FAKE + 4, *ok[1:], 1, 5120, 160, 6, 2, None, 0, None) == -3  # x not 16-B aligned
    assert f(*ok, 1, 5120, 160, 6, 2, None, 0, None) == -4
    need = lib.moe_router_workspace_bytes(1, 5120, 160)
    assert need > 0 and lib.moe_router_workspace_bytes(65, 5120, 160) == 0
    assert f(*ok, 1, 5120, 160, 6, 2, FAKE + 64, need, None) == -3


def test_layer_rejects_bad_arguments(lib):
    f = lib.moe_q4_0_layer
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert f(None, *ok[1:], 1, 5120, 1536, 160, 6, 2, None, 0, None) == -1
    assert f(*ok, 1, 5120, 1530, 160, 6, 2, None, 0, None) == -2     # I % 32
    assert f(*ok, 1, 5120, 1536, 1023, 6, 2, None, 0, None) == -2    # E + n_shared > 1024
    assert f(*ok, 1, 5120, 1536, 160, 7, 2, None, 0, None) == -2     # 9 slots
    assert f(*ok, 1, 5120, 1536, 160, 6, 2, None, 0, None) == -4
    need = lib.moe_q4_0_layer_workspace_bytes(32, 5120, 1536, 160, 6, 2)
    assert need > lib.moe_q4_0_workspace_bytes(32, 5120, 1536, 162, 8)
    assert lib.moe_q4_0_layer_workspace_bytes(32, 5120, 1536, 1023, 6, 2) == 0
    assert f(*ok, 32, 5120, 1536, 160, 6, 2, FAKE + 64, need, None) == -3


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, 1, 32, 1), -1),
    ((FAKE, FAKE, FAKE, 9, 32, 4), -2),
    ((FAKE, FAKE, FAKE, 1, 48, 4), -2),
    ((FAKE, FAKE + 1, FAKE, 1, 32, 4), -3),
    ((FAKE, FAKE, FAKE, 1, 1 << 29, 1 << 27), -6),   # Q8_0 matrix larger than 2 GiB
])
def test_q8_gemv_rejects_bad_arguments(lib, args, code):
    f = lib.q8_0_gemv
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_size_t,
                                                                ctypes.c_void_p]
    assert f(*args, None, 0, None) == code
    lib.q8_0_gemv_workspace_bytes.restype = ctypes.c_size_t
    assert lib.q8_0_gemv_workspace_bytes(1, 4096, 4096) > 0
    assert lib.q8_0_gemv_workspace_bytes(9, 4096, 4096) == 0


def test_moe_prefill_rejects_bad_arguments(lib):
    f = lib.moe_q4_0_prefill
    f.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_size_t,
                                                                ctypes.c_void_p]
    ws = lib.moe_q4_0_prefill_workspace_bytes
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int] * 5
    ok = (FAKE,) * 7
    assert f(None, *ok[1:], 64, 5120, 1536, 160, 6, None, 0, None) == -1
    assert f(*ok, 64, 5120, 1504, 160, 6, None, 0, None) == -2     # I % 128
    assert f(*ok, 64, 5184, 1536, 160, 6, None, 0, None) == -2     # H % 128
    assert f(*ok, 65537, 5120, 1536, 160, 6, None, 0, None) == -2  # T > 65536
    assert f(*ok, 64, 5120, 1536, 160, 9, None, 0, None) == -2     # topk > 8
    assert f(FAKE + 8, *ok[1:], 64, 5120, 1536, 160, 6, None, 0, None) == -3
    assert f(*ok[:6], FAKE + 4, 64, 5120, 1536, 160, 6, None, 0, None) == -3  # out not 16-B aligned
    assert f(*ok, 64, 5120, 1536, 160, 6, None, 0, None) == -4
    assert f(*ok, 60000, 5120, 1536, 160, 8, None, 0, None) == -6  # down rows > 2 GiB
    assert ws(2048, 5120, 1536, 160, 6) > 2048 * 6 * (4 * 5120 + 2 * 1536)
    assert ws(64, 5120, 1504, 160, 6) == 0


EXTREME = [-1, 0, 1, 3, 32, 33, 64, 96, 128, 4096, 5120, 11008, 65536, 1 << 20, (1 << 31) - 32,
           (1 << 31) - 1]


def test_sizing_functions_over_extreme_shapes(lib):
    """Every workspace-size and layout function answers for any shape, from
    negative to INT_MAX, without overflowing (run under UndefinedBehaviorSanitizer
    by tests/test_sanitizers.py): unsupported shapes give 0 (or an error), and
    a supported one a size that covers at least its largest array."""
    import itertools
    Z = ctypes.c_size_t
    lib.q8_0_gemv_workspace_bytes.restype = Z
    lib.q8_0_gemv_workspace_bytes.argtypes = [ctypes.c_int] * 3
    lib.moe_q4_0_prefill_workspace_bytes.restype = Z
    lib.moe_q4_0_prefill_workspace_bytes.argtypes = [ctypes.c_int] * 5
    lib.moe_q4_0_route_layout.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(Z)] * 3
    small = [-1, 0, 1, 2, 6, 8, 9, 64, 65, 160, 1024, 1025, 65536, 65537, (1 << 31) - 1]
    for M, N, K in itertools.product([-1, 0, 1, 3, 8, 9, (1 << 31) - 1], EXTREME, EXTREME):
        for f in (lib.q4_0_gemv_workspace_bytes, lib.q8_0_gemv_workspace_bytes):
            ws = f(M, N, K)
            if 1 <= M <= 8 and N > 0 and N % 32 == 0 and K > 0 and ws:
                assert ws >= 4 * M * N  # at least two splits of [M][N] fp32, or 0 for one
    a, b, c = Z(), Z(), Z()
    for T, H, I in itertools.product(small, EXTREME, EXTREME):
        for E, topk in ((160, 6), (1024, 8), (-1, 1), (1, 0)):
            lib.moe_q4_0_workspace_bytes(T, H, I, E, topk)
            lib.moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk)
            lib.moe_q4_0_layer_workspace_bytes(T, H, I, E, topk, 2)
            lib.moe_router_workspace_bytes(T, H, E)
            rc = lib.moe_q4_0_route_layout(T, H, I, E, topk, ctypes.byref(a), ctypes.byref(b),
                                           ctypes.byref(c))
            if rc == 0:
                need = lib.moe_q4_0_workspace_bytes(T, H, I, E, topk)
                assert a.value < b.value < c.value < need
