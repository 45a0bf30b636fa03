"""Thin Python binding of libq4moe (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libq4moe.so``. PyTorch supplies device memory and the current
HIP stream. The library must have been built (``moe_experts_amd.build``);
importing this module fails loudly if it is missing - there is no fallback.

The functions carry the names of the C entry points in ``include/q4moe.h``.
Before any call reaches the library, the binding checks that every tensor is a
contiguous device tensor of the dtype and number of elements the shape
arguments imply, so a mismatched tensor can never be read or written out of
bounds by a kernel.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq4moe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m moe_experts_amd.build` "
        "(the Q4_0 kernels have no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_lib.q4_strerror.restype = ctypes.c_char_p
_lib.q4_strerror.argtypes = [_I]
_lib.q4_0_gemv_workspace_bytes.restype = _Z
_lib.q4_0_gemv_workspace_bytes.argtypes = [_I, _I, _I]
_lib.q4_0_gemv.restype = _I
_lib.q4_0_gemv.argtypes = [_P, _P, _P, _I, _I, _I, _P, _Z, _P]
_lib.q4_0_gemv_noalloc.restype = _I
_lib.q4_0_gemv_noalloc.argtypes = [_P, _P, _P, _I, _I, _I, _P]
_lib.q8_0_gemv_workspace_bytes.restype = _Z
_lib.q8_0_gemv_workspace_bytes.argtypes = [_I, _I, _I]
_lib.q8_0_gemv.restype = _I
_lib.q8_0_gemv.argtypes = [_P, _P, _P, _I, _I, _I, _P, _Z, _P]
_lib.q4_0_gemm.restype = _I
_lib.q4_0_gemm.argtypes = [_P, _P, _P, _I, _I, _I, _P]
_lib.moe_q4_0_workspace_bytes.restype = _Z
_lib.moe_q4_0_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.moe_q4_0_decode.restype = _I
_lib.moe_q4_0_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P]
_lib.moe_q4_0_prefill_workspace_bytes.restype = _Z
_lib.moe_q4_0_prefill_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.moe_q4_0_prefill.restype = _I
_lib.moe_q4_0_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P]
_lib.moe_router_workspace_bytes.restype = _Z
_lib.moe_router_workspace_bytes.argtypes = [_I, _I, _I]
_lib.moe_router_topk.restype = _I
_lib.moe_router_topk.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P]
_lib.moe_q4_0_layer_workspace_bytes.restype = _Z
_lib.moe_q4_0_layer_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
_lib.moe_q4_0_layer.restype = _I
_lib.moe_q4_0_layer.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _Z, _P]

_lib.moe_q4_0_route_layout.restype = _I
_lib.moe_q4_0_route_layout.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(_Z), ctypes.POINTER(_Z),
                                       ctypes.POINTER(_Z)]

_lib.moe_q4_0_prefill_route_layout.restype = _I
_lib.moe_q4_0_prefill_route_layout.argtypes = [_I, _I, _I, _I, _I] + [ctypes.POINTER(_Z)] * 4

BLOCK_BYTES = 18
Q8_BLOCK_BYTES = 34


class Q4Error(RuntimeError):
    """A non-zero status returned by libq4moe."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libq4moe status {status}: {q4_strerror(status)}")


def q4_strerror(status: int) -> str:
    return _lib.q4_strerror(int(status)).decode()


def _check(rc: int):
    if rc != 0:
        raise Q4Error(rc)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype, numel: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


# Workspaces: one scratch buffer per (device, stream), grown on demand. Calls
# on one stream run in order, so they can share it.
_ws_lock = threading.Lock()
_ws_cache: dict = {}


def workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
            _ws_cache[key] = buf
        return buf


def q4_0_gemv_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.q4_0_gemv_workspace_bytes(M, N, K))


def moe_q4_0_workspace_bytes(T: int, H: int, I: int, E: int, topk: int) -> int:
    return int(_lib.moe_q4_0_workspace_bytes(T, H, I, E, topk))


def q4_0_gemv(x: torch.Tensor, B: torch.Tensor, N: int, y: torch.Tensor | None = None,
              ws: torch.Tensor | None = None) -> torch.Tensor:
    """y[M, N] = x[M, K] . deq(B) for a Q4_0 matrix B (uint8, K*(N/32)*18 bytes)."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if N <= 0 or N % 32:
        raise ValueError("N must be a positive multiple of 32")
    px = _dev(x, "x", torch.float32, M * K)
    pb = _dev(B, "B", torch.uint8, K * (N // 32) * BLOCK_BYTES)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py = _dev(y, "y", torch.float32, M * N)
    need = q4_0_gemv_workspace_bytes(M, N, K)
    if ws is None:
        ws = workspace(need, x.device)
    pw, nw = (None, 0) if ws is None else (_dev(ws, "ws", torch.uint8, ws.numel()), ws.numel())
    _check(_lib.q4_0_gemv(px, pb, py, M, N, K, pw, nw, _stream(x.device)))
    return y


# Largest q4_0_gemv workspace q4_0_gemv_noalloc serves from its static array.
GEMV_NOALLOC_MAX_WS = 16 << 20


def q4_0_gemv_noalloc(x: torch.Tensor, B: torch.Tensor, N: int,
                      y: torch.Tensor) -> torch.Tensor:
    """q4_0_gemv into a caller-provided y without any device allocation: the
    K-split partials live in the library's static per-GPU array."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if N <= 0 or N % 32:
        raise ValueError("N must be a positive multiple of 32")
    px = _dev(x, "x", torch.float32, M * K)
    pb = _dev(B, "B", torch.uint8, K * (N // 32) * BLOCK_BYTES)
    py = _dev(y, "y", torch.float32, M * N)
    _check(_lib.q4_0_gemv_noalloc(px, pb, py, M, N, K, _stream(x.device)))
    return y


def q8_0_gemv_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.q8_0_gemv_workspace_bytes(M, N, K))


def q8_0_gemv(x: torch.Tensor, B: torch.Tensor, N: int, y: torch.Tensor | None = None,
              ws: torch.Tensor | None = None) -> torch.Tensor:
    """y[M, N] = x[M, K] . deq(B) for a Q8_0 matrix B (uint8, K*(N/32)*34 bytes)."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if N <= 0 or N % 32:
        raise ValueError("N must be a positive multiple of 32")
    px = _dev(x, "x", torch.float32, M * K)
    pb = _dev(B, "B", torch.uint8, K * (N // 32) * Q8_BLOCK_BYTES)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py = _dev(y, "y", torch.float32, M * N)
    pw, nw = _ws_arg(ws, q8_0_gemv_workspace_bytes(M, N, K), x.device)
    _check(_lib.q8_0_gemv(px, pb, py, M, N, K, pw, nw, _stream(x.device)))
    return y


def q4_0_gemm(X: torch.Tensor, B: torch.Tensor, N: int, Y: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] = X[M, K] (float16) . deq(B) with fp32 accumulation, on MFMA."""
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M, K = X.shape
    if N <= 0 or N % 32:
        raise ValueError("N must be a positive multiple of 32")
    px = _dev(X, "X", torch.float16, M * K)
    pb = _dev(B, "B", torch.uint8, K * (N // 32) * BLOCK_BYTES)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    py = _dev(Y, "Y", torch.float32, M * N)
    _check(_lib.q4_0_gemm(px, pb, py, M, N, K, _stream(X.device)))
    return Y


def moe_q4_0_decode(x: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor,
                    topk_ids: torch.Tensor, topk_w: torch.Tensor, I: int, E: int,
                    out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Routed-expert MoE decode; x [T, H] fp32, ids/weights [T, topk]."""
    if x.dim() != 2 or topk_ids.dim() != 2:
        raise ValueError("x must be [T, H] and topk_ids [T, topk]")
    T, H = x.shape
    topk = topk_ids.shape[1]
    mat = H * (I // 32) * BLOCK_BYTES
    px = _dev(x, "x", torch.float32, T * H)
    pg = _dev(Wg, "Wg", torch.uint8, E * mat)
    pu = _dev(Wu, "Wu", torch.uint8, E * mat)
    pd = _dev(Wd, "Wd", torch.uint8, E * mat)
    pi = _dev(topk_ids, "topk_ids", torch.int32, T * topk)
    pw_ = _dev(topk_w, "topk_w", torch.float32, T * topk)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    po = _dev(out, "out", torch.float32, T * H)
    need = moe_q4_0_workspace_bytes(T, H, I, E, topk)
    if ws is None:
        ws = workspace(need, x.device)
    pws, nws = (None, 0) if ws is None else (_dev(ws, "ws", torch.uint8, ws.numel()), ws.numel())
    _check(_lib.moe_q4_0_decode(px, pg, pu, pd, pi, pw_, po, T, H, I, E, topk, pws, nws,
                                _stream(x.device)))
    return out


def moe_q4_0_route_layout(T: int, H: int, I: int, E: int, topk: int):
    """Byte offsets (items, counts, mitems) of the routing table that
    moe_q4_0_decode leaves in its workspace (T >= 2)."""
    a, b, c = _Z(), _Z(), _Z()
    _check(_lib.moe_q4_0_route_layout(T, H, I, E, topk, ctypes.byref(a), ctypes.byref(b),
                                      ctypes.byref(c)))
    return a.value, b.value, c.value


def moe_q4_0_prefill_route_layout(T: int, H: int, I: int, E: int, topk: int):
    """Byte offsets (src, pos, tiles, counts) of the routing that
    moe_q4_0_prefill leaves in its workspace."""
    o = [_Z() for _ in range(4)]
    _check(_lib.moe_q4_0_prefill_route_layout(T, H, I, E, topk, *[ctypes.byref(v) for v in o]))
    return tuple(v.value for v in o)


def moe_router_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(_lib.moe_router_workspace_bytes(T, H, E))


def moe_q4_0_layer_workspace_bytes(T: int, H: int, I: int, E: int, topk: int,
                                   n_shared: int) -> int:
    return int(_lib.moe_q4_0_layer_workspace_bytes(T, H, I, E, topk, n_shared))


def _ws_arg(ws, need: int, device):
    if ws is None:
        ws = workspace(need, device)
    return (None, 0) if ws is None else (_dev(ws, "ws", torch.uint8, ws.numel()), ws.numel())


def moe_router_topk(x: torch.Tensor, Wr: torch.Tensor, topk: int, n_shared: int = 0,
                    ws: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                    ids: torch.Tensor | None = None, w: torch.Tensor | None = None):
    """MoE router: x [T, H] fp32, Wr [E, H] fp32. Returns (logits [T, E],
    topk_ids int32 [T, topk + n_shared], topk_w fp32 [T, topk + n_shared]),
    written into the given tensors when passed."""
    if x.dim() != 2 or Wr.dim() != 2:
        raise ValueError("x must be [T, H] and Wr [E, H]")
    T, H = x.shape
    E = Wr.shape[0]
    px = _dev(x, "x", torch.float32, T * H)
    pr = _dev(Wr, "Wr", torch.float32, E * H)
    slots = topk + n_shared
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty((T, slots), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, slots), dtype=torch.float32, device=x.device)
    pl = _dev(logits, "logits", torch.float32, T * E)
    pi = _dev(ids, "ids", torch.int32, T * slots)
    pwt = _dev(w, "w", torch.float32, T * slots)
    pws, nws = _ws_arg(ws, moe_router_workspace_bytes(T, H, E), x.device)
    _check(_lib.moe_router_topk(px, pr, pl, pi, pwt, T, H, E, topk, n_shared, pws, nws,
                                _stream(x.device)))
    return logits, ids, w


def moe_q4_0_layer(x: torch.Tensor, Wr: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor,
                   Wd: torch.Tensor, I: int, topk: int, n_shared: int = 0,
                   out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Router, then routed and shared experts: x [T, H] fp32, Wr [E, H] fp32, and
    Wg/Wu/Wd holding E + n_shared Q4_0 expert matrices (routed, then shared)."""
    if x.dim() != 2 or Wr.dim() != 2:
        raise ValueError("x must be [T, H] and Wr [E, H]")
    T, H = x.shape
    E = Wr.shape[0]
    mat = H * (I // 32) * BLOCK_BYTES
    px = _dev(x, "x", torch.float32, T * H)
    pr = _dev(Wr, "Wr", torch.float32, E * H)
    pg = _dev(Wg, "Wg", torch.uint8, (E + n_shared) * mat)
    pu = _dev(Wu, "Wu", torch.uint8, (E + n_shared) * mat)
    pd = _dev(Wd, "Wd", torch.uint8, (E + n_shared) * mat)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    po = _dev(out, "out", torch.float32, T * H)
    pws, nws = _ws_arg(ws, moe_q4_0_layer_workspace_bytes(T, H, I, E, topk, n_shared), x.device)
    _check(_lib.moe_q4_0_layer(px, pr, pg, pu, pd, po, T, H, I, E, topk, n_shared, pws, nws,
                               _stream(x.device)))
    return out


def moe_q4_0_prefill_workspace_bytes(T: int, H: int, I: int, E: int, topk: int) -> int:
    return int(_lib.moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk))


def moe_q4_0_prefill(x16: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor,
                     topk_ids: torch.Tensor, topk_w: torch.Tensor, I: int, E: int,
                     out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Routed-expert MoE at prefill on the matrix cores; x16 [T, H] float16,
    ids/weights [T, topk]."""
    if x16.dim() != 2 or topk_ids.dim() != 2:
        raise ValueError("x16 must be [T, H] and topk_ids [T, topk]")
    T, H = x16.shape
    topk = topk_ids.shape[1]
    mat = H * (I // 32) * BLOCK_BYTES
    px = _dev(x16, "x16", torch.float16, T * H)
    pg = _dev(Wg, "Wg", torch.uint8, E * mat)
    pu = _dev(Wu, "Wu", torch.uint8, E * mat)
    pd = _dev(Wd, "Wd", torch.uint8, E * mat)
    pi = _dev(topk_ids, "topk_ids", torch.int32, T * topk)
    pw_ = _dev(topk_w, "topk_w", torch.float32, T * topk)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x16.device)
    po = _dev(out, "out", torch.float32, T * H)
    pws, nws = _ws_arg(ws, moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk), x16.device)
    _check(_lib.moe_q4_0_prefill(px, pg, pu, pd, pi, pw_, po, T, H, I, E, topk, pws, nws,
                                 _stream(x16.device)))
    return out
