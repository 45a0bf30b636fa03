"""CPU oracle (ctypes binding of ``liboracle.so``).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this module; the product package
``moe_experts_amd`` never does, and the two share no code.

The C++ source (``q4_oracle.cpp``) is the plain dequantize-then-multiply
definition from the "2000-line C++ DeepSeek inference engine" article (§2.2
block_q4_0 / dequantize, §3.2 loop order, §3.4 fused matmul_q4_0) evaluated in
double precision, plus the routed-expert MoE composition of the KTransformers
DeepSeek-V2 tutorial ("Optimization 3": top-6 of 160 routed experts as batched
GEMVs; the gate's top-k ids and weights, and the shared experts every token
uses). See ``q4_oracle.h`` for the exact contract of each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with g++ (single-threaded, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "q4_oracle.h"))
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """Compile the oracle with AddressSanitizer and UndefinedBehaviorSanitizer
    (any finding aborts) into `out`. Load it with ORACLE_LIB=out in a Python
    started with gcc's libasan preloaded."""
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared",
           "-o", out, _SRC]
    subprocess.check_call(cmd)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIB")  # a sanitized build (tests only)
    if not path:
        path = build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_fp16_to_double.restype = ctypes.c_double
    lib.oracle_fp16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_dequant_block.restype = None
    lib.oracle_dequant_block.argtypes = [P, P]
    lib.oracle_dequant_rows.restype = i32
    lib.oracle_dequant_rows.argtypes = [P, i32, i32, i32, P]
    lib.oracle_q4_0_matmul.restype = i32
    lib.oracle_q4_0_matmul.argtypes = [P, P, i32, i32, i32, P, P]
    lib.oracle_q4_0_matmul_f16.restype = i32
    lib.oracle_q4_0_matmul_f16.argtypes = [P, P, i32, i32, i32, P, P]
    lib.oracle_moe_decode.restype = i32
    lib.oracle_moe_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P]
    lib.oracle_q8_0_dequant_block.restype = None
    lib.oracle_q8_0_dequant_block.argtypes = [P, P]
    lib.oracle_q8_0_matmul.restype = i32
    lib.oracle_q8_0_matmul.argtypes = [P, P, i32, i32, i32, P, P]
    lib.oracle_router_logits.restype = i32
    lib.oracle_router_logits.argtypes = [P, P, i32, i32, i32, P, P]
    lib.oracle_router_topk.restype = i32
    lib.oracle_router_topk.argtypes = [P, i32, i32, i32, i32, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _blocks_u8(B: np.ndarray) -> np.ndarray:
    """View a packed Q4_0 array (structured or uint8) as contiguous bytes."""
    B = np.ascontiguousarray(B)
    return B.view(np.uint8).reshape(-1)


def fp16_to_double(bits: int) -> float:
    return _load().oracle_fp16_to_double(int(bits) & 0xFFFF)


def dequant_block(block18) -> np.ndarray:
    b = np.ascontiguousarray(np.frombuffer(bytes(block18), dtype=np.uint8))
    assert b.size == 18
    out = np.empty(32, dtype=np.float64)
    _load().oracle_dequant_block(_ptr(b), _ptr(out))
    return out


def dequant_rows(B: np.ndarray, N: int, k0: int, k1: int) -> np.ndarray:
    b = _blocks_u8(B)
    out = np.empty((k1 - k0, N), dtype=np.float32)
    rc = _load().oracle_dequant_rows(_ptr(b), N, k0, k1, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequant_rows: bad arguments")
    return out


def q4_0_matmul(x: np.ndarray, B: np.ndarray, N: int, K: int, with_bound: bool = True):
    """y = x . deq(B) in double, rounded to float32. Returns (y, bound|None)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
    M = x.shape[0]
    b = _blocks_u8(B)
    assert b.size == K * (N // 32) * 18, "B has the wrong number of bytes"
    y = np.empty((M, N), dtype=np.float32)
    bnd = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = _load().oracle_q4_0_matmul(_ptr(x), _ptr(b), M, N, K, _ptr(y), _ptr(bnd))
    if rc != 0:
        raise ValueError("oracle_q4_0_matmul: bad arguments")
    return y, bnd


def q4_0_matmul_f16(x16: np.ndarray, B: np.ndarray, N: int, K: int, with_bound: bool = True):
    """Prefill oracle: activations given as float16 (their bit patterns are used)."""
    x16 = np.ascontiguousarray(x16, dtype=np.float16).reshape(-1, K)
    M = x16.shape[0]
    b = _blocks_u8(B)
    assert b.size == K * (N // 32) * 18, "B has the wrong number of bytes"
    y = np.empty((M, N), dtype=np.float32)
    bnd = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = _load().oracle_q4_0_matmul_f16(_ptr(x16.view(np.uint16)), _ptr(b), M, N, K,
                                        _ptr(y), _ptr(bnd))
    if rc != 0:
        raise ValueError("oracle_q4_0_matmul_f16: bad arguments")
    return y, bnd


def moe_decode(x, Wg, Wu, Wd, ids, w, H: int, I: int, E: int, with_bound: bool = True,
               with_h: bool = False):
    """Routed-expert MoE decode. Returns (out, bound|None, h|None)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, H)
    T = x.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(T, -1)
    topk = ids.shape[1]
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(T, topk)
    mat = H * (I // 32) * 18
    g8, u8, d8 = _blocks_u8(Wg), _blocks_u8(Wu), _blocks_u8(Wd)
    assert g8.size == E * mat and u8.size == E * mat and d8.size == E * mat
    out = np.empty((T, H), dtype=np.float32)
    bnd = np.empty((T, H), dtype=np.float64) if with_bound else None
    h = np.empty((T, topk, I), dtype=np.float64) if with_h else None
    rc = _load().oracle_moe_decode(_ptr(x), _ptr(g8), _ptr(u8), _ptr(d8), _ptr(ids), _ptr(w),
                                   T, H, I, E, topk, _ptr(out), _ptr(bnd), _ptr(h))
    if rc != 0:
        raise ValueError("oracle_moe_decode: bad arguments")
    return out, bnd, h


def router_logits(x, Wr, with_bound: bool = True):
    """Router logits [T, E] = x [T, H] . Wr[E, H]^T in double, rounded to float32."""
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    E, H = Wr.shape
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, H)
    T = x.shape[0]
    lg = np.empty((T, E), dtype=np.float32)
    bnd = np.empty((T, E), dtype=np.float64) if with_bound else None
    rc = _load().oracle_router_logits(_ptr(x), _ptr(Wr), T, H, E, _ptr(lg), _ptr(bnd))
    if rc != 0:
        raise ValueError("oracle_router_logits: bad arguments")
    return lg, bnd


def router_topk(logits, topk: int, n_shared: int = 0):
    """Top-k ids (largest first, ties to the lower index, NaN never chosen) and
    softmax weights over them; n_shared shared-expert slots appended (id E + s,
    weight 1). Returns (ids int32 [T, topk + n_shared], w float32 [T, topk + n_shared])."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, topk + n_shared), dtype=np.int32)
    w = np.empty((T, topk + n_shared), dtype=np.float32)
    rc = _load().oracle_router_topk(_ptr(lg), T, E, topk, n_shared, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_router_topk: bad arguments")
    return ids, w


def q8_0_dequant_block(block34) -> np.ndarray:
    b = np.ascontiguousarray(np.frombuffer(bytes(block34), dtype=np.uint8))
    assert b.size == 34
    out = np.empty(32, dtype=np.float64)
    _load().oracle_q8_0_dequant_block(_ptr(b), _ptr(out))
    return out


def q8_0_matmul(x: np.ndarray, B: np.ndarray, N: int, K: int, with_bound: bool = True):
    """y = x . deq(B) for Q8_0 B (34-byte blocks) in double, rounded to float32."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
    M = x.shape[0]
    b = _blocks_u8(B)
    assert b.size == K * (N // 32) * 34, "B has the wrong number of bytes"
    y = np.empty((M, N), dtype=np.float32)
    bnd = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = _load().oracle_q8_0_matmul(_ptr(x), _ptr(b), M, N, K, _ptr(y), _ptr(bnd))
    if rc != 0:
        raise ValueError("oracle_q8_0_matmul: bad arguments")
    return y, bnd
