"""ctypes binding of libq4probe.so (include/q4probe.h): the attainable-roof
probes the benchmark runs beside the Q4_0 kernels. Argument marshalling
only; the probes run as HIP kernels. Fails at import if the library is
missing."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq4probe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_experts_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_lib.q4_probe_stream.restype = _I
_lib.q4_probe_stream.argtypes = [_P, _Z, _I, _P, _P]
_lib.q4_probe_mfma_f16.restype = _I
_lib.q4_probe_mfma_f16.argtypes = [_I, _I, _P, _P]
_lib.q4_probe_mfma_f32.restype = _I
_lib.q4_probe_mfma_f32.argtypes = [_I, _I, _P, _P]
_lib.q4_probe_tile.restype = _I
_lib.q4_probe_tile.argtypes = [_P, _I, _I, _I, _I, _P, _P]
_lib.q4_probe_empty.restype = _I
_lib.q4_probe_empty.argtypes = [_P, _P]


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: status {rc}")


def stream_read(buf: torch.Tensor, offset: int, nbytes: int, grid: int, sink: torch.Tensor):
    """Read nbytes of the uint8 device tensor buf from byte offset (16-byte
    aligned) once, with 16-byte loads; sink: int32 device tensor of >= grid."""
    if buf.dtype != torch.uint8 or offset < 0 or offset + nbytes > buf.numel():
        raise ValueError("range outside the buffer")
    if sink.dtype != torch.int32 or sink.numel() < grid or sink.device != buf.device:
        raise ValueError("sink must be an int32 device tensor of at least grid words")
    _check(_lib.q4_probe_stream(buf.data_ptr() + offset, nbytes, grid, sink.data_ptr(),
                                _stream(buf.device)), "q4_probe_stream")


def tile_read(buf: torch.Tensor, offset: int, K: int, pitch: int, seg: int, kt: int,
              sink: torch.Tensor) -> int:
    """Read a K x pitch-byte matrix at byte offset (16-byte aligned) of the
    uint8 device tensor buf in split-K tiles of seg bytes x kt rows; returns
    the number of workgroups (sink: int32 device tensor of at least that)."""
    grid = -(-pitch // seg) * -(-K // kt)
    if buf.dtype != torch.uint8 or offset < 0 or offset + K * pitch > buf.numel():
        raise ValueError("matrix outside the buffer")
    if sink.dtype != torch.int32 or sink.numel() < grid or sink.device != buf.device:
        raise ValueError("sink must be an int32 device tensor of at least one word per tile")
    _check(_lib.q4_probe_tile(buf.data_ptr() + offset, K, pitch, seg, kt, sink.data_ptr(),
                              _stream(buf.device)), "q4_probe_tile")
    return grid


def empty(sink: torch.Tensor):
    """Launch the empty kernel (sink: any int32 device tensor, not written)."""
    if sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("sink must be an int32 device tensor")
    _check(_lib.q4_probe_empty(sink.data_ptr(), _stream(sink.device)), "q4_probe_empty")


def mfma_loop(kind: str, iters: int, grid: int, sink: torch.Tensor) -> int:
    """Run the f16 (16x16x32) or f32 (4x4x1) MFMA loop; returns its flops.
    sink: float32 device tensor of >= grid * 256."""
    if sink.dtype != torch.float32 or sink.numel() < grid * 256:
        raise ValueError("sink must be a float32 device tensor of at least grid * 256")
    fn, macs = {"f16": (_lib.q4_probe_mfma_f16, 8192), "f32": (_lib.q4_probe_mfma_f32, 256)}[kind]
    _check(fn(iters, grid, sink.data_ptr(), _stream(sink.device)), f"q4_probe_mfma_{kind}")
    return 2 * grid * 4 * iters * 8 * macs
