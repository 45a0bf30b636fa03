"""Build libq4moe.so (gfx950 HIP kernels + C ABI) and libq4probe.so (the
attainable-roof probes) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq4moe.so")
PROBE_LIB = os.path.join(PKG, "libq4probe.so")
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["q4moe_api.cpp", "gemv_q4_0.hip", "gemv_mfma_q4_0.hip", "gemv_q8_0.hip",
           "moe_q4_0.hip", "router_moe.hip", "moe_prefill.hip", "gemm_q4_0.hip",
           "gemv_noalloc.hip"]
# Per-source extra flags. The matrix-core tiles keep their accumulators in
# ordinary VGPRs (MFMA "VGPR form"): with accumulation registers the
# allocator rotated the accumulators between loop iterations (register copies
# on every batch).
EXTRA = {"gemv_mfma_q4_0.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "moe_q4_0.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # packed-FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every source into libq4moe.so and the probes into libq4probe.so
    (always recompiles). Returns the path of libq4moe.so."""
    _build_lib(SOURCES, LIB, verbose)
    _build_lib(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


# Host-side sanitizers for the C ABI's argument checks and plans: each
# -fsanitize applies to the host pass only (-Xarch_host); device code is
# built as usual.
SANITIZE_HOST = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()


def build_sanitized(out: str, verbose: bool = False) -> str:
    """Build libq4moe.so with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host code into `out` (load it in a process started with clang's
    ASan runtime preloaded)."""
    return _build_lib(SOURCES, out, verbose, extra=SANITIZE_HOST)


def _build_lib(sources, lib, verbose: bool, extra=()) -> str:
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    cflags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="q4moe_build_") as tmpdir:
        def compile_one(src: str):
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *cflags, *EXTRA.get(src, []), *extra, "-c", "-o", obj,
                   os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=min(4, len(sources))) as ex:
            results = list(ex.map(compile_one, sources))
        objs = []
        for obj, res in results:
            err = "\n".join(l for l in res.stderr.splitlines()
                            if "packed-fp32-ops" not in l and l.strip())
            if res.returncode != 0:
                sys.stderr.write(err + "\n")
                raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
            if err and verbose:
                sys.stderr.write(err + "\n")
            objs.append(obj)
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stderr + "\n")
            raise RuntimeError(f"hipcc failed linking {os.path.basename(lib)}")
        os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
