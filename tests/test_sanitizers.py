"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host code, on
the CPU: the oracle (every pin of test_oracle.py) and the C ABI's argument
checks, workspace sizing and plans (every check of test_abi.py, including the
sweep over extreme shapes). Each sanitized build runs in a child Python that
has the matching sanitizer runtime preloaded and allocates through malloc, so
out-of-bounds accesses to numpy and ctypes buffers are caught; any finding
aborts the child."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.slow


def run_child(tests, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONMALLOC"] = "malloc"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *tests]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc's libasan is not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    out = run_child(["tests/test_oracle.py"], {"LD_PRELOAD": libasan, "ORACLE_LIB": lib})
    assert "passed" in out


def test_abi_host_code_under_asan_ubsan(tmp_path):
    from moe_experts_amd import build
    if not shutil.which(build.HIPCC) and not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang's ASan runtime is not installed")
    lib = build.build_sanitized(str(tmp_path / "libq4moe_san.so"))
    out = run_child(["tests/test_abi.py"], {"LD_PRELOAD": rts[-1], "Q4MOE_ABI_LIB": lib})
    assert "passed" in out
