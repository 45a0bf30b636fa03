"""GPU parity at the size limits the C ABI accepts: a Q4_0 matrix just under
2 GiB (the kernels address it with 32-bit byte offsets) through the decode GEMV
at batch 1 and 8 and through the prefill GEMM, and a prefill output just under
2 GiB. Each call runs in full; the oracle checks sampled block columns (all K
rows of each, so a wrong offset anywhere in the matrix shows) and sampled
rows."""
import numpy as np
import pytest
import torch

import oracle
from moe_experts_amd import datagen
from tests.gpu_util import check_tol, dev, to_dev, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# 65536 x 58240: 65536 * 1820 * 18 = 2 147 020 800 bytes, 462 847 below 2^31 - 1
K_BIG, N_BIG = 65536, 58240
LIMIT = (1 << 31) - 1
COLS = [0, 1, 909, 1818, 1819]  # block columns checked: both ends and the middle


@pytest.fixture(scope="module")
def big_matrix():
    B = datagen.q4_0_random(7101, K_BIG, N_BIG)
    assert B.nbytes <= LIMIT and B.nbytes > LIMIT - (1 << 20)
    return B, to_dev(B)


def block_columns(B, cols):
    """The sub-matrix of the given block columns (all rows), as Q4_0 bytes."""
    sub = np.ascontiguousarray(B.reshape(K_BIG, N_BIG // 32, 18)[:, cols, :])
    return sub, 32 * len(cols)


def sampled(y, cols):
    return np.concatenate([y[:, 32 * j:32 * j + 32] for j in cols], axis=1)


@pytest.mark.parametrize("M", [1, 8])
def test_gemv_matrix_just_under_2gib(big_matrix, M):
    from moe_experts_amd import q4_0_gemv
    B, Bd = big_matrix
    x = datagen.activations(7200 + M, M, K_BIG)
    y = to_host(q4_0_gemv(to_dev(x), Bd, N_BIG))
    sub, n = block_columns(B, COLS)
    ref, bnd = oracle.q4_0_matmul(x, sub, n, K_BIG)
    check_tol(sampled(y, COLS), ref, bnd, 1e-4, f"M={M} K={K_BIG} N={N_BIG}")
    assert np.isfinite(y).all()


def test_gemm_matrix_just_under_2gib(big_matrix):
    from moe_experts_amd import q4_0_gemm
    B, Bd = big_matrix
    M = 256
    x16 = datagen.activations(7301, M, K_BIG).astype(np.float16)
    y = to_host(q4_0_gemm(to_dev(x16), Bd, N_BIG))
    rows = [0, 1, 127, 128, 255]
    sub, n = block_columns(B, COLS)
    ref, bnd = oracle.q4_0_matmul_f16(x16[rows], sub, n, K_BIG)
    check_tol(sampled(y[rows], COLS), ref, bnd, 1e-2, "prefill on a 2 GiB matrix")


def test_gemm_output_just_under_2gib():
    """Y of 65536 x 8064 fp32 is 2 113 929 216 bytes: the last tiles' stores sit
    next to the 2^31 limit."""
    from moe_experts_amd import q4_0_gemm
    M, K, N = 65536, 256, 8064
    assert M * N * 4 <= LIMIT
    x16 = datagen.activations(7401, M, K).astype(np.float16)
    B = datagen.q4_0_random(7402, K, N)
    Y = torch.full((M * N + 64,), 1234.5, dtype=torch.float32, device=dev())
    q4_0_gemm(to_dev(x16), to_dev(B), N, Y=Y[:M * N].view(M, N))
    tail = to_host(Y[M * N:])
    assert (tail == 1234.5).all(), "GEMM wrote past Y"
    rows = [0, 255, 256, 32767, 65279, 65280, 65535]
    got = to_host(Y[:M * N].view(M, N)[rows])
    ref, bnd = oracle.q4_0_matmul_f16(x16[rows], B, N, K)
    check_tol(got, ref, bnd, 1e-2, "prefill with a 2 GiB output")
