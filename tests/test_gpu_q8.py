"""GPU parity of q8_0_gemv (Q8_0 weights: binary16 scale, 32 signed bytes)
against the CPU oracle."""
import numpy as np
import pytest

import oracle
from moe_experts_amd import datagen
from tests.gpu_util import check_tol, guarded, guards_intact, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = 1e-4


def gemv8(x, B, N):
    from moe_experts_amd import q8_0_gemv
    return to_host(q8_0_gemv(to_dev(x), to_dev(B), N))


# Batches 1..8 (half blocks per lane at M = 1, quarter blocks above), odd K
# and K below one row phase, N = 32 (one block, a tile of 8 mostly idle),
# N not a multiple of the 8-block tile, and K long enough to split.
@pytest.mark.parametrize("M,K,N", [(1, 1, 32), (1, 7, 96), (2, 33, 256), (3, 130, 288),
                                   (4, 515, 4128), (5, 64, 1056), (6, 1000, 512), (7, 9, 32),
                                   (8, 2049, 800), (1, 4097, 4128)])
def test_q8_small_shapes_match_oracle(M, K, N):
    x = datagen.activations(M * 13 + K, M, K)
    B = datagen.q8_0_random(K + 3 * N, K, N)
    ref, bnd = oracle.q8_0_matmul(x, B, N, K)
    check_tol(gemv8(x, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (8, 11008, 4096), (3, 4096, 11008)])
def test_q8_integer_exact_bitwise(M, K, N):
    g = np.random.Generator(np.random.PCG64(M + K + N))
    q = g.integers(-128, 128, size=(K, N // 32, 32)).astype(np.int8)
    d_bits = g.choice(np.array([0x3C00, 0x3800, 0x4000], dtype=np.uint16), size=(K, N // 32))
    B = datagen.assemble_q8(d_bits, q)
    x = g.integers(-4, 5, size=(M, K)).astype(np.float32)
    ref, _ = oracle.q8_0_matmul(x, B, N, K)
    assert (gemv8(x, B, N) == ref).all()


@pytest.mark.parametrize("M", [1, 2, 8])
def test_q8_invariants_bitwise(M):
    K, N = 2048, 1536
    x = datagen.activations(15, M, K)
    B = datagen.q8_0_random(16, K, N)
    y = gemv8(x, B, N)
    assert (gemv8(x, B, N) == y).all()                         # determinism
    B2 = B.copy()
    B2[..., 0:2] = (B[..., 0:2].copy().view(np.uint16) + 0x0400).view(np.uint8)
    assert (gemv8(x, B2, N) == 2 * y).all()                    # doubled scales
    assert (gemv8(x * np.float32(0.0625), B, N) == y * np.float32(0.0625)).all()
    Bz = B.copy()
    Bz[..., 0:2] = 0
    assert (gemv8(x, Bz, N) == 0).all()                        # zero scales
    rows = [0, 777, K - 1, 5, 1024, 1500, 2000, 3][:M]         # one-hot rows
    oh = np.zeros((M, K), dtype=np.float32)
    for m, k in enumerate(rows):
        oh[m, k] = 1
    y1 = gemv8(oh, B, N)
    for m, k in enumerate(rows):
        dq = np.concatenate([oracle.q8_0_dequant_block(B[k, j]) for j in range(N // 32)])
        assert (y1[m] == dq.astype(np.float32)).all(), (m, k)


@pytest.mark.parametrize("name,K,N", [("attn_proj", 4096, 4096), ("ffn_up", 4096, 11008),
                                      ("ffn_down", 11008, 4096)])
@pytest.mark.parametrize("M", [1, 8])
def test_q8_dense_7b_shapes(name, K, N, M):
    x = datagen.activations(2100 + M, M, K)
    B = datagen.q8_0_random(6200 + K % 97 + N % 89, K, N)
    ref, bnd = oracle.q8_0_matmul(x, B, N, K)
    check_tol(gemv8(x, B, N), ref, bnd, TOL, f"{name} M={M}")


def test_q8_guard_bands_untouched():
    from moe_experts_amd import q8_0_gemv
    M, K, N = 3, 700, 800
    x = datagen.activations(3, M, K)
    B = datagen.q8_0_random(4, K, N)
    full, y = guarded(M * N)
    q8_0_gemv(to_dev(x), to_dev(B), N, y=y.view(M, N))
    ref, bnd = oracle.q8_0_matmul(x, B, N, K)
    check_tol(to_host(y).reshape(M, N), ref, bnd, TOL, "guarded")
    assert guards_intact(full, M * N)


@pytest.mark.parametrize("M,K,N", [(8, 8192, 102400), (5, 4096, 152064)])
def test_q8_wide_matrices_fit_lds(M, K, N):
    """As for Q4_0: the plan splits K further when the activation tile would
    not fit in LDS."""
    x = datagen.activations(M + K + N + 1, M, K)
    B = datagen.q8_0_random(K + N + 1, K, N)
    ref, bnd = oracle.q8_0_matmul(x, B, N, K)
    check_tol(gemv8(x, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")
