"""GPU parity of q4_0_gemm (prefill, fp16 MFMA) against the CPU oracle."""
import numpy as np
import pytest

import oracle
from moe_experts_amd import datagen
from tests.gpu_util import check_tol, guarded, guards_intact, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = 1e-2


def gemm(X16: np.ndarray, B: np.ndarray, N: int) -> np.ndarray:
    from moe_experts_amd import q4_0_gemm
    return to_host(q4_0_gemm(to_dev(X16), to_dev(B), N))


@pytest.mark.parametrize("M,K,N", [(1, 1, 32), (5, 17, 96), (128, 64, 128), (200, 100, 160),
                                   (130, 1000, 288), (257, 4096, 256), (64, 33, 4128)])
def test_gemm_small_match_oracle(M, K, N):
    X16 = datagen.to_f16(datagen.activations(M + K, M, K))
    B = datagen.q4_0_random(N * 3 + K, K, N)
    ref, bnd = oracle.q4_0_matmul_f16(X16, B, N, K)
    check_tol(gemm(X16, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")


# K % 64 == 0, N % 128 == 0, a 16-byte aligned X and a 4-byte aligned matrix
# take the pipelined kernel (256 x 128 tiles, K steps of 64): a single step
# and row, ragged M tails (one row past a tile, a tile and a bit), a single
# column tile and odd tile counts. The K values that are not multiples of 64
# take the other kernel.
ALIGNED = [(1, 64, 256), (130, 128, 512), (129, 1024, 768), (300, 192, 256), (2, 4096, 1024),
           (128, 64, 256), (130, 72, 512), (129, 1000, 768), (1, 64, 128), (257, 192, 384),
           (70, 4096, 640), (513, 128, 128)]


@pytest.mark.parametrize("M,K,N", ALIGNED)
def test_gemm_aligned_shapes_match_oracle(M, K, N):
    X16 = datagen.to_f16(datagen.activations(M + K + 11, M, K))
    B = datagen.q4_0_random(N * 5 + K, K, N)
    ref, bnd = oracle.q4_0_matmul_f16(X16, B, N, K)
    check_tol(gemm(X16, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")


def test_gemm_misaligned_x_takes_generic_path():
    """X only 4-byte aligned: the per-lane kernel must agree with the oracle on
    a shape that would otherwise take the pipelined one."""
    import torch
    from moe_experts_amd import q4_0_gemm
    from tests.gpu_util import dev
    M, K, N = 96, 256, 512
    X16 = datagen.to_f16(datagen.activations(21, M, K))
    B = datagen.q4_0_random(22, K, N)
    ref, bnd = oracle.q4_0_matmul_f16(X16, B, N, K)
    raw = torch.zeros(M * K + 8, dtype=torch.float16, device=dev())
    Xmis = raw[2:2 + M * K].view(M, K)
    Xmis.copy_(torch.from_numpy(X16))
    check_tol(to_host(q4_0_gemm(Xmis, to_dev(B), N)), ref, bnd, TOL, "misaligned X")


def test_gemm_integer_exact_bitwise():
    M, K, N = 256, 4096, 512
    g = np.random.Generator(np.random.PCG64(77))
    q = g.integers(0, 16, size=(K, N), dtype=np.uint8)
    d_bits = g.choice(np.array([0x3C00, 0x3800, 0x4000], dtype=np.uint16), size=(K, N // 32))
    B = datagen.assemble(d_bits, datagen.pack_nibbles(q))
    X16 = g.integers(-4, 5, size=(M, K)).astype(np.float16)
    ref, _ = oracle.q4_0_matmul_f16(X16, B, N, K)
    assert (gemm(X16, B, N) == ref).all()


def test_gemm_doubling_scales_doubles_output():
    M, K, N = 192, 512, 256
    X16 = datagen.to_f16(datagen.activations(3, M, K))
    B = datagen.q4_0_random(4, K, N)
    Y = gemm(X16, B, N)
    d = B[..., 0:2].copy().view(np.uint16)[..., 0]
    assert (gemm(X16, datagen.assemble(d + 0x0400, B[..., 2:]), N) == 2 * Y).all()
    assert (gemm(X16, B, N) == Y).all()


@pytest.mark.parametrize("which", [0, 1])
def test_gemm_prefill_full_size_every_band(which):
    """The prefill configuration (2048 x 4096 times 4096 x {4096, 11008}):
    one whole output row in every 32-row MFMA band of every m-tile (64 rows,
    each at a different offset inside its band), against the oracle; Y is
    written only inside its bounds."""
    from moe_experts_amd import q4_0_gemm
    c = datagen.PREFILL
    M, K, N = c["M"], c["K"], c["Ns"][which]
    X16 = datagen.to_f16(datagen.activations(c["x_seed"], M, K))
    B = datagen.q4_0_random(c["b_seeds"][which], K, N)
    full, Yv = guarded(M * N)
    q4_0_gemm(to_dev(X16), to_dev(B), N, Y=Yv)
    Y = to_host(Yv).reshape(M, N)
    assert guards_intact(full, M * N), "write outside Y"
    rows = np.array([32 * b + (7 * b + 3) % 32 for b in range(M // 32)])
    ref, bnd = oracle.q4_0_matmul_f16(X16[rows], B, N, K)
    check_tol(Y[rows], ref, bnd, TOL, f"prefill N={N}")
    assert np.isfinite(Y).all()
