"""GPU parity of q4_0_gemv against the CPU oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from moe_experts_amd import datagen
from tests.golden_io import gemv_cases, handworked_block
from tests.gpu_util import check_tol, dev, guarded, guards_intact, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = 1e-4


def gemv(x: np.ndarray, B: np.ndarray, N: int) -> np.ndarray:
    from moe_experts_amd import q4_0_gemv
    return to_host(q4_0_gemv(to_dev(x), to_dev(B), N))


SMALL = [(1, 1, 32), (1, 2, 64), (2, 31, 96), (3, 33, 256), (8, 64, 288), (1, 4097, 4128),
         (5, 300, 160), (4, 1000, 512), (8, 4097, 96), (7, 129, 1024), (6, 2, 4128)]
# Shapes whose rows are whole 16-byte chunks (N % 256 == 0, N >= 512) take the
# LDS-staged weight path: a single row, a partial last column tile
# (N % 512 == 256), odd row counts, every batch size.
STAGED = [(1, 1, 512), (2, 17, 768), (3, 5, 1280), (8, 3000, 768), (5, 4097, 2304),
          (1, 257, 512), (4, 63, 1792), (6, 1111, 1280)]


@pytest.mark.parametrize("M,K,N", SMALL)
def test_gemv_small_shapes_match_oracle(M, K, N):
    x = datagen.activations(M * 1000 + K, M, K)
    B = datagen.q4_0_random(N + K, K, N)
    ref, bnd = oracle.q4_0_matmul(x, B, N, K)
    check_tol(gemv(x, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", STAGED)
def test_gemv_staged_shapes_match_oracle(M, K, N):
    x = datagen.activations(M * 1000 + K + 7, M, K)
    B = datagen.q4_0_random(N + K + 7, K, N)
    ref, bnd = oracle.q4_0_matmul(x, B, N, K)
    check_tol(gemv(x, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")


def test_gemv_every_split_count_range():
    """The split-K sum is compiled for at most 8, 16, 32 and 64 splits and for
    any count; a narrow matrix with a growing K walks through all five."""
    from moe_experts_amd import q4_0_gemv_workspace_bytes
    M, N = 2, 512
    seen = set()
    for K in (1024, 2048, 3000, 4096, 6000, 8192, 16384):
        S = max(1, q4_0_gemv_workspace_bytes(M, N, K) // (4 * M * N))
        seen.add(next(c for c in (8, 16, 32, 64, 1 << 30) if S <= c))
        x = datagen.activations(K + 3, M, K)
        B = datagen.q4_0_random(K + 4, K, N)
        ref, bnd = oracle.q4_0_matmul(x, B, N, K)
        check_tol(gemv(x, B, N), ref, bnd, TOL, f"M={M} K={K} N={N} S={S}")
    assert seen == {8, 16, 32, 64, 1 << 30}, seen


def test_gemv_misaligned_matrix_takes_generic_path():
    """A matrix that is only 2-byte aligned cannot be staged in 16-byte
    chunks; the per-lane path must give the same bits as the staged one."""
    from moe_experts_amd import q4_0_gemv
    M, K, N = 3, 700, 1024
    x = datagen.activations(11, M, K)
    B = datagen.q4_0_random(12, K, N)
    ref, bnd = oracle.q4_0_matmul(x, B, N, K)
    raw = torch.zeros(B.size + 16, dtype=torch.uint8, device=dev())
    Bmis = raw[2:2 + B.size]
    Bmis.copy_(torch.from_numpy(B.reshape(-1)))
    y = to_host(q4_0_gemv(to_dev(x), Bmis, N))
    check_tol(y, ref, bnd, TOL, "misaligned B")


def test_gemv_handworked():
    qs, _, _, _ = handworked_block()
    blk = lambda d: np.frombuffer(bytes([d & 255, d >> 8]) + qs, dtype=np.uint8)
    B = np.stack([blk(0x3C00), blk(0x3800)]).reshape(2, 1, 18)
    for xs, ys in gemv_cases():
        y = gemv(np.array([xs], dtype=np.float32), B, 32)
        assert (y[0] == np.array(ys, dtype=np.float32)).all(), y


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (8, 11008, 4096), (3, 4096, 11008)])
def test_gemv_integer_exact_bitwise(M, K, N):
    g = np.random.Generator(np.random.PCG64(K + N + M))
    q = g.integers(0, 16, size=(K, N), dtype=np.uint8)
    d_bits = g.choice(np.array([0x3C00, 0x3800, 0x4000], dtype=np.uint16), size=(K, N // 32))
    B = datagen.assemble(d_bits, datagen.pack_nibbles(q))
    x = g.integers(-4, 5, size=(M, K)).astype(np.float32)
    ref, _ = oracle.q4_0_matmul(x, B, N, K)
    assert (gemv(x, B, N) == ref).all()


@pytest.mark.parametrize("M", [2, 4, 8])  # vector tiles; matrix cores with 1 and 2 row halves
def test_gemv_invariants_bitwise(M):
    K, N = 2048, 1536
    x = datagen.activations(5, M, K)
    B = datagen.q4_0_random(6, K, N)
    y = gemv(x, B, N)
    # determinism
    assert (gemv(x, B, N) == y).all()
    # doubling every scale doubles y bitwise
    d = B[..., 0:2].copy().view(np.uint16)[..., 0]
    assert (gemv(x, datagen.assemble(d + 0x0400, B[..., 2:]), N) == 2 * y).all()
    # x * 2^-4 scales y bitwise
    assert (gemv(x * np.float32(0.0625), B, N) == y * np.float32(0.0625)).all()
    # zero scales and all-8 nibbles give zeros
    Bz = B.copy(); Bz[..., 0:2] = 0
    assert (gemv(x, Bz, N) == 0).all()
    B8 = B.copy(); B8[..., 2:] = 0x88
    assert (gemv(x, B8, N) == 0).all()
    # one-hot x selects the dequantized row bitwise (M one-hot rows)
    W = oracle.dequant_rows(B, N, 0, K)
    rows = [0, 777, K - 1, 5, 1024, 1500, 2000, 3][:M]
    oh = np.zeros((M, K), dtype=np.float32)
    for m, k in enumerate(rows):
        oh[m, k] = 1
    y1 = gemv(oh, B, N)
    for m, k in enumerate(rows):
        assert (y1[m] == W[k]).all(), (m, k)


# Batches 3..8 run on the matrix-core kernel: tile widths of 4 or 8 block
# columns with a partial last tile (N/32 = 13, 21, 43), fewer rows than the
# tile's row phases (K = 1, 3, 15), one and two activation halves, odd batches,
# and a matrix too wide for that kernel's plan (the vector tiles take it).
# N/32 a multiple of 8 plans only 8-block tiles: one column tile (N = 256), two,
# three, with ragged row counts.
MATRIX_CORE = [(3, 1, 416), (5, 3, 672), (7, 15, 416), (8, 17, 96), (4, 129, 4128),
               (6, 300, 1376), (8, 700, 11008), (3, 5000, 672), (8, 64, 262144),
               (5, 77, 256), (3, 2049, 512), (4, 130, 768), (8, 4099, 256)]


@pytest.mark.parametrize("M,K,N", MATRIX_CORE)
def test_gemv_matrix_core_edges(M, K, N):
    x = datagen.activations(M * 7 + K, M, K)
    B = datagen.q4_0_random(N + 3 * K, K, N)
    ref, bnd = oracle.q4_0_matmul(x, B, N, K)
    check_tol(gemv(x, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")


def test_gemv_rows_independent_of_batch():
    # The tile plan may differ with M, so rows agree to rounding, not bitwise.
    K, N = 4096, 11008
    x = datagen.activations(9, 8, K)
    B = datagen.q4_0_random(10, K, N)
    y8 = gemv(x, B, N)
    _, bnd = oracle.q4_0_matmul(x, B, N, K)
    for m in (0, 3, 7):
        check_tol(gemv(x[m:m + 1], B, N)[0], y8[m], bnd[m], 1e-5, f"row {m}")
    check_tol(gemv(x[2:5], B, N), y8[2:5], bnd[2:5], 1e-5, "rows 2..4")


def test_gemv_guard_bands_untouched():
    from moe_experts_amd import q4_0_gemv
    M, K, N = 3, 1000, 4128
    x = datagen.activations(11, M, K)
    B = datagen.q4_0_random(12, K, N)
    full, yv = guarded(M * N)
    q4_0_gemv(to_dev(x), to_dev(B), N, y=yv.view(M, N))
    torch.cuda.synchronize()
    assert guards_intact(full, M * N)
    ref, bnd = oracle.q4_0_matmul(x, B, N, K)
    check_tol(to_host(yv).reshape(M, N), ref, bnd, TOL)


def test_gemv_single_vector_4096():
    # single GEMV, 4096 x 4096, batch 1, seeds of the small workload
    c = datagen.GEMV_4096
    x = datagen.activations(c["x_seed"], 1, c["K"])
    B = datagen.q4_0_random(c["b_seed"], c["K"], c["N"])
    ref, bnd = oracle.q4_0_matmul(x, B, c["N"], c["K"])
    check_tol(gemv(x, B, c["N"]), ref, bnd, TOL, "gemv 4096")


@pytest.mark.parametrize("name,K,N,seed", datagen.DENSE_7B_SHAPES)
def test_gemv_dense_7b_shapes(name, K, N, seed):
    B = datagen.q4_0_random(seed, K, N)
    Bd = to_dev(B)
    from moe_experts_amd import q4_0_gemv
    for M in datagen.DENSE_7B_BATCHES:
        x = datagen.activations(datagen.dense_x_seed(M), M, K)
        ref, bnd = oracle.q4_0_matmul(x, B, N, K)
        got = to_host(q4_0_gemv(to_dev(x), Bd, N))
        check_tol(got, ref, bnd, TOL, f"{name} M={M}")


@pytest.mark.parametrize("M,K,N", [(8, 8192, 102400), (5, 4096, 152064), (1, 16384, 65536)])
def test_gemv_wide_matrices_fit_lds(M, K, N):
    """Wide matrices: the grid target alone would leave tiles whose activation
    tile does not fit in LDS; the plan splits K further and the call works."""
    x = datagen.activations(M + K + N, M, K)
    B = datagen.q4_0_random(K + N, K, N)
    ref, bnd = oracle.q4_0_matmul(x, B, N, K)
    check_tol(gemv(x, B, N), ref, bnd, TOL, f"M={M} K={K} N={N}")


def test_gemv_rejects_mismatched_tensors():
    from moe_experts_amd import q4_0_gemv
    x = torch.zeros((1, 64), device=dev())
    B = torch.zeros((64 * 2 * 18 - 1,), dtype=torch.uint8, device=dev())
    with pytest.raises(ValueError):
        q4_0_gemv(x, B, 64)
    with pytest.raises(TypeError):
        q4_0_gemv(x.double(), torch.zeros((64 * 2 * 18,), dtype=torch.uint8, device=dev()), 64)
