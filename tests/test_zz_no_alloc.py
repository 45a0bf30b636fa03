"""q4_0_gemv_noalloc (the allocation-free entry point) against q4_0_gemv on
the GPU: same kernels, so the outputs must be identical, on two calls in a row
(the second smaller, so stale partial sums from the first would show), and
against the oracle's tolerance on the small case."""
import numpy as np
import pytest
import torch

import oracle
from moe_experts_amd import datagen
from tests.gpu_util import check_tol, dev, guarded, guards_intact, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = 1e-4


def run_both(M, K, N, seed):
    from moe_experts_amd import q4_0_gemv, q4_0_gemv_noalloc, q4_0_gemv_workspace_bytes
    x = datagen.activations(seed, M, K)
    B = datagen.q4_0_random(seed + 1, K, N)
    xd, Bd = to_dev(x), to_dev(B)
    want = to_host(q4_0_gemv(xd, Bd, N))
    buf, y = guarded(M * N)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    q4_0_gemv_noalloc(xd, Bd, N, y.view(M, N))
    after = torch.cuda.memory_allocated()
    torch.cuda.synchronize()
    got = to_host(y.view(M, N))
    assert guards_intact(buf, M * N), f"noalloc wrote outside y at M={M} K={K} N={N}"
    assert after == before, "noalloc allocated through torch"
    assert q4_0_gemv_workspace_bytes(M, N, K) > 0, "case must use the K-split partials"
    return x, B, got, want


def test_noalloc_matches_q4_0_gemv_on_two_calls():
    # first: the 7B gate/up shape at batch 8 (3.7 MiB of partials); second:
    # a smaller, ragged case that reuses the front of the same array
    cases = [(8, 4096, 11008, 8801), (3, 4097, 1056, 8802)]
    for i, (M, K, N, seed) in enumerate(cases):
        x, B, got, want = run_both(M, K, N, seed)
        np.testing.assert_array_equal(got, want, err_msg=f"call {i}: M={M} K={K} N={N}")
        if i == 1:
            ref, bnd = oracle.q4_0_matmul(x, B, N, K)
            check_tol(got, ref, bnd, TOL, f"noalloc M={M} K={K} N={N}")

