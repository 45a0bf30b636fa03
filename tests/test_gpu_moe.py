"""GPU parity of moe_q4_0_decode against the CPU oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from moe_experts_amd import datagen
from tests.gpu_util import (check_route_table, check_tol, guarded, guarded_ws, guards_intact,
                            to_dev, to_host, ws_guards_intact)

pytestmark = pytest.mark.gpu
TOL = 1e-4


def moe_gpu(x, Wg, Wu, Wd, ids, w, I, E, dev_w=None):
    from moe_experts_amd import moe_q4_0_decode
    g, u, d = dev_w if dev_w is not None else (to_dev(Wg), to_dev(Wu), to_dev(Wd))
    return to_host(moe_q4_0_decode(to_dev(x), g, u, d, to_dev(ids.astype(np.int32)),
                                   to_dev(w.astype(np.float32)), I, E))


def moe_gpu_guarded(x, dw, ids, w, I, E):
    """moe_q4_0_decode with sentinel bands around out and around the workspace;
    checks the bands and returns (out, host copy of the workspace)."""
    from moe_experts_amd import moe_q4_0_decode, moe_q4_0_workspace_bytes
    T, H = x.shape
    topk = ids.shape[1]
    need = moe_q4_0_workspace_bytes(T, H, I, E, topk)
    wsfull, ws = guarded_ws(need)
    ofull, out = guarded(T * H)
    moe_q4_0_decode(to_dev(x), *dw, to_dev(ids.astype(np.int32)), to_dev(w.astype(np.float32)),
                    I, E, out=out, ws=ws)
    got = to_host(out).reshape(T, H)
    assert guards_intact(ofull, T * H), "write outside out"
    assert ws_guards_intact(wsfull, need), "write outside the workspace"
    return got, to_host(ws)


def small_experts(seed, H, I, E):
    Wg = np.stack([datagen.q4_0_random(seed + 3 * e, H, I) for e in range(E)])
    Wu = np.stack([datagen.q4_0_random(seed + 3 * e + 1, H, I) for e in range(E)])
    Wd = np.stack([datagen.q4_0_random(seed + 3 * e + 2, I, H) for e in range(E)])
    return Wg, Wu, Wd


@pytest.mark.parametrize("T,H,I,E,topk", [(1, 64, 32, 5, 1), (3, 64, 32, 5, 2), (17, 96, 64, 4, 6),
                                          (5, 320, 160, 7, 3), (64, 64, 64, 3, 8), (2, 1024, 512, 9, 6),
                                          (9, 768, 256, 6, 4), (33, 512, 768, 12, 6),
                                          (1, 512, 256, 6, 4), (1, 1024, 768, 9, 6),
                                          # long down K: the combine sums 6, 16 and 17 splits
                                          (2, 64, 4608, 3, 2), (1, 64, 13056, 3, 2),
                                          (2, 64, 13056, 3, 2)])
def test_moe_small_match_oracle(T, H, I, E, topk):
    x = datagen.activations(T * 7 + H, T, H)
    Wg, Wu, Wd = small_experts(100 * E + I, H, I, E)
    ids, w, _ = datagen.routing(T + E, T, E, topk)
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E)
    check_tol(moe_gpu(x, Wg, Wu, Wd, ids, w, I, E), ref, bnd, TOL, f"T={T} E={E} topk={topk}")


def test_moe_duplicates_out_of_range_and_crowded_expert():
    T, H, I, E, topk = 20, 128, 64, 6, 4
    x = datagen.activations(1, T, H)
    Wg, Wu, Wd = small_experts(7, H, I, E)
    g = np.random.Generator(np.random.PCG64(3))
    ids = g.integers(0, E, size=(T, topk)).astype(np.int32)
    ids[:, 0] = 2                    # every token uses expert 2: 20 pairs -> 3 matrix-core items
    ids[0, 1] = ids[0, 2] = 5        # a duplicate within a token
    ids[1, 3] = E + 3                # out of range -> contributes nothing
    ids[2, 2] = -1
    w = g.random((T, topk)).astype(np.float32)
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E)
    got = moe_gpu(x, Wg, Wu, Wd, ids, w, I, E)
    check_tol(got, ref, bnd, TOL, "edge routing")


@pytest.mark.parametrize("T,H,I,E,topk", [(2, 64, 32, 5, 2), (17, 96, 64, 4, 6), (64, 64, 64, 3, 8),
                                          (33, 512, 768, 12, 6), (40, 128, 96, 160, 6),
                                          (64, 64, 64, 1024, 8)])  # every limit at once
def test_moe_route_table_and_guards(T, H, I, E, topk):
    """The grouping step (pairs -> per-expert items) recomputed on the host from
    the ids matches the table the call left in its workspace; out and the
    workspace are written only inside their bounds."""
    x = datagen.activations(T * 3 + I, T, H)
    Wg, Wu, Wd = small_experts(11 * E + H, H, I, E)
    ids, w, _ = datagen.routing(7 * T + E, T, E, topk)
    ids[0, 0] = -1                   # an invalid id appears in no item
    if T > 3:
        ids[1, :] = ids[2, 0]        # a token with every slot on one expert (duplicates)
    got, ws = moe_gpu_guarded(x, (to_dev(Wg), to_dev(Wu), to_dev(Wd)), ids, w, I, E)
    check_route_table(ws, ids, T, H, I, E)
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E)
    check_tol(got, ref, bnd, TOL, f"T={T} E={E} topk={topk}")


@pytest.mark.parametrize("H,I", [(256, 128), (320, 96)])
def test_moe_batch_invariance_across_item_kinds(H, I):
    """Experts chosen by 3+ pairs run on the matrix-core tiles, by 1-2 pairs on
    the vector tiles; a token's output must be bitwise the same either way."""
    T, E, topk = 12, 4, 2
    x = datagen.activations(H + I, T, H)
    Wg, Wu, Wd = small_experts(5 * H + I, H, I, E)
    ids, w, _ = datagen.routing(H, T, E, topk)
    got = moe_gpu(x, Wg, Wu, Wd, ids, w, I, E)
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E)
    check_tol(got, ref, bnd, TOL, "12 tokens on 4 experts")
    counts = np.bincount(ids.reshape(-1), minlength=E)
    assert counts.max() >= 3  # some expert takes the matrix-core path
    for t in range(T):
        sel = [t, (t + 5) % T]
        pair = moe_gpu(x[sel], Wg, Wu, Wd, ids[sel], w[sel], I, E)
        assert (pair[0] == got[t]).all(), f"token {t} differs in a batch of 2 vs 12"


def test_moe_all_ids_invalid_gives_zero():
    T, H, I, E, topk = 2, 64, 32, 3, 2
    x = datagen.activations(2, T, H)
    Wg, Wu, Wd = small_experts(9, H, I, E)
    ids = np.full((T, topk), E, dtype=np.int32)
    w = np.ones((T, topk), dtype=np.float32)
    assert (moe_gpu(x, Wg, Wu, Wd, ids, w, I, E) == 0).all()


@pytest.fixture(scope="module")
def dsv2_experts():
    c = datagen.MOE_DSV2
    Wg, Wu, Wd = datagen.moe_experts(c["H"], c["I"], c["E"])
    return (Wg, Wu, Wd), (to_dev(Wg), to_dev(Wu), to_dev(Wd))


def test_moe_dsv2_single_token(dsv2_experts):
    c, t1 = datagen.MOE_DSV2, datagen.MOE_T1
    (Wg, Wu, Wd), dw = dsv2_experts
    x = datagen.activations(t1["x_seed"], 1, c["H"])
    ids, w, _ = datagen.routing(t1["logit_seed"], 1, c["E"], c["topk"])
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, c["H"], c["I"], c["E"])
    got, _ = moe_gpu_guarded(x, dw, ids, w, c["I"], c["E"])
    check_tol(got, ref, bnd, TOL, "dsv2 T=1")
    again = moe_gpu(x, None, None, None, ids, w, c["I"], c["E"], dev_w=dw)
    assert (again == got).all()


@pytest.mark.parametrize("skewed", [False, True])
def test_moe_dsv2_32_tokens(dsv2_experts, skewed):
    c, t32 = datagen.MOE_DSV2, datagen.MOE_T32
    (Wg, Wu, Wd), dw = dsv2_experts
    T = t32["T"]
    x = datagen.activations(t32["x_seed"], T, c["H"])
    ids, w, _ = datagen.routing(t32["logit_seed"], T, c["E"], c["topk"],
                                hot_bias=t32["hot_bias"] if skewed else 0.0, n_hot=t32["n_hot"])
    got, ws = moe_gpu_guarded(x, dw, ids, w, c["I"], c["E"])
    check_route_table(ws, ids, T, c["H"], c["I"], c["E"])
    # every token against the oracle
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, c["H"], c["I"], c["E"])
    check_tol(got, ref, bnd, TOL, f"dsv2 T=32 skewed={skewed}")
    # batch invariance: every token is bitwise equal to the same token decoded
    # in a batch of two with another token
    for t in range(T):
        sel = [t, (t + 7) % T]
        pair = moe_gpu(x[sel], None, None, None, ids[sel], w[sel], c["I"], c["E"], dev_w=dw)
        assert (pair[0] == got[t]).all(), f"token {t} differs in a batch of 2 vs 32"
    # a token decoded alone (finer K splits) agrees with the oracle
    for t in (0, 31):
        alone = moe_gpu(x[t:t + 1], None, None, None, ids[t:t + 1], w[t:t + 1], c["I"], c["E"], dev_w=dw)
        ref, bnd, _ = oracle.moe_decode(x[t:t + 1], Wg, Wu, Wd, ids[t:t + 1], w[t:t + 1],
                                        c["H"], c["I"], c["E"])
        check_tol(alone, ref, bnd, TOL, f"dsv2 token {t} alone")
