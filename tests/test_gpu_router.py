"""GPU parity of the MoE router (moe_router_topk) and the whole layer
(moe_q4_0_layer: router, routed and shared experts) against the CPU oracle."""
import numpy as np
import pytest

import oracle
from moe_experts_amd import datagen
from tests.gpu_util import check_tol, guarded, guards_intact, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = 1e-4
# Softmax weights: expf within 2 ulp, at most 7 roundings in the sum of <= 8
# terms, one in the quotient: about 1.3e-6 relative; checked at 2e-6.
W_RTOL = 2e-6


def router_gpu(x, Wr, topk, n_shared):
    from moe_experts_amd import moe_router_topk
    lg, ids, w = moe_router_topk(to_dev(x), to_dev(Wr), topk, n_shared)
    return to_host(lg), to_host(ids), to_host(w)


def check_router(x, Wr, topk, n_shared, what):
    lg, ids, w = router_gpu(x, Wr, topk, n_shared)
    ref_lg, bnd = oracle.router_logits(x, Wr)
    fin = np.isfinite(ref_lg)
    check_tol(lg[fin], ref_lg[fin], bnd[fin], TOL, f"{what} logits")
    assert np.isnan(lg[~fin]).all(), f"{what}: a NaN logit came out finite"
    # the top-k decision is taken on the GPU's float logits on both sides
    ref_ids, ref_w = oracle.router_topk(lg, topk, n_shared)
    assert (ids == ref_ids).all(), f"{what}: ids differ"
    assert np.all(np.abs(w.astype(np.float64) - ref_w) <= W_RTOL * np.abs(ref_w) + 1e-7), what
    return lg, ids, w


@pytest.mark.parametrize("T,H,E,topk,n_shared", [
    (1, 64, 5, 1, 0), (3, 256, 40, 6, 2), (17, 516, 160, 6, 2), (2, 4, 3, 3, 0),
    (64, 1024, 1024, 8, 0), (33, 5120, 160, 6, 2), (1, 5120, 160, 6, 2), (5, 1284, 77, 4, 4)])
def test_router_matches_oracle(T, H, E, topk, n_shared):
    x = datagen.activations(T + 11 * H, T, H)
    Wr = datagen.router_weights(E + H, E, H)
    check_router(x, Wr, topk, n_shared, f"T={T} H={H} E={E} topk={topk}")


def test_router_ties_and_nan():
    T, H, E, topk = 6, 256, 12, 5
    x = datagen.activations(9, T, H)
    Wr = datagen.router_weights(10, E, H)
    Wr[7] = Wr[3]          # experts 3 and 7 tie for every token: 3 comes first
    Wr[9] = Wr[3]
    Wr[5, 17] = np.nan     # expert 5's logit is NaN: never chosen
    x[2] = 0.0             # token 2: all logits +0.0 except the NaN: ids 0,1,2,3,4
    lg, ids, w = check_router(x, Wr, topk, 1, "ties/NaN")
    assert not (ids[:, :topk] == 5).any()
    assert ids[2].tolist() == [0, 1, 2, 3, 4, E]
    assert np.all(np.abs(w[2, :topk] - 0.2) <= 1e-7)
    for t in range(T):
        row = ids[t, :topk].tolist()
        if 7 in row:
            assert 3 in row and row.index(3) < row.index(7)


def layer_gpu(x, Wr, dw, I, topk, n_shared):
    from moe_experts_amd import moe_q4_0_layer
    return to_host(moe_q4_0_layer(to_dev(x), to_dev(Wr), *dw, I, topk, n_shared))


@pytest.mark.parametrize("T,H,I,E,topk,n_shared", [(1, 256, 64, 6, 2, 1), (12, 320, 96, 8, 3, 2),
                                                   (40, 128, 64, 5, 2, 2), (7, 512, 256, 20, 6, 2)])
def test_layer_small_matches_oracle(T, H, I, E, topk, n_shared):
    from moe_experts_amd import moe_q4_0_decode
    x = datagen.activations(T + H, T, H)
    Wr = datagen.router_weights(H + I, E, H)
    Es = E + n_shared
    Wg = np.stack([datagen.q4_0_random(7 * e + 1, H, I) for e in range(Es)])
    Wu = np.stack([datagen.q4_0_random(7 * e + 2, H, I) for e in range(Es)])
    Wd = np.stack([datagen.q4_0_random(7 * e + 3, I, H) for e in range(Es)])
    dw = (to_dev(Wg), to_dev(Wu), to_dev(Wd))
    got = layer_gpu(x, Wr, dw, I, topk, n_shared)
    _, ids, w = check_router(x, Wr, topk, n_shared, "layer router")
    # the layer is the router followed by the decode over routed + shared experts
    dec = to_host(moe_q4_0_decode(to_dev(x), *dw, to_dev(ids), to_dev(w), I, Es))
    assert (got == dec).all()
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, Es)
    check_tol(got, ref, bnd, TOL, f"layer T={T}")


@pytest.fixture(scope="module")
def dsv2_layer():
    c, L = datagen.MOE_DSV2, datagen.MOE_LAYER
    Es = c["E"] + L["n_shared"]
    Wg, Wu, Wd = datagen.moe_experts(c["H"], c["I"], Es)
    Wr = datagen.router_weights(L["router_seed"], c["E"], c["H"])
    return (Wg, Wu, Wd), (to_dev(Wg), to_dev(Wu), to_dev(Wd)), Wr


@pytest.mark.parametrize("T", [1, 32])
def test_layer_dsv2(dsv2_layer, T):
    c, L = datagen.MOE_DSV2, datagen.MOE_LAYER
    (Wg, Wu, Wd), dw, Wr = dsv2_layer
    seed = datagen.MOE_T1["x_seed"] if T == 1 else datagen.MOE_T32["x_seed"]
    x = datagen.activations(seed, T, c["H"])
    _, ids, w = check_router(x, Wr, c["topk"], L["n_shared"], f"dsv2 router T={T}")
    from moe_experts_amd import moe_q4_0_layer
    full, outv = guarded(T * c["H"])
    moe_q4_0_layer(to_dev(x), to_dev(Wr), *dw, c["I"], c["topk"], L["n_shared"], out=outv)
    got = to_host(outv).reshape(T, c["H"])
    assert guards_intact(full, T * c["H"]), "write outside out"
    Es = c["E"] + L["n_shared"]
    # every token against the oracle (routed + shared experts)
    ref, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, c["H"], c["I"], Es)
    check_tol(got, ref, bnd, TOL, f"dsv2 layer T={T}")


def test_router_outputs_stay_in_bounds():
    """logits, ids and weights are written only inside their bounds."""
    import torch
    from moe_experts_amd import moe_router_topk
    T, H, E, topk, n_shared = 33, 5120, 160, 6, 2
    x = datagen.activations(5, T, H)
    Wr = datagen.router_weights(6, E, H)
    slots = topk + n_shared
    lf, lv = guarded(T * E)
    wf, wv = guarded(T * slots)
    idf, idv = guarded(T * slots, dtype=torch.int32, fill=-77)
    moe_router_topk(to_dev(x), to_dev(Wr), topk, n_shared, logits=lv, ids=idv, w=wv)
    assert guards_intact(lf, T * E) and guards_intact(wf, T * slots)
    assert guards_intact(idf, T * slots, fill=-77)
    ref_ids, ref_w = oracle.router_topk(to_host(lv).reshape(T, E), topk, n_shared)
    assert (to_host(idv).reshape(T, slots) == ref_ids).all()
