"""GPU parity of moe_q4_0_prefill (experts as grouped GEMMs on the fp16 matrix
cores) against the CPU oracle, which takes the same fp16 activations and keeps
every product and sum in double. Tolerance: the prefill GEMM's relative bound,
1e-2 * sum_slot |w| * sum_k |h_k * Wd[k][n]| + 1e-6 (each dequantized weight
and h are rounded to fp16 on the GPU)."""
import numpy as np
import pytest
import torch

import oracle
from moe_experts_amd import datagen
from tests.gpu_util import (check_prefill_route, check_tol, guarded, guarded_ws, guards_intact,
                            to_dev, to_host, ws_guards_intact)

pytestmark = pytest.mark.gpu
TOL = 1e-2


def prefill_gpu(x16, dw, ids, w, I, E):
    from moe_experts_amd import moe_q4_0_prefill
    return to_host(moe_q4_0_prefill(to_dev(x16), *dw, to_dev(ids.astype(np.int32)),
                                    to_dev(w.astype(np.float32)), I, E))


def experts(seed, H, I, E):
    Wg = np.stack([datagen.q4_0_random(seed + 3 * e, H, I) for e in range(E)])
    Wu = np.stack([datagen.q4_0_random(seed + 3 * e + 1, H, I) for e in range(E)])
    Wd = np.stack([datagen.q4_0_random(seed + 3 * e + 2, I, H) for e in range(E)])
    return (Wg, Wu, Wd), (to_dev(Wg), to_dev(Wu), to_dev(Wd))


# one token; several tokens per expert; several m-tiles per expert; every slot
# on one expert (duplicates, 6 tiles of one expert); wide I
@pytest.mark.parametrize("T,H,I,E,topk", [(1, 128, 128, 3, 1), (300, 256, 128, 6, 2),
                                          (513, 384, 256, 9, 6), (70, 128, 384, 1, 8),
                                          (40, 256, 640, 20, 4)])
def test_prefill_small_match_oracle(T, H, I, E, topk):
    x16 = datagen.to_f16(datagen.activations(T + H + I, T, H))
    (Wg, Wu, Wd), dw = experts(50 * E + I, H, I, E)
    if E > 1:
        ids, w, _ = datagen.routing(T + E + topk, T, E, topk)
    else:
        ids = np.zeros((T, topk), dtype=np.int32)
        w = np.random.Generator(np.random.PCG64(T)).random((T, topk)).astype(np.float32)
    got = prefill_gpu(x16, dw, ids, w, I, E)
    ref, bnd, _ = oracle.moe_decode(x16.astype(np.float32), Wg, Wu, Wd, ids, w, H, I, E)
    check_tol(got, ref, bnd, TOL, f"T={T} E={E} topk={topk}")
    assert (prefill_gpu(x16, dw, ids, w, I, E) == got).all()   # deterministic


def test_prefill_invalid_and_duplicate_ids():
    T, H, I, E, topk = 33, 128, 128, 4, 3
    x16 = datagen.to_f16(datagen.activations(5, T, H))
    (Wg, Wu, Wd), dw = experts(9, H, I, E)
    g = np.random.Generator(np.random.PCG64(6))
    ids = g.integers(0, E, size=(T, topk)).astype(np.int32)
    ids[0, :] = 2          # a token that picks one expert three times
    ids[1, 1] = -1         # invalid ids contribute zero
    ids[2, 2] = E + 5
    ids[3, :] = -3         # a token with no valid slot: zeros
    w = g.random((T, topk)).astype(np.float32)
    got = prefill_gpu(x16, dw, ids, w, I, E)
    ref, bnd, _ = oracle.moe_decode(x16.astype(np.float32), Wg, Wu, Wd, ids, w, H, I, E)
    check_tol(got, ref, bnd, TOL, "invalid/duplicate ids")
    assert (got[3] == 0).all()


def test_prefill_dsv2_shape():
    c = datagen.MOE_DSV2
    H, I, E, topk = c["H"], c["I"], c["E"], c["topk"]
    T = 256
    ids, w, _ = datagen.routing(5301, T, E, topk)
    used = sorted(set(ids.ravel().tolist()))
    Wg, Wu, Wd = datagen.moe_experts(H, I, E, experts=used)
    x16 = datagen.to_f16(datagen.activations(5101, T, H))
    got = prefill_gpu(x16, (to_dev(Wg), to_dev(Wu), to_dev(Wd)), ids, w, I, E)
    for t in (0, 77, T - 1):
        ref, bnd, _ = oracle.moe_decode(x16[t:t + 1].astype(np.float32), Wg, Wu, Wd,
                                        ids[t:t + 1], w[t:t + 1], H, I, E)
        check_tol(got[t:t + 1], ref, bnd, TOL, f"dsv2 prefill token {t}")


def expert_cover(ids, E, limit=64):
    """Greedy set cover: tokens (at most `limit`) whose routed experts together
    include every expert the routing uses."""
    need = set(int(e) for e in ids.ravel() if 0 <= e < E)
    chosen = []
    while need and len(chosen) < limit:
        t = max(range(ids.shape[0]), key=lambda t: len(need & set(ids[t].tolist())))
        chosen.append(t)
        need -= set(ids[t].tolist())
    assert not need, "no cover within the limit"
    return sorted(chosen)


def test_prefill_dsv2_2048_tokens_every_expert():
    """The benchmarked MoE prefill: 2048 tokens, DeepSeek-V2 experts, the
    benchmark's first routing table. A set of tokens that together use every
    routed expert is checked against the oracle; out is written only inside
    its bounds."""
    from moe_experts_amd import moe_q4_0_prefill
    c = datagen.MOE_DSV2
    H, I, E, topk = c["H"], c["I"], c["E"], c["topk"]
    T = 2048
    ids, w, _ = datagen.routing(5301, T, E, topk)
    Wg, Wu, Wd = datagen.moe_experts(H, I, E)
    x16 = datagen.to_f16(datagen.activations(5101, T, H))
    full, outv = guarded(T * H)
    moe_q4_0_prefill(to_dev(x16), to_dev(Wg), to_dev(Wu), to_dev(Wd), to_dev(ids.astype(np.int32)),
                     to_dev(w.astype(np.float32)), I, E, out=outv)
    got = to_host(outv).reshape(T, H)
    assert guards_intact(full, T * H), "write outside out"
    toks = expert_cover(ids, E)
    assert len(set(ids[toks].ravel().tolist())) == E
    ref, bnd, _ = oracle.moe_decode(x16[toks].astype(np.float32), Wg, Wu, Wd, ids[toks], w[toks],
                                    H, I, E)
    check_tol(got[toks], ref, bnd, TOL, f"dsv2 prefill T=2048, {len(toks)} tokens")
    assert np.isfinite(got).all()


# The routing the call leaves in its workspace, rebuilt on the host: one group
# of 64 pairs; several groups per wave; waves with no pairs; invalid ids; one
# expert taking every pair; the benchmarked 2048-token routing.
@pytest.mark.parametrize("T,E,topk,seed,bad", [(1, 3, 1, 1, False), (33, 4, 3, 6, True),
                                               (513, 9, 6, 11, True), (70, 1, 8, 2, False),
                                               (2048, 160, 6, 5301, False),
                                               (5000, 1024, 8, 12, True)])
def test_prefill_route_table(T, E, topk, seed, bad):
    from moe_experts_amd import moe_q4_0_prefill, moe_q4_0_prefill_workspace_bytes
    H, I = 128, 128
    if E > 1:
        ids, w, _ = datagen.routing(seed, T, E, topk)
    else:
        ids = np.zeros((T, topk), dtype=np.int32)
        w = np.ones((T, topk), dtype=np.float32)
    if bad:
        g = np.random.Generator(np.random.PCG64(seed))
        ids[g.random(ids.shape) < 0.05] = -1
        ids[g.random(ids.shape) < 0.05] = E + 3
    x16 = datagen.to_f16(datagen.activations(seed + 1, T, H))
    _, dw = experts(seed + 2, H, I, E)
    need = moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk)
    wsfull, ws = guarded_ws(need)
    moe_q4_0_prefill(to_dev(x16), *dw, to_dev(ids.astype(np.int32)), to_dev(w), I, E, ws=ws)
    assert ws_guards_intact(wsfull, need), "write outside the workspace"
    check_prefill_route(to_host(ws), ids, T, H, I, E)


@pytest.mark.slow
def test_prefill_at_the_token_limit():
    """65536 tokens (Q4_MOE_PREFILL_MAX_T) x 8 slots (the topk limit): 524288
    pairs, 512 groups of 64 per ranking wave, about 5500 m-tiles; out between guard
    bands; the routing rebuilt on the host; 64 tokens spread over the batch
    checked against the oracle."""
    from moe_experts_amd import moe_q4_0_prefill
    T, H, I, E, topk = 65536, 128, 128, 8, 8
    x16 = datagen.to_f16(datagen.activations(8101, T, H))
    (Wg, Wu, Wd), dw = experts(8102, H, I, E)
    ids, w, _ = datagen.routing(8103, T, E, topk)
    ofull, out = guarded(T * H)
    from moe_experts_amd import moe_q4_0_prefill_workspace_bytes
    ws = torch.empty(moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk), dtype=torch.uint8,
                     device=out.device)
    moe_q4_0_prefill(to_dev(x16), *dw, to_dev(ids.astype(np.int32)), to_dev(w.astype(np.float32)),
                     I, E, out=out.view(T, H), ws=ws)
    assert guards_intact(ofull, T * H), "write outside out"
    check_prefill_route(to_host(ws), ids, T, H, I, E)
    got = to_host(out).reshape(T, H)
    tok = np.linspace(0, T - 1, 64).astype(np.int64)
    ref, bnd, _ = oracle.moe_decode(x16[tok].astype(np.float32), Wg, Wu, Wd, ids[tok], w[tok],
                                    H, I, E)
    check_tol(got[tok], ref, bnd, TOL, "65536 tokens x 8 slots")
