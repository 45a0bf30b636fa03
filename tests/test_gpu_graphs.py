"""Every entry point enqueues only kernel launches (no host synchronization,
allocation or memset), so a call can be captured in a HIP graph. Each capture
here is replayed several times, with new inputs copied into the captured
buffers and eager work between the replays, and every replay must equal the
eager call bitwise."""
import numpy as np
import pytest
import torch

from moe_experts_amd import datagen
from tests.gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


def replay_check(fn, inputs, new_inputs, out):
    """Capture fn() (which reads `inputs` and writes `out`), then for each set
    in new_inputs: copy it into `inputs`, replay, and compare with an eager
    call on the same data."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for vals in new_inputs:
        for buf, v in zip(inputs, vals):
            buf.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out.fill_(float("nan"))   # eager work between replays
        fn()
        torch.cuda.synchronize()
        assert torch.equal(got, out)


def test_graph_replays_gemv_and_q8():
    from moe_experts_amd import q4_0_gemv, q8_0_gemv
    for M, kind in ((1, 4), (8, 4), (3, 8)):
        K, N = 1024, 2048
        B = to_dev(datagen.q4_0_random(1, K, N) if kind == 4 else datagen.q8_0_random(1, K, N))
        x = to_dev(datagen.activations(2, M, K))
        y = torch.empty((M, N), dtype=torch.float32, device=dev())
        f = q4_0_gemv if kind == 4 else q8_0_gemv
        replay_check(lambda: f(x, B, N, y=y), [x],
                     [[to_dev(datagen.activations(s, M, K))] for s in (3, 4, 5)], y)


def test_graph_replays_moe_decode_layer_and_prefill():
    from moe_experts_amd import moe_q4_0_decode, moe_q4_0_layer, moe_q4_0_prefill
    T, H, I, E, topk = 12, 256, 128, 6, 2
    Wg = to_dev(np.stack([datagen.q4_0_random(10 + 3 * e, H, I) for e in range(E + 1)]))
    Wu = to_dev(np.stack([datagen.q4_0_random(11 + 3 * e, H, I) for e in range(E + 1)]))
    Wd = to_dev(np.stack([datagen.q4_0_random(12 + 3 * e, I, H) for e in range(E + 1)]))
    mat = H * (I // 32) * 18
    gE, uE, dE = (w.view(-1)[:E * mat] for w in (Wg, Wu, Wd))
    x = to_dev(datagen.activations(1, T, H))
    ids0, w0, _ = datagen.routing(2, T, E, topk)
    ids, w = to_dev(ids0), to_dev(w0)
    out = torch.empty((T, H), dtype=torch.float32, device=dev())
    sets = []
    for s in (3, 4, 5):
        i2, w2, _ = datagen.routing(s, T, E, topk)
        sets.append([to_dev(datagen.activations(s, T, H)), to_dev(i2), to_dev(w2)])
    replay_check(lambda: moe_q4_0_decode(x, gE, uE, dE, ids, w, I, E, out=out),
                 [x, ids, w], sets, out)
    Wr = to_dev(datagen.router_weights(6, E, H))
    replay_check(lambda: moe_q4_0_layer(x, Wr, Wg, Wu, Wd, I, topk, 1, out=out), [x],
                 [[to_dev(datagen.activations(s, T, H))] for s in (7, 8)], out)
    x16 = to_dev(datagen.to_f16(datagen.activations(9, T, H)))
    replay_check(lambda: moe_q4_0_prefill(x16, gE, uE, dE, ids, w, I, E, out=out),
                 [x16, ids, w],
                 [[to_dev(datagen.to_f16(datagen.activations(s, T, H))), st[1], st[2]]
                  for s, st in zip((10, 11), sets)], out)
