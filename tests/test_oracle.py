"""Pins of the CPU oracle against things other than itself (runs on the CPU).

Each test names what fixes the expected value: a hand-worked fixture derived
from the pages, the IEEE definition (checked against numpy's float16), an
integer-exact special case checked against numpy's matmul, or an invariant
that the mathematics fixes.
"""
import math

import numpy as np
import pytest

import oracle
from moe_experts_amd import datagen
from tests.golden_io import fp16_patterns, gemv_cases, handworked_block, same_float


def _block(d_bits: int, qs: bytes) -> bytes:
    return bytes([d_bits & 0xFF, d_bits >> 8]) + qs


# --------------------------------------------------------------------------
# binary16 decode
# --------------------------------------------------------------------------

def test_fp16_decode_handworked_patterns():
    for bits, val in fp16_patterns():
        got = oracle.fp16_to_double(bits)
        assert same_float(got, val), (hex(bits), got, val)


def test_fp16_decode_all_patterns_match_numpy():
    # numpy's float16 -> float64 conversion is an independent implementation.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


# --------------------------------------------------------------------------
# Block decode (dequantize)
# --------------------------------------------------------------------------

def test_dequant_handworked_block_all_nibbles_both_positions():
    qs, qm8, ds, checks = handworked_block()
    assert sorted(qm8[0::2]) == list(range(-8, 8)) and sorted(qm8[1::2]) == list(range(-8, 8))
    for d_bits, d_val in ds.items():
        got = oracle.dequant_block(_block(d_bits, qs))
        for l in range(32):
            assert got[l] == qm8[l] * d_val, (hex(d_bits), l, got[l])
    for d_bits, idx, val in checks:
        assert oracle.dequant_block(_block(d_bits, qs))[idx] == val


def test_dequant_zero_scale_signs():
    qs, _, _, _ = handworked_block()
    assert (oracle.dequant_block(_block(0x0000, qs)) == 0).all()
    assert (oracle.dequant_block(_block(0x8000, qs)) == 0).all()


def test_dequant_rows_layout_blocks_along_columns():
    # Row k, block j covers columns 32j..32j+31 (article §3.4 indexing).
    qs, qm8, _, _ = handworked_block()
    K, N = 3, 96
    B = np.zeros((K, N // 32, 18), dtype=np.uint8)
    for k in range(K):
        for j in range(N // 32):
            d_bits = [0x3C00, 0x3800, 0xBC00][(k + j) % 3]
            B[k, j] = np.frombuffer(_block(d_bits, qs), dtype=np.uint8)
    W = oracle.dequant_rows(B, N, 0, K)
    scale = {0: 1.0, 1: 0.5, 2: -1.0}
    for k in range(K):
        for j in range(N // 32):
            s = scale[(k + j) % 3]
            assert (W[k, 32 * j:32 * j + 32] == np.array(qm8, dtype=np.float32) * s).all()


# --------------------------------------------------------------------------
# GEMV / matmul
# --------------------------------------------------------------------------

def _handworked_matrix():
    qs, qm8, _, _ = handworked_block()
    B = np.stack([np.frombuffer(_block(0x3C00, qs), dtype=np.uint8),
                  np.frombuffer(_block(0x3800, qs), dtype=np.uint8)]).reshape(2, 1, 18)
    return B


def test_handworked_gemv():
    B = _handworked_matrix()
    for xs, ys in gemv_cases():
        y, bnd = oracle.q4_0_matmul(np.array([xs], dtype=np.float32), B, 32, 2)
        assert (y[0] == np.array(ys, dtype=np.float32)).all(), y
        assert (bnd[0] >= np.abs(y[0])).all()


def _int_case(seed, M, K, N, d_choices=(0x3C00,)):
    """Integer-exact case: x in [-4, 4], nibbles uniform, d a power of two."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.integers(0, 16, size=(K, N), dtype=np.uint8)
    d_bits = g.choice(np.array(d_choices, dtype=np.uint16), size=(K, N // 32))
    B = datagen.assemble(d_bits, datagen.pack_nibbles(q))
    x = g.integers(-4, 5, size=(M, K)).astype(np.float32)
    d = d_bits.view(np.float16).astype(np.float64)
    W = (q.astype(np.float64) - 8.0) * np.repeat(d, 32, axis=1)
    return x, B, W


@pytest.mark.parametrize("M,K,N", [(1, 1, 32), (3, 7, 64), (2, 33, 96), (8, 130, 256)])
def test_matmul_integer_exact_matches_numpy(M, K, N):
    x, B, W = _int_case(100 + M * K, M, K, N, d_choices=(0x3C00, 0x3800, 0x4000, 0xB400))
    y, _ = oracle.q4_0_matmul(x, B, N, K)
    ref = x.astype(np.float64) @ W   # every partial sum is exact here
    assert (y == ref.astype(np.float32)).all()


def test_matmul_random_close_to_numpy_float64():
    # Brute force against numpy on a dense float64 copy of the dequantized matrix.
    M, K, N = 3, 45, 160
    x = datagen.activations(7, M, K)
    B = datagen.q4_0_random(8, K, N)
    W = oracle.dequant_rows(B, N, 0, K).astype(np.float64)
    y, bnd = oracle.q4_0_matmul(x, B, N, K)
    ref = x.astype(np.float64) @ W
    assert np.allclose(y, ref, rtol=0, atol=1e-6 * bnd.max())
    assert (np.abs(y - ref) <= 1e-7 * bnd + 1e-30).all()


def test_matmul_one_hot_selects_dequantized_row():
    K, N = 9, 64
    B = datagen.q4_0_random(11, K, N)
    W = oracle.dequant_rows(B, N, 0, K)
    for k in (0, 4, 8):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y, _ = oracle.q4_0_matmul(x, B, N, K)
        assert (y[0] == W[k]).all()


def test_matmul_invariants():
    M, K, N = 2, 40, 96
    x = datagen.activations(21, M, K)
    B = datagen.q4_0_random(22, K, N)
    y, bnd = oracle.q4_0_matmul(x, B, N, K)
    # zero scales -> zero output
    Bz = B.copy(); Bz[..., 0:2] = 0
    assert (oracle.q4_0_matmul(x, Bz, N, K)[0] == 0).all()
    # all nibbles 8 -> zero output
    B8 = B.copy(); B8[..., 2:] = 0x88
    assert (oracle.q4_0_matmul(x, B8, N, K)[0] == 0).all()
    # doubling every scale (binary16 exponent + 1) doubles y exactly
    d = B[..., 0:2].copy().view(np.uint16)[..., 0]
    B2 = datagen.assemble(d + 0x0400, B[..., 2:])
    assert (oracle.q4_0_matmul(x, B2, N, K)[0] == 2 * y).all()
    # scaling x by 2^-3 scales y exactly
    assert (oracle.q4_0_matmul(x * np.float32(0.125), B, N, K)[0] == y * np.float32(0.125)).all()
    # changing block (k, j) changes only columns 32j..32j+31
    Bc = B.copy(); Bc[5, 1, 2:] ^= 0x5A
    yc = oracle.q4_0_matmul(x, Bc, N, K)[0]
    changed = np.nonzero((yc != y).any(axis=0))[0]
    assert changed.size > 0 and changed.min() >= 32 and changed.max() < 64
    # linearity in x (within double-then-float rounding)
    x2 = datagen.activations(23, M, K)
    ya = oracle.q4_0_matmul(x + x2, B, N, K)[0]
    yb = y + oracle.q4_0_matmul(x2, B, N, K)[0]
    b2 = oracle.q4_0_matmul(np.abs(x) + np.abs(x2), B, N, K)[1]
    assert (np.abs(ya - yb) <= 1e-6 * b2).all()
    # the bound dominates |y|; it equals y when every term is non-negative
    assert (bnd >= np.abs(y) * (1 - 1e-7)).all()
    Bp = B.copy(); Bp[..., 2:] |= 0x88            # nibbles >= 8 -> w >= 0
    yp, bp = oracle.q4_0_matmul(np.abs(x), Bp, N, K)
    assert np.allclose(yp, bp, rtol=1e-7, atol=0)


def test_matmul_row_permutation_within_tolerance():
    M, K, N = 1, 64, 64
    x = datagen.activations(31, M, K)
    B = datagen.q4_0_random(32, K, N)
    perm = np.random.Generator(np.random.PCG64(33)).permutation(K)
    y, bnd = oracle.q4_0_matmul(x, B, N, K)
    yp, _ = oracle.q4_0_matmul(x[:, perm], B[perm], N, K)
    assert (np.abs(y - yp) <= 1e-6 * bnd).all()


def test_matmul_f16_equals_fp32_path_on_f16_values():
    M, K, N = 4, 64, 128
    x16 = datagen.to_f16(datagen.activations(41, M, K))
    B = datagen.q4_0_random(42, K, N)
    y16, b16 = oracle.q4_0_matmul_f16(x16, B, N, K)
    y32, b32 = oracle.q4_0_matmul(x16.astype(np.float32), B, N, K)
    assert (y16 == y32).all() and (b16 == b32).all()


def test_matmul_rejects_bad_shapes():
    B = datagen.q4_0_random(1, 2, 32)
    with pytest.raises(ValueError):
        oracle.dequant_rows(B, 33, 0, 1)


# --------------------------------------------------------------------------
# MoE decode
# --------------------------------------------------------------------------

def _expit(z):
    from scipy.special import expit   # library logistic function
    return expit(z)


def _ffn_reference(x, Wg, Wu, Wd, e, H, I):
    """Expert FFN from library pieces: numpy matmul on the dequantized float64
    matrices and scipy's logistic function for SiLU(z) = z * sigmoid(z)."""
    G = oracle.dequant_rows(Wg[e], I, 0, H).astype(np.float64)
    U = oracle.dequant_rows(Wu[e], I, 0, H).astype(np.float64)
    D = oracle.dequant_rows(Wd[e], H, 0, I).astype(np.float64)
    g = x.astype(np.float64) @ G
    u = x.astype(np.float64) @ U
    h = g * _expit(g) * u
    return h @ D, h


def _small_moe(seed=5, T=3, H=64, I=32, E=5, topk=2):
    x = datagen.activations(seed, T, H)
    Wg = np.stack([datagen.q4_0_random(seed * 100 + 3 * e, H, I) for e in range(E)])
    Wu = np.stack([datagen.q4_0_random(seed * 100 + 3 * e + 1, H, I) for e in range(E)])
    Wd = np.stack([datagen.q4_0_random(seed * 100 + 3 * e + 2, I, H) for e in range(E)])
    ids, w, _ = datagen.routing(seed + 1, T, E, topk)
    return x, Wg, Wu, Wd, ids, w


def test_moe_matches_library_composition():
    H, I, E = 64, 32, 5
    x, Wg, Wu, Wd, ids, w = _small_moe(H=H, I=I, E=E)
    out, bnd, h = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E, with_h=True)
    for t in range(x.shape[0]):
        ref = np.zeros(H)
        for j in range(ids.shape[1]):
            yd, hr = _ffn_reference(x[t], Wg, Wu, Wd, ids[t, j], H, I)
            assert np.allclose(h[t, j], hr, rtol=1e-12, atol=1e-15)
            ref += np.float64(w[t, j]) * yd
        assert (np.abs(out[t] - ref) <= 1e-6 * bnd[t] + 1e-12).all()


def test_moe_single_slot_unit_weight_is_the_expert_ffn():
    H, I, E = 64, 64, 3
    x, Wg, Wu, Wd, _, _ = _small_moe(seed=9, T=2, H=H, I=I, E=E)
    ids = np.array([[2], [0]], dtype=np.int32)
    w = np.ones((2, 1), dtype=np.float32)
    out, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E)
    for t in range(2):
        ref, _ = _ffn_reference(x[t], Wg, Wu, Wd, ids[t, 0], H, I)
        assert (np.abs(out[t] - ref) <= 1e-6 * bnd[t] + 1e-12).all()


def test_moe_invariants():
    H, I, E, topk = 64, 32, 4, 3
    x, Wg, Wu, Wd, ids, w = _small_moe(seed=13, T=2, H=H, I=I, E=E, topk=topk)
    out, bnd, _ = oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E)
    # same expert in every slot -> (sum of weights) * FFN
    same = np.full_like(ids, 1)
    o2, b2, _ = oracle.moe_decode(x, Wg, Wu, Wd, same, w, H, I, E)
    for t in range(2):
        ref, _ = _ffn_reference(x[t], Wg, Wu, Wd, 1, H, I)
        assert (np.abs(o2[t] - w[t].astype(np.float64).sum() * ref) <= 1e-6 * b2[t] + 1e-12).all()
    # an out-of-range id contributes nothing
    bad = ids.copy(); bad[:, 1] = E + 7
    keep = w.copy(); keep[:, 1] = 0
    assert (oracle.moe_decode(x, Wg, Wu, Wd, bad, w, H, I, E)[0]
            == oracle.moe_decode(x, Wg, Wu, Wd, ids, keep, H, I, E)[0]).all()
    neg = ids.copy(); neg[:, 0] = -1
    keep0 = w.copy(); keep0[:, 0] = 0
    assert (oracle.moe_decode(x, Wg, Wu, Wd, neg, w, H, I, E)[0]
            == oracle.moe_decode(x, Wg, Wu, Wd, ids, keep0, H, I, E)[0]).all()
    # doubling every routing weight doubles the output exactly
    assert (oracle.moe_decode(x, Wg, Wu, Wd, ids, 2 * w, H, I, E)[0] == 2 * out).all()
    # doubling every down-projection scale doubles the output exactly
    d = Wd[..., 0:2].copy().view(np.uint16)[..., 0]
    Wd2 = datagen.assemble(d + 0x0400, Wd[..., 2:])
    assert (oracle.moe_decode(x, Wg, Wu, Wd2, ids, w, H, I, E)[0] == 2 * out).all()
    # slot order does not matter beyond rounding
    p = ids[:, ::-1].copy(); pw = w[:, ::-1].copy()
    op, _, _ = oracle.moe_decode(x, Wg, Wu, Wd, p, pw, H, I, E)
    assert (np.abs(op - out) <= 1e-6 * bnd + 1e-12).all()
    # tokens are independent: token 1 alone equals token 1 in the batch
    o1, _, _ = oracle.moe_decode(x[1:], Wg, Wu, Wd, ids[1:], w[1:], H, I, E)
    assert (o1[0] == out[1]).all()


def test_moe_silu_gate_closed_form_points():
    # One-hot x picks row 0 of gate/up, so g and u are single dequantized weights.
    # With u = 1 and g = 0 the slot contributes nothing (SiLU(0) = 0); with
    # g = 2 (nibble 10, d = 1) h = 2 * sigmoid(2) = 2 / (1 + e^-2).
    H, I, E = 32, 32, 1
    x = np.zeros((1, H), dtype=np.float32); x[0, 0] = 1.0
    qg = np.full((H, I), 8, dtype=np.uint8); qg[0, 0] = 10; qg[0, 1] = 8
    qu = np.full((H, I), 8, dtype=np.uint8); qu[0, :] = 9
    qd = np.full((I, H), 8, dtype=np.uint8); qd[0, :] = 9     # yd[n] = h[0]
    one = lambda r, c: np.full((r, c // 32), 0x3C00, dtype=np.uint16)
    Wg = datagen.assemble(one(H, I), datagen.pack_nibbles(qg))[None]
    Wu = datagen.assemble(one(H, I), datagen.pack_nibbles(qu))[None]
    Wd = datagen.assemble(one(I, H), datagen.pack_nibbles(qd))[None]
    out, _, h = oracle.moe_decode(x, Wg, Wu, Wd, np.zeros((1, 1), np.int32),
                                  np.ones((1, 1), np.float32), H, I, E, with_h=True)
    assert h[0, 0, 1] == 0.0
    assert abs(h[0, 0, 0] - 2.0 / (1.0 + math.exp(-2.0))) <= 1e-15
    assert (out[0] == np.float32(2.0 / (1.0 + math.exp(-2.0)))).all()


# --------------------------------------------------------------------------
# Harness routing (input preparation, shared by both sides)
# --------------------------------------------------------------------------

def test_routing_topk_ties_and_softmax():
    logits = np.array([[0.5, 2.0, 2.0, -1.0, 2.0]], dtype=np.float32)
    ids, w = datagen.topk_softmax(logits, 3)
    assert ids.tolist() == [[1, 2, 4]]
    assert np.allclose(w, 1.0 / 3.0) and abs(float(w.sum()) - 1.0) < 1e-6
    ids, w, _ = datagen.routing(4201, 32, 160, 6, hot_bias=2.0)
    assert ids.shape == (32, 6) and (np.diff(np.take_along_axis(
        datagen.routing(4201, 32, 160, 6, hot_bias=2.0)[2], ids, 1), axis=1) <= 0).all()
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert (ids < 8).sum() > (32 * 6) * 8 / 160 * 3   # the hot experts dominate


def test_generator_layout_and_ranges():
    B = datagen.q4_0_random(1201, 64, 4096)
    assert B.shape == (64, 128, 18) and B.dtype == np.uint8
    d = B[..., 0:2].copy().view(np.uint16)[..., 0].view(np.float16).astype(np.float64)
    assert d.min() >= 0.00099 and d.max() <= 0.0201
    nib = np.concatenate([(B[..., 2:] & 15).ravel(), (B[..., 2:] >> 4).ravel()])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16
    # deterministic from the seed
    assert (datagen.q4_0_random(1201, 64, 4096) == B).all()


# --------------------------------------------------------------------------
# Router: logits, top-k selection, softmax weights, shared-expert slots
# --------------------------------------------------------------------------

def test_router_logits_integer_exact_and_random():
    g = np.random.Generator(np.random.PCG64(71))
    # integer data: every partial sum is an integer below 2^24, so the double
    # sum is exact and must equal numpy's integer matmul bitwise
    x = g.integers(-4, 5, size=(3, 96)).astype(np.float32)
    Wr = g.integers(-7, 8, size=(10, 96)).astype(np.float32)
    lg, bnd = oracle.router_logits(x, Wr)
    ref = x.astype(np.int64) @ Wr.astype(np.int64).T
    assert (lg == ref.astype(np.float32)).all()
    xa, wa = np.abs(x.astype(np.int64)), np.abs(Wr.astype(np.int64))
    assert (bnd == (xa[:, None, :] * wa[None]).sum(-1)).all()
    # random data: within a few float ulps of numpy's float64 product
    x = g.standard_normal((5, 640)).astype(np.float32)
    Wr = (g.standard_normal((33, 640)) / np.sqrt(640)).astype(np.float32)
    lg, bnd = oracle.router_logits(x, Wr)
    ref = x.astype(np.float64) @ Wr.astype(np.float64).T
    assert np.all(np.abs(lg - ref) <= 1e-7 * bnd + 1e-30)


def test_router_topk_handworked():
    lg = np.array([[1.0, 3.0, 3.0, 2.0],            # tie: lower index first
                   [0.0, math.log(3.0), -5.0, -5.0],  # weights 3/4 and 1/4
                   [np.nan, 1.0, np.nan, np.nan],      # one candidate only
                   [np.nan, np.nan, np.nan, np.nan]],  # none
                  dtype=np.float32)
    ids, w = oracle.router_topk(lg, 2, n_shared=1)
    assert ids.tolist() == [[1, 2, 4], [1, 0, 4], [1, -1, 4], [-1, -1, 4]]
    assert w[0, :2].tolist() == [0.5, 0.5]
    assert abs(w[1, 0] - 0.75) <= 1e-7 and abs(w[1, 1] - 0.25) <= 1e-7
    assert w[2, :2].tolist() == [1.0, 0.0] and w[3, :2].tolist() == [0.0, 0.0]
    assert (w[:, 2] == 1.0).all()
    # -inf logits are still candidates (lower index first among equals)
    ids, w = oracle.router_topk(np.array([[-np.inf, 0.0, -np.inf]], np.float32), 2)
    assert ids.tolist() == [[1, 0]] and w.tolist() == [[1.0, 0.0]]


def test_router_topk_matches_stable_argsort_and_shift_invariance():
    g = np.random.Generator(np.random.PCG64(72))
    lg = g.standard_normal((40, 160)).astype(np.float32)
    lg[:4, 10:20] = 0.25          # rows with many equal logits
    ids, w = oracle.router_topk(lg, 6, n_shared=2)
    ref_ids, ref_w = datagen.topk_softmax(lg, 6)   # numpy stable argsort, float64 softmax
    assert (ids[:, :6] == ref_ids).all()
    assert np.all(np.abs(w[:, :6] - ref_w) <= 1e-7 * ref_w)
    assert (ids[:, 6:] == np.array([160, 161])).all() and (w[:, 6:] == 1.0).all()
    assert np.all(np.abs(w[:, :6].astype(np.float64).sum(1) - 1.0) <= 1e-6)
    assert (np.diff(np.take_along_axis(lg, ids[:, :6], 1), axis=1) <= 0).all()
    # on a grid of 2^-10 adding 1 to every logit is exact and changes nothing
    lq = (np.round(lg * 1024) / 1024).astype(np.float32)
    ids1, w1 = oracle.router_topk(lq, 6, n_shared=2)
    ids2, w2 = oracle.router_topk(lq + np.float32(1.0), 6, n_shared=2)
    assert (ids2 == ids1).all() and (w2 == w1).all()


# --------------------------------------------------------------------------
# Q8_0 (34-byte blocks: binary16 scale, 32 signed bytes; w = q * d)
# --------------------------------------------------------------------------

def test_q8_0_block_handworked():
    # weights -128, -120, ..., 120 (every eighth signed byte value, both signs)
    q = np.array([8 * l - 128 for l in range(32)], dtype=np.int8)
    blk = datagen.assemble_q8(np.uint16(0x3C00), q)      # d = 1.0
    assert oracle.q8_0_dequant_block(blk).tolist() == [float(8 * l - 128) for l in range(32)]
    blk = datagen.assemble_q8(np.uint16(0xB800), q)      # d = -0.5
    assert oracle.q8_0_dequant_block(blk).tolist() == [-0.5 * (8 * l - 128) for l in range(32)]
    # sign extension at the ends: bytes 0x7F, 0x80, 0xFF, 0x01 are 127, -128, -1, 1
    q = np.zeros(32, dtype=np.uint8)
    q[:4] = [0x7F, 0x80, 0xFF, 0x01]
    blk = datagen.assemble_q8(np.uint16(0x4000), q)      # d = 2.0
    assert oracle.q8_0_dequant_block(blk)[:5].tolist() == [254.0, -256.0, -2.0, 2.0, 0.0]
    # subnormal and zero scales
    assert oracle.q8_0_dequant_block(datagen.assemble_q8(np.uint16(0x0001), q))[0] == 127 * 2.0 ** -24
    assert not oracle.q8_0_dequant_block(datagen.assemble_q8(np.uint16(0x8000), q)).any()


def test_q8_0_matmul_integer_exact_and_invariants():
    g = np.random.Generator(np.random.PCG64(81))
    K, N, M = 96, 160, 3
    q = g.integers(-128, 128, size=(K, N // 32, 32)).astype(np.int8)
    d_bits = g.choice(np.array([0x3C00, 0x3800, 0x4000], dtype=np.uint16), size=(K, N // 32))
    B = datagen.assemble_q8(d_bits, q)
    x = g.integers(-4, 5, size=(M, K)).astype(np.float32)
    y, bnd = oracle.q8_0_matmul(x, B, N, K)
    d = d_bits.view(np.float16).astype(np.float64)
    W = (q.astype(np.float64) * d[..., None]).reshape(K, N)   # dequantized by numpy
    assert (y == (x.astype(np.float64) @ W).astype(np.float32)).all()
    assert (bnd == np.abs(x.astype(np.float64)) @ np.abs(W)).all()
    # one-hot rows select dequantized rows; doubling every scale doubles y
    B = datagen.q8_0_random(82, K, N)
    oh = np.zeros((2, K), dtype=np.float32)
    oh[0, 5] = oh[1, K - 1] = 1.0
    y, _ = oracle.q8_0_matmul(oh, B, N, K)
    dq = np.stack([oracle.q8_0_dequant_block(B[k, j]) for k in (5, K - 1) for j in range(N // 32)])
    assert (y == dq.reshape(2, N).astype(np.float32)).all()
    x = datagen.activations(83, 2, K)
    y, _ = oracle.q8_0_matmul(x, B, N, K)
    B2 = B.copy()
    B2[..., 0:2] = (B[..., 0:2].copy().view(np.uint16) + 0x0400).view(np.uint8)
    assert (oracle.q8_0_matmul(x, B2, N, K)[0] == 2 * y).all()
    Bz = B.copy()
    Bz[..., 0:2] = 0
    assert not oracle.q8_0_matmul(x, Bz, N, K)[0].any()
