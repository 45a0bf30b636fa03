"""Seeded synthetic inputs, shared by the GPU path's tests/benchmark and the oracle.

This module holds no arithmetic of the method itself: it draws random numbers,
packs them into the Q4_0 byte layout and prepares the routing table that the
MoE decode consumes as input. Everything is reproducible from a seed with
numpy's ``Generator(PCG64(seed))``.

Layout produced (the pages' Q4_0 record, "2000-line C++ DeepSeek inference
engine" article §2.2/§2.3/§7.1): a K x N weight matrix is K rows of N/32
blocks; each block is 18 little-endian bytes, the binary16 scale ``d`` in
bytes 0..1 followed by 16 bytes ``qs`` where weight 2i is the low nibble and
weight 2i+1 the high nibble of ``qs[i]``.

Workload recipe (mirrors the MoE decode and dense decode shapes of the pages:
7B-class 4096/11008 linears, DeepSeek-V2 experts 5120/1536/160, top-6):
  * activations ~ N(0, 1) in float32;
  * nibbles i.i.d. uniform on 0..15 (qs bytes uniform on 0..255);
  * scales uniform on [0.001, 0.02], rounded to binary16 (round to nearest
    even, numpy ``astype``);
  * router logits ~ N(0, 1) over E experts, optionally +bias on experts
    0..n_hot-1 (skewed routing); top-k by logit (ties to the lower index),
    softmax over the k selected logits in float64 after subtracting their max,
    cast to float32 (the decode-only configurations take this table as input);
  * for the whole layer, router weights fp32 [E, H] ~ N(0, 1/H), so that the
    router's logits of N(0, 1) activations are ~ N(0, 1) as above, and two
    shared experts drawn like the routed ones.
"""
from __future__ import annotations

import numpy as np

BLOCK_BYTES = 18
BLOCK_WEIGHTS = 32

#: numpy view of one block (itemsize 18, no padding)
BLOCK_DTYPE = np.dtype([("d", "<u2"), ("qs", "u1", (16,))])
assert BLOCK_DTYPE.itemsize == BLOCK_BYTES


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def activations(seed: int, M: int, K: int) -> np.ndarray:
    """float32 [M, K] ~ N(0, 1)."""
    return rng(seed).standard_normal((M, K), dtype=np.float32)


def q4_0_random(seed: int, K: int, N: int, d_lo: float = 0.001, d_hi: float = 0.02) -> np.ndarray:
    """Random Q4_0 matrix (K rows, N columns, blocks along N) as uint8 [K, N/32, 18]."""
    if N % BLOCK_WEIGHTS:
        raise ValueError("N must be a multiple of 32")
    nb = N // BLOCK_WEIGHTS
    g = rng(seed)
    qs = g.integers(0, 256, size=(K, nb, 16), dtype=np.uint8)
    d = g.uniform(d_lo, d_hi, size=(K, nb)).astype(np.float16)
    return assemble(d.view(np.uint16), qs)


Q8_BLOCK_BYTES = 34


def q8_0_random(seed: int, K: int, N: int, d_lo: float = 0.001, d_hi: float = 0.02) -> np.ndarray:
    """Q8_0 matrix [K, N/32, 34] (uint8 bytes): binary16 scale then 32 signed
    bytes per block; the signed bytes uniform on -128..127, scales as for Q4_0."""
    assert N % BLOCK_WEIGHTS == 0
    g = rng(seed)
    q = g.integers(0, 256, size=(K, N // BLOCK_WEIGHTS, BLOCK_WEIGHTS), dtype=np.uint8)
    d = g.uniform(d_lo, d_hi, size=(K, N // BLOCK_WEIGHTS)).astype(np.float16).view(np.uint16)
    return assemble_q8(d, q)


def assemble_q8(d_bits: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack scale bits [..] and signed-byte weights [.., 32] (any 8-bit dtype)
    into Q8_0 blocks [.., 34]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    out = np.empty(d_bits.shape + (Q8_BLOCK_BYTES,), dtype=np.uint8)
    out[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (d_bits >> 8).astype(np.uint8)
    out[..., 2:] = np.asarray(q).view(np.uint8)
    return out


def assemble(d_bits: np.ndarray, qs: np.ndarray) -> np.ndarray:
    """Pack scale bit patterns [..., nb] and qs bytes [..., nb, 16] into [..., nb, 18]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    qs = np.asarray(qs, dtype=np.uint8)
    out = np.empty(qs.shape[:-1] + (BLOCK_BYTES,), dtype=np.uint8)
    out[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (d_bits >> 8).astype(np.uint8)
    out[..., 2:] = qs
    return out


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Nibble values q[..., N] (0..15) -> qs bytes [..., N/32, 16] (even index in the low nibble)."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape[-1] % BLOCK_WEIGHTS:
        raise ValueError("last dimension must be a multiple of 32")
    if (q > 15).any():
        raise ValueError("nibble values must lie in 0..15")
    pairs = q.reshape(q.shape[:-1] + (q.shape[-1] // 2, 2))
    qs = (pairs[..., 0] | (pairs[..., 1] << 4)).astype(np.uint8)
    return qs.reshape(q.shape[:-1] + (q.shape[-1] // BLOCK_WEIGHTS, 16))


def routing(seed: int, T: int, E: int, topk: int, hot_bias: float = 0.0, n_hot: int = 8):
    """Router table for T tokens: (ids int32 [T, topk], weights float32 [T, topk], logits)."""
    logits = rng(seed).standard_normal((T, E), dtype=np.float32)
    if hot_bias:
        logits[:, :n_hot] += np.float32(hot_bias)
    return topk_softmax(logits, topk) + (logits,)


def topk_softmax(logits: np.ndarray, topk: int):
    """Top-k experts per row (largest first, ties to the lower index) and the
    softmax over the k selected logits (float64, max subtracted), as float32."""
    logits = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    sel = sel - sel.max(axis=1, keepdims=True)
    ex = np.exp(sel)
    w = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), w


def to_f16(x: np.ndarray) -> np.ndarray:
    """Round float32 activations to binary16 (round to nearest even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------
# Workload definitions (shapes, seeds). Names describe the workload.
# --------------------------------------------------------------------------

#: single GEMV, 4096 x 4096, batch 1
GEMV_4096 = dict(M=1, K=4096, N=4096, x_seed=1101, b_seed=1201)

#: dense 7B-shaped decode linears (K rows x N cols), one seed per matrix
DENSE_7B_SHAPES = [
    ("attn_proj", 4096, 4096, 2201),
    ("ffn_gate", 4096, 11008, 2202),
    ("ffn_up", 4096, 11008, 2203),
    ("ffn_down", 11008, 4096, 2204),
]
DENSE_7B_BATCHES = (1, 4, 8)


def dense_x_seed(M: int) -> int:
    return 2100 + M


#: DeepSeek-V2-shaped routed experts
MOE_DSV2 = dict(H=5120, I=1536, E=160, topk=6)
MOE_T1 = dict(T=1, x_seed=3101, logit_seed=3201)
MOE_T32 = dict(T=32, x_seed=4101, logit_seed=4201, hot_bias=2.0, n_hot=8)


#: whole layer: the same experts plus 2 shared experts of the routed experts'
#: shape (stored as experts E, E + 1, seeds by expert_seed), and an fp32 router
#: [E, H] ~ N(0, 1/H), so that the logits of x ~ N(0, 1) are ~ N(0, 1)
MOE_LAYER = dict(n_shared=2, router_seed=3901)


def router_weights(seed: int, E: int, H: int) -> np.ndarray:
    """Router (gate) weights fp32 [E, H], N(0, 1/H)."""
    return (rng(seed).standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)


def expert_seed(e: int, m: int) -> int:
    """Seed of expert e's matrix m (0 gate, 1 up, 2 down)."""
    return 3300 + 3 * e + m


def moe_experts(H: int, I: int, E: int, experts=None):
    """Stacked expert weights: Wg, Wu [E, H, I/32, 18] and Wd [E, I, H/32, 18].

    ``experts`` (optional iterable of ids) limits generation to those experts;
    the others are left zero (useful for oracle-only checks)."""
    Wg = np.zeros((E, H, I // 32, BLOCK_BYTES), dtype=np.uint8)
    Wu = np.zeros_like(Wg)
    Wd = np.zeros((E, I, H // 32, BLOCK_BYTES), dtype=np.uint8)
    for e in (range(E) if experts is None else experts):
        Wg[e] = q4_0_random(expert_seed(e, 0), H, I)
        Wu[e] = q4_0_random(expert_seed(e, 1), H, I)
        Wd[e] = q4_0_random(expert_seed(e, 2), I, H)
    return Wg, Wu, Wd


#: prefill GEMM: X [2048 x 4096] (float32 -> float16) times Q4_0 4096 x {4096, 11008}
PREFILL = dict(M=2048, K=4096, Ns=(4096, 11008), x_seed=5101, b_seeds=(5201, 5202))
