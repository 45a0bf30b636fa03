/*
 * q4moe — Q4_0 fused-dequantization matmul and routed-expert MoE decode for
 * AMD Instinct MI355X (gfx950). Plain C ABI: device pointers, sizes, and a
 * HIP stream handle passed as void*. No C++ or framework types.
 *
 * Q4_0 (the "2000-line C++ DeepSeek inference engine" article, §2.2 block_q4_0
 * and dequantize; §2.3 layout; §7.1 byte order): a block is 18 little-endian
 * bytes holding 32 weights, a binary16 scale d followed by 16 bytes qs. Weight
 * 2i is the low nibble of qs[i] and weight 2i+1 the high nibble; its value is
 * (nibble - 8) * d.
 *
 * Matrix layout (same article, §3.4 matmul_q4_0): a K x N weight matrix B is
 * stored row-major as K rows of N/32 consecutive blocks; block (k, j) covers
 * columns 32j..32j+31 of row k. N must be a multiple of 32 (the article pads
 * columns to a multiple of 32 at load time). Activations and outputs are
 * row-major; y[m][n] = sum_k x[m][k] * w[k][n]. Outputs are overwritten.
 *
 * Common rules for every entry point:
 *  - Ownership: every pointer argument is device memory owned by the caller.
 *    The library keeps no pointer after the call returns and allocates nothing.
 *  - Asynchrony: arguments are checked on the host, the work is enqueued on
 *    `stream` (a hipStream_t; NULL is the default stream) and the call returns
 *    without synchronizing. Results are visible after the stream is synchronized.
 *  - Errors: 0 (Q4_OK) on success, a negative q4_status otherwise. On a host-side
 *    argument error nothing is enqueued and the outputs are untouched. Q4_EHIP
 *    reports a launch failure returned by the HIP runtime.
 *  - Workspace: entry points that take `ws` need at least the number of bytes
 *    the matching *_workspace_bytes() returns, 256-byte aligned device memory.
 *    A *_workspace_bytes() function returns 0 for every shape its entry point
 *    refuses (and for shapes that need no workspace); it never fails otherwise.
 *    Its contents are scratch (no initialisation needed). One workspace serves
 *    one call at a time: calls that overlap in time (for example on two
 *    streams) need separate workspaces.
 *  - Determinism: for the same arguments a call produces bitwise identical
 *    results (fixed reduction order, no floating-point atomics).
 */
#ifndef Q4MOE_H
#define Q4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One Q4_0 block: 18 bytes, 2-byte aligned, little-endian. */
typedef struct __attribute__((packed, aligned(2))) q4_0_block {
  uint16_t d;      /* binary16 scale bit pattern */
  uint8_t qs[16];  /* 32 packed nibbles, even weight in the low nibble */
} q4_0_block;

#ifdef __cplusplus
static_assert(sizeof(q4_0_block) == 18, "q4_0_block must be 18 bytes");
#else
_Static_assert(sizeof(q4_0_block) == 18, "q4_0_block must be 18 bytes");
#endif

/* One Q8_0 block: 34 bytes, 2-byte aligned, little-endian. The article's
 * §2.2 compares Q8_0 with Q4_0 (twice the memory) without defining it; read
 * as 32 weights q[l] * d with a binary16 scale d and signed 8-bit q. */
typedef struct __attribute__((packed, aligned(2))) q8_0_block {
  uint16_t d;     /* binary16 scale bit pattern */
  int8_t qs[32];  /* weights in two's complement */
} q8_0_block;

#ifdef __cplusplus
static_assert(sizeof(q8_0_block) == 34, "q8_0_block must be 34 bytes");
#else
_Static_assert(sizeof(q8_0_block) == 34, "q8_0_block must be 34 bytes");
#endif

typedef enum q4_status {
  Q4_OK = 0,
  Q4_EINVAL = -1,      /* null pointer or non-positive dimension */
  Q4_ESHAPE = -2,      /* N/H/I not a multiple of 32, or M/T/topk/E out of range */
  Q4_EALIGN = -3,      /* pointer misaligned (blocks 2 B, fp32/fp16 arrays 4 B, router x and
                          Wr 16 B, ws 256 B) */
  Q4_EWORKSPACE = -4,  /* workspace missing or smaller than required */
  Q4_EHIP = -5,        /* the HIP runtime reported an error at launch */
  Q4_ETOOBIG = -6      /* a size exceeds the limits of the implementation */
} q4_status;

/* Limits of the decode paths. */
#define Q4_GEMV_MAX_M 8    /* rows of x in one q4_0_gemv call */
#define Q4_MOE_MAX_T 64    /* tokens in one moe_q4_0_decode call */
#define Q4_MOE_MAX_TOPK 8  /* routed experts per token */
#define Q4_MOE_MAX_E 1024  /* experts per layer */
#define Q4_MOE_PREFILL_MAX_T 65536  /* tokens in one moe_q4_0_prefill call */

/* Static description of a status code (never NULL). */
const char* q4_strerror(int status);

/* ---------------------------------------------------------------------------
 * Decode GEMV (batch 1..8): y[M x N] = x[M x K] . deq(B[K x N]).
 * The article's fused matmul_q4_0(A, B, C, M, N, K) (§3.4), for decode batches.
 *   x   fp32 [M][K], 4-byte aligned      B  Q4_0 [K][N/32] blocks, 2-byte aligned
 *   y   fp32 [M][N], 4-byte aligned, overwritten
 *   1 <= M <= Q4_GEMV_MAX_M, K >= 1, N >= 32, N % 32 == 0; B, x and y each
 *   smaller than 2 GiB.
 *   ws/ws_bytes: workspace of q4_0_gemv_workspace_bytes(M, N, K) bytes (K-split
 *   partial sums; may be 0, then ws may be NULL).
 * Accumulation is fp32; each product x * (q - 8) * d is formed in fp32.
 * ------------------------------------------------------------------------- */
size_t q4_0_gemv_workspace_bytes(int M, int N, int K);
int q4_0_gemv(const float* x, const q4_0_block* B, float* y, int M, int N, int K, void* ws,
              size_t ws_bytes, void* stream);

/* Allocation-free q4_0_gemv, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results as q4_0_gemv, without ws:
 * the K-split partial sums go to a static device array of
 * Q4_GEMV_NOALLOC_MAX_WS bytes that the library holds on each GPU it runs on
 * until the process ends. Nothing in it needs to start at zero (every partial
 * is written before it is read). All calls on one GPU share that array, so
 * calls that overlap on one GPU (concurrent streams, or threads) race; calls
 * in one stream do not.
 * Errors: those of q4_0_gemv, and Q4_ETOOBIG when
 * q4_0_gemv_workspace_bytes(M, N, K) exceeds Q4_GEMV_NOALLOC_MAX_WS (nothing
 * enqueued). Calls no allocating routine. */
#define Q4_GEMV_NOALLOC_MAX_WS (16u << 20)
int q4_0_gemv_noalloc(const float* x, const q4_0_block* B, float* y, int M, int N, int K,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Decode GEMV over Q8_0 weights (batch 1..8): y[M x N] = x[M x K] . deq(B[K x N]),
 * the Q8_0 counterpart of q4_0_gemv for the article's Q8_0-versus-Q4_0
 * comparison (§2.2). Same layout rules (blocks along N), arguments, limits
 * and errors as q4_0_gemv, with B of q8_0_block (2-byte aligned, < 2 GiB).
 *   ws/ws_bytes: workspace of q8_0_gemv_workspace_bytes(M, N, K) bytes.
 * Accumulation is fp32; each product x * q * d is formed as (x * d) * q.
 * ------------------------------------------------------------------------- */
size_t q8_0_gemv_workspace_bytes(int M, int N, int K);
int q8_0_gemv(const float* x, const q8_0_block* B, float* y, int M, int N, int K, void* ws,
              size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill GEMM: Y[M x N] = X[M x K] . deq(B[K x N]) on the fp16 matrix cores.
 * The batched-prompt matmul of the same article (§5.2) and the quantized
 * tensor-core GEMM that the KTransformers tutorial uses for prefill ("Optimization
 * 2", Marlin), as one fused kernel: B tiles are dequantized to fp16 in LDS and
 * contracted with fp32 accumulation.
 *   X   fp16 [M][K] (the caller rounds its activations to fp16), 4-byte aligned
 *   B   Q4_0 [K][N/32] blocks, 2-byte aligned      Y fp32 [M][N], overwritten
 *   M >= 1, K >= 1, N >= 32, N % 32 == 0.
 * Each dequantized weight (q - 8) * d is rounded to fp16 before the product.
 * ------------------------------------------------------------------------- */
int q4_0_gemm(const uint16_t* X, const q4_0_block* B, float* Y, int M, int N, int K,
              void* stream);

/* ---------------------------------------------------------------------------
 * Routed-expert MoE decode (DeepSeek-V2 shape: KTransformers tutorial,
 * "Optimization 3": top-6 of 160 routed experts evaluated as batched GEMVs;
 * the MoE module's gate hands top-k ids and weights to the experts):
 *   out[t] = sum_{s < topk} topk_w[t][s] * Wd_e ( SiLU(x_t . Wg_e) * (x_t . Wu_e) ),
 *   e = topk_ids[t][s], SiLU(z) = z / (1 + exp(-z)).
 *   x        fp32 [T][H]                     out  fp32 [T][H], overwritten
 *   Wg, Wu   Q4_0, E consecutive H x I matrices (blocks along I)
 *   Wd       Q4_0, E consecutive I x H matrices (blocks along H)
 *   topk_ids int32 [T][topk]                 topk_w fp32 [T][topk]
 *   1 <= T <= Q4_MOE_MAX_T, 1 <= topk <= Q4_MOE_MAX_TOPK, 1 <= E <= Q4_MOE_MAX_E,
 *   H % 32 == 0, I % 32 == 0.
 * Work is grouped by expert from the routing table on the device: each routed
 * expert's weights are streamed once per call for all tokens that chose it
 * (in chunks of at most 8 tokens).
 * Data-dependent rules (not checked on the host): an id outside [0, E)
 * contributes zero; an expert repeated within a token contributes once per slot.
 * The slot contributions of a token are summed in slot order 0..topk-1.
 *   ws/ws_bytes: workspace of moe_q4_0_workspace_bytes(T, H, I, E, topk) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_q4_0_workspace_bytes(int T, int H, int I, int E, int topk);
int moe_q4_0_decode(const float* x, const q4_0_block* Wg, const q4_0_block* Wu,
                    const q4_0_block* Wd, const int32_t* topk_ids, const float* topk_w,
                    float* out, int T, int H, int I, int E, int topk, void* ws,
                    size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Inspection of the routing table that moe_q4_0_decode builds in its
 * workspace: the grouping of (token, slot) pairs by expert that lets each
 * routed expert's weights be streamed once for all the tokens that chose it
 * (the MoE module's gate hands the experts top-k ids; "Optimization 3" runs
 * the routed experts as batched GEMVs). Meant for tests and debugging: after
 * a call with T >= 2 on the same (T, H, I, E, topk), the workspace holds
 *   counts      int32[2] at *counts_off: the number of vector items and of
 *               matrix-core items;
 *   vector items q4_moe_item[counts[0]] at *items_off: one item per expert
 *               chosen by 1 or 2 pairs, in increasing expert order;
 *   matrix items q4_moe_item[counts[1]] at *mitems_off: an expert chosen by
 *               n >= 3 pairs gives c = ceil(n / 8) items holding consecutive
 *               runs of its pairs, the first n mod c of size n / c + 1 and the
 *               others n / c, in increasing expert order.
 * A pair is p = t * topk + slot; within an expert the pairs appear in
 * increasing p; an id outside [0, E) appears nowhere; pairs[] entries past
 * count are 0. A single token (T == 1) skips this pass and leaves no table.
 * The offsets are byte offsets into the workspace (ws); the table lives
 * there until the next call that uses the workspace. Returns Q4_OK, or the
 * status moe_q4_0_decode would return for the shape; outputs untouched on error.
 * ------------------------------------------------------------------------- */
typedef struct q4_moe_item {
  int32_t expert;        /* expert id */
  int32_t count;         /* pairs in this item (1 .. 8) */
  int32_t reserved[2];
  int32_t pairs[8];      /* pair indices t * topk + slot */
} q4_moe_item;

int moe_q4_0_route_layout(int T, int H, int I, int E, int topk, size_t* items_off,
                          size_t* counts_off, size_t* mitems_off);

/* ---------------------------------------------------------------------------
 * Routed-expert MoE at prefill (many tokens per expert): the same layer as
 * moe_q4_0_decode, with every expert's gate, up and down products run as
 * GEMMs on the fp16 matrix cores. The KTransformers tutorial gives the
 * experts separate prefill and generate operators and runs prefill on the
 * GPU ("KExpertsTorch"); the dense prefill GEMMs run on tensor cores
 * ("Optimization 2").
 *   out[t] = sum_{s < topk} topk_w[t][s] * Wd_e ( SiLU(x_t . Wg_e) * (x_t . Wu_e) )
 *   x16      fp16 [T][H] (the caller rounds its activations), 16-byte aligned
 *   Wg, Wu, Wd, topk_ids, topk_w, out   as in moe_q4_0_decode; weights 4-byte
 *            aligned, out 16-byte aligned
 *   1 <= T <= Q4_MOE_PREFILL_MAX_T, 1 <= topk <= Q4_MOE_MAX_TOPK,
 *   1 <= E <= Q4_MOE_MAX_E, H % 128 == 0, I % 128 == 0.
 * Pairs are sorted by expert on the device (stable); each expert's rows go
 * through Q4_MOE_PREFILL_TILE_ROWS-row tiles. Each dequantized weight and h = SiLU(g) * u are
 * rounded to fp16 before their products; sums are fp32. Ids outside [0, E)
 * contribute zero; slots are summed in order 0..topk-1.
 *   ws/ws_bytes: workspace of moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk)
 *   bytes (the per-pair h and down rows: about T * topk * (2 * I + 4 * H) bytes).
 * ------------------------------------------------------------------------- */
size_t moe_q4_0_prefill_workspace_bytes(int T, int H, int I, int E, int topk);
int moe_q4_0_prefill(const uint16_t* x16, const q4_0_block* Wg, const q4_0_block* Wu,
                     const q4_0_block* Wd, const int32_t* topk_ids, const float* topk_w,
                     float* out, int T, int H, int I, int E, int topk, void* ws,
                     size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Where moe_q4_0_prefill leaves its routing, a stable sort of the (token,
 * slot) pairs by expert, in its workspace (the expert grouping that the
 * KTransformers tutorial's "Optimization 3" schedules by; here it orders the
 * GEMM rows). Meant for tests and debugging: after a call on the same
 * (T, H, I, E, topk), the workspace holds
 *   counts  int32[2] at *counts_off: the number of m-tiles and of valid pairs
 *           (sorted rows);
 *   src     int32[counts[1]] at *src_off: the token t of sorted row q;
 *   pos     int32[T * topk] at *pos_off: the sorted row of pair
 *           p = t * topk + slot, -1 for an id outside [0, E);
 *   tiles   int32[counts[0]][4] at *tiles_off: (expert, first sorted row,
 *           rows, 0); each expert's rows cut into Q4_MOE_PREFILL_TILE_ROWS-row
 *           tiles (the last one shorter), in increasing expert order.
 * Sorted rows run over the experts in increasing id and, within an expert,
 * over its pairs in increasing p. The offsets are byte offsets into ws; the
 * data lives there until the next call that uses the workspace. Returns Q4_OK,
 * or the status moe_q4_0_prefill would return for the shape; outputs untouched
 * on error.
 * ------------------------------------------------------------------------- */
#define Q4_MOE_PREFILL_TILE_ROWS 96   /* rows of one expert m-tile */

int moe_q4_0_prefill_route_layout(int T, int H, int I, int E, int topk, size_t* src_off,
                                  size_t* pos_off, size_t* tiles_off, size_t* counts_off);

/* ---------------------------------------------------------------------------
 * MoE router: the gate in front of moe_q4_0_decode, on the device. The
 * KTransformers tutorial's YAML-injection section has the KDeepseekV2MoE
 * forward run the gate first for each token's top-k ids and weights;
 * "Optimization 3" keeps the shared experts, which every token uses, on the GPU.
 *   logits[t][e] = sum_h x[t][h] * Wr[e][h]   (fp32 products and sums)
 *   topk_ids[t][j], j < topk: the topk largest logits, largest first; equal
 *     logits go to the lower expert index; a NaN logit is never chosen, and a
 *     slot that finds no candidate gets id -1 (moe_q4_0_decode adds nothing
 *     for it) and weight 0;
 *   topk_w[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the chosen
 *     logits l_0 >= l_1 >= ... (softmax over the chosen ones only);
 *   slots topk .. topk + n_shared - 1: id E + s and weight 1, the shared
 *     experts, stored after the E routed experts in the decode's weights.
 *   x        fp32 [T][H], 16-byte aligned    Wr  fp32 [E][H] (one row per
 *            routed expert), 16-byte aligned
 *   logits   fp32 [T][E], overwritten        topk_ids int32, topk_w fp32
 *            [T][topk + n_shared], overwritten; all 4-byte aligned
 *   1 <= T <= Q4_MOE_MAX_T, 1 <= E <= Q4_MOE_MAX_E, 1 <= topk <= E,
 *   0 <= n_shared, topk + n_shared <= Q4_MOE_MAX_TOPK, H >= 4, H % 4 == 0.
 *   ws/ws_bytes: workspace of moe_router_workspace_bytes(T, H, E) bytes
 *   (K-split partial logits).
 * The outputs feed moe_q4_0_decode(..., E + n_shared experts, topk + n_shared
 * slots) on the same stream with no host round trip.
 * ------------------------------------------------------------------------- */
size_t moe_router_workspace_bytes(int T, int H, int E);
int moe_router_topk(const float* x, const float* Wr, float* logits, int32_t* topk_ids,
                    float* topk_w, int T, int H, int E, int topk, int n_shared, void* ws,
                    size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Whole MoE layer at decode: moe_router_topk, then moe_q4_0_decode over the
 * routed and shared experts, on one stream:
 *   out[t] = sum_{j < topk} w_j * FFN_{e_j}(x_t) + sum_{s < n_shared} FFN_{E+s}(x_t),
 *   FFN_e(x) = Wd_e ( SiLU(x . Wg_e) * (x . Wu_e) ).
 *   Wg, Wu, Wd  Q4_0 as in moe_q4_0_decode, E + n_shared consecutive matrices
 *               (the E routed experts, then the shared ones)
 *   Other arguments and limits as in moe_router_topk and moe_q4_0_decode
 *   (H % 32 == 0, I % 32 == 0); E + n_shared <= Q4_MOE_MAX_E.
 *   ws/ws_bytes: workspace of moe_q4_0_layer_workspace_bytes(...) bytes; the
 *   router's logits, ids and weights are kept there.
 * ------------------------------------------------------------------------- */
size_t moe_q4_0_layer_workspace_bytes(int T, int H, int I, int E, int topk, int n_shared);
int moe_q4_0_layer(const float* x, const float* Wr, const q4_0_block* Wg, const q4_0_block* Wu,
                   const q4_0_block* Wd, float* out, int T, int H, int I, int E, int topk,
                   int n_shared, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4MOE_H */
