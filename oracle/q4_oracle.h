/*
 * CPU oracle for Q4_0 fused-dequantization matmul and routed-expert MoE decode.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and
 * its Python binding) includes, links or calls this code. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * It is plain, single-threaded C++ that writes out the definitions on the
 * pages: dequantize a weight, then multiply in double precision. It shares no
 * code, header or table with the GPU library.
 *
 * Sources (pages, by title and section):
 *  - "2000-line C++ DeepSeek inference engine" article (news.rkmt.cn/news/19011)
 *    §2.2: the block_q4_0 record (fp16 scale d, 16 bytes of packed nibbles for
 *    32 weights) and dequantize(): byte index/2, low nibble for even index,
 *    high nibble for odd, value (q - 8) * fp16_to_fp32(d).
 *    §2.3: row-major layout, one row's blocks stored contiguously, columns
 *    padded to a multiple of 32.
 *    §3.2: the (i, k, j) loop order with C cleared first.
 *    §3.4: the fused matmul_q4_0(A, B, C, M, N, K): block (k, j) is
 *    B[k*(N/32) + j/32] and covers columns j..j+31 of row k.
 *    §7.1: weight files are little-endian.
 *  - "KTransformers DeepSeek-V2 heterogeneous MoE inference" tutorial
 *    (www.mhpn.cn/news/2178346), section "Optimization 3" (arithmetic-intensity
 *    offload): routed experts of DeepSeek-V2, top-6 of 160, run as a set of
 *    batched GEMVs; the MoE module's gate yields top-k ids and weights that the
 *    experts consume; the shared experts are used by every token (kept in GPU
 *    memory for that reason). Its YAML-injection section: the KDeepseekV2MoE
 *    forward first runs the gate for each token's top-k ids and weights.
 *
 * Parity pins: every function here is pinned by tests that do not reuse its
 * code (hand-worked blocks, IEEE bit patterns checked against numpy's float16,
 * integer-exact special cases checked against numpy matmul, invariants). No
 * function is "parity unpinned".
 *
 * Conventions: B is K rows x N columns, row-major, blocks of 32 along N; each
 * block is 18 little-endian bytes [d (binary16) | qs[16]]. N % 32 == 0.
 * Return value of the int functions: 0 on success, -1 on invalid arguments.
 */
#ifndef Q4_ORACLE_H
#define Q4_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE-754 binary16 -> double, exact (every binary16 value is a double). */
double oracle_fp16_to_double(uint16_t bits);

/* Dequantize one 18-byte block into 32 doubles (all exact). */
void oracle_dequant_block(const uint8_t* block18, double* out32);

/* Dequantize rows [k0, k1) of a K x N matrix into out[(k1-k0) * N] (float;
 * every dequantized weight is exactly representable in binary32). */
int oracle_dequant_rows(const uint8_t* B, int N, int k0, int k1, float* out);

/* y[M x N] = x[M x K] . deq(B[K x N]), accumulated in double in (i, k, j)
 * order, rounded once to float. If bound != NULL it receives
 * sum_k |x[m][k] * w[k][n]| in double (the per-output error scale). */
int oracle_q4_0_matmul(const float* x, const uint8_t* B, int M, int N, int K,
                       float* y, double* bound);

/* Same, with the activations given as binary16 bit patterns (prefill). */
int oracle_q4_0_matmul_f16(const uint16_t* x16, const uint8_t* B, int M, int N,
                           int K, float* y, double* bound);

/* Routed-expert MoE decode:
 *   out[t] = sum_{j < topk, 0 <= ids[t][j] < E} w[t][j] * down_e(SiLU(x_t . Wg_e) * (x_t . Wu_e))
 * with e = ids[t][j]. Wg and Wu are E consecutive H x I Q4_0 matrices (blocks
 * along I); Wd is E consecutive I x H matrices (blocks along H). The gate and
 * up products, SiLU and the down product are all kept in double; out is rounded
 * once to float. bound[t][n] (optional) = sum_j |w| * sum_k |h_k * Wd[k][n]|.
 * h_out (optional, [T*topk][I] doubles) receives each slot's h (zeros for an
 * out-of-range id). */
int oracle_moe_decode(const float* x, const uint8_t* Wg, const uint8_t* Wu,
                      const uint8_t* Wd, const int32_t* ids, const float* w,
                      int T, int H, int I, int E, int topk, float* out,
                      double* bound, double* h_out);

/* Q8_0 weights. The article's §2.2 compares Q8_0 with Q4_0 (twice the memory,
 * about 60 % of Q4_0's token rate on the author's CPU) but does not define
 * it; the plainest reading, used here: a block of 32 weights is 34
 * little-endian bytes, a binary16 scale d then 32 signed (two's complement)
 * bytes q, weight l = q[l] * d (exact in double and in float). Blocks run
 * along N as for Q4_0. */
void oracle_q8_0_dequant_block(const uint8_t* block34, double* out32);

/* y[M x N] = x[M x K] . deq(B[K x N]) for Q8_0 B, as oracle_q4_0_matmul. */
int oracle_q8_0_matmul(const float* x, const uint8_t* B, int M, int N, int K, float* y,
                       double* bound);

/* MoE router (the gate in front of the routed experts):
 *   logits[t][e] = sum_h x[t][h] * Wr[e][h]
 * accumulated in double in h order and rounded once to float. Wr holds one row
 * of H floats per routed expert (E rows). bound[t][e] (optional) receives
 * sum_h |x[t][h] * Wr[e][h]| in double. */
int oracle_router_logits(const float* x, const float* Wr, int T, int H, int E,
                         float* logits, double* bound);

/* Top-k routing of float logits [T][E]. Per token: the topk largest logits,
 * largest first; equal logits go to the lower expert index; a NaN logit is
 * never chosen, and a slot that finds no candidate gets id -1 and weight 0.
 * The weights are the softmax over the chosen logits, computed in double with
 * their maximum subtracted and rounded to float. n_shared shared experts
 * follow the routed slots: slot topk + s holds id E + s with weight 1.
 * ids and w are [T][topk + n_shared]. */
int oracle_router_topk(const float* logits, int T, int E, int topk, int n_shared,
                       int32_t* ids, float* w);

#ifdef __cplusplus
}
#endif

#endif /* Q4_ORACLE_H */
