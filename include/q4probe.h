/*
 * q4probe — attainable-roof probes for MI355X (gfx950), measured beside the
 * Q4_0 kernels so their rates can be read against what the GPU delivers in
 * practice, not only against the nominal peaks. The pages set the frame: the
 * decode path is bound by memory bandwidth ("2000-line C++ DeepSeek inference
 * engine" article, §2.1 and §6.2: find the bottleneck before optimising), the
 * prefill path by the matrix units (KTransformers tutorial, "Optimization 2").
 *
 * Plain C ABI, same conventions as q4moe.h: device pointers owned by the
 * caller, work enqueued on `stream` (a hipStream_t passed as void*), 0 on
 * success, a negative q4_status on a bad argument (nothing enqueued) or a
 * launch error. The library allocates nothing.
 */
#ifndef Q4PROBE_H
#define Q4PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read-only stream: every 16-byte chunk of [src, src + bytes) is loaded once
 * with an aligned buffer_load_dwordx4 (consecutive lanes, consecutive
 * chunks; 8 loads in flight per lane; grid workgroups of 256 lanes striding
 * over the buffer). Nothing is stored except, per workgroup, one word into
 * sink[blockIdx] when the data's xor happens to equal a fixed constant (so the
 * loads are not optimised away); sink must hold `grid` words.
 *   src 16-byte aligned; bytes a multiple of 16, 16 <= bytes < 2^32;
 *   1 <= grid <= 65536.
 * Errors: Q4_EINVAL (null pointer, bytes or grid out of range), Q4_EALIGN. */
int q4_probe_stream(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream);

/* Read-only pass over a K x pitch-byte matrix in split-K tiles, the access
 * pattern of the decode GEMV: tile (c, s) covers bytes [c*seg, c*seg + seg)
 * of rows [s*kt, s*kt + kt) (the last column tile may be narrower), one
 * workgroup of 256 lanes per tile, ceil(pitch/seg) * ceil(K/kt) workgroups.
 * Lanes read the tile's 16-byte chunks in row-major order, 8 in flight per
 * lane. sink as for q4_probe_stream (one word per workgroup).
 *   src 16-byte aligned; pitch and seg multiples of 16; K * pitch < 2^31;
 *   at most 65536 workgroups.
 * Errors: Q4_EINVAL, Q4_ETOOBIG (matrix of 2 GiB or more), Q4_EALIGN. */
int q4_probe_tile(const void* src, int K, int pitch, int seg, int kt, uint32_t* sink,
                  void* stream);

/* One workgroup of 64 lanes that does nothing: the fixed cost of a kernel
 * boundary (for example between a GEMV and its split-K sum in a graph).
 * Errors: Q4_EINVAL (null sink; nothing is written to it). */
int q4_probe_empty(uint32_t* sink, void* stream);

/* Matrix-unit loops: each of grid workgroups of 256 lanes (4 waves) issues
 * `iters` rounds of 8 independent MFMAs per wave, then writes one value per
 * lane to sink (sink must hold grid * 256 floats).
 *   q4_probe_mfma_f16: v_mfma_f32_16x16x32_f16 (8192 multiply-adds each);
 *   q4_probe_mfma_f32: v_mfma_f32_4x4x1_16b_f32 (256 multiply-adds each).
 * Multiply-adds per call: grid * 4 * iters * 8 * (8192 or 256).
 * Errors: Q4_EINVAL (null sink, iters or grid out of range: 1 <= iters <=
 * 1 << 20, 1 <= grid <= 65536). */
int q4_probe_mfma_f16(int iters, int grid, float* sink, void* stream);
int q4_probe_mfma_f32(int iters, int grid, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4PROBE_H */
