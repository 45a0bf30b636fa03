// Device-side building blocks shared by the Q4_0 decode kernels (gfx950).
//
// Q4_0 block ("2000-line C++ DeepSeek inference engine" article, §2.2): 18
// bytes, binary16 scale d then 16 bytes qs; weight 2i is the low nibble of
// qs[i], weight 2i+1 the high nibble; value (q - 8) * d.
//
// Arithmetic used on the GPU for one block and one activation value a:
//   s       = a * d                      (one fp32 multiply per block and row)
//   acc[2i]   += s * lo_i                (lo_i = q & 0x0F converted exactly)
//   acc[2i+1] += s * (16 * hi_i)         (the byte masked with 0xF0 converted
//                                         exactly; the factor 16 is removed at
//                                         the end, which is exact in binary32)
//   corr      += s
//   result    = acc - 8 * corr           (so each weight costs one convert and
//                                         one FMA per activation row)
// Scaling by 16 commutes with every rounding step (no overflow or underflow for
// finite inputs of the decode workloads), so the odd-column accumulators equal
// 16x the plain accumulation bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr int kBlockBytes = 18;
constexpr int kBlockWeights = 32;
constexpr int kWaveSize = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// Workgroups are dispatched round-robin over the XCDs (block b runs on XCD
// b % 8). Returns a logical tile index such that consecutive logical tiles
// run on the same XCD, so tiles that share cache lines share that XCD's L2.
__device__ __forceinline__ int xcd_logical_tile(int b, int total) {
  const int full = (total / kNumXcd) * kNumXcd;
  if (b >= full) return b;
  const int per = full / kNumXcd;
  return (b % kNumXcd) * per + b / kNumXcd;
}

// binary16 bits (low 16 bits of v) -> fp32, exact (v_cvt_f32_f16).
__device__ __forceinline__ float half_bits_to_float(uint32_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v)));
}

// Raw bytes of one lane's share of a block: LPB lanes split the 16 qs bytes.
template <int LPB>
struct BlockPart {
  static constexpr int kWords = 4 / LPB;  // dwords of qs held by one lane
  uint32_t d;                              // scale bits in the low half
  uint32_t q[kWords];
};

// Load part `part` (0..LPB-1) of the block at byte address p (2-byte aligned).
// The qs share is kWords dwords starting at byte 2 + 8 * part * (2 / LPB).
template <int LPB>
__device__ __forceinline__ void load_part(const uint8_t* __restrict__ p, int part,
                                          BlockPart<LPB>& out) {
  out.d = *reinterpret_cast<const uint16_t*>(p);
  const uint8_t* qp = p + 2 + part * (16 / LPB);
  __builtin_memcpy(out.q, qp, sizeof(out.q));  // unaligned dwordx{4,2} load
}

// Accumulate one block share for M activation rows.
//   xv[m] : activation of row m at this k (0 for rows past the end)
//   acc[m][c] : c indexes the lane's 32/LPB columns
template <int M, int LPB>
__device__ __forceinline__ void fma_part(const float (&xv)[M], const BlockPart<LPB>& b,
                                         float (&acc)[M][32 / LPB], float (&corr)[M]) {
  const float d = half_bits_to_float(b.d);
  float s[M];
  {
    // corr must sum exactly the rounded s that the FMAs below use, so that
    // acc - 8 * corr cancels exactly when every nibble is 8: no contraction
    // of s into the corr addition.
#pragma clang fp contract(off)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      s[m] = xv[m] * d;
      corr[m] += s[m];
    }
  }
#pragma unroll
  for (int w = 0; w < BlockPart<LPB>::kWords; ++w) {
    const uint32_t lo = b.q[w] & 0x0f0f0f0fu;
    const uint32_t hi = b.q[w] & 0xf0f0f0f0u;
#pragma unroll
    for (int by = 0; by < 4; ++by) {
      const float fl = static_cast<float>((lo >> (8 * by)) & 0xffu);  // v_cvt_f32_ubyteN
      const float fh = static_cast<float>((hi >> (8 * by)) & 0xffu);  // 16 * high nibble
      const int c = 2 * (4 * w + by);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        acc[m][c] = __builtin_fmaf(s[m], fl, acc[m][c]);
        acc[m][c + 1] = __builtin_fmaf(s[m], fh, acc[m][c + 1]);
      }
    }
  }
}

// Finish a lane's accumulators: even columns acc - 8*corr, odd columns
// acc/16 - 8*corr (both exact rescalings, one rounding in the subtraction).
template <int M, int LPB>
__device__ __forceinline__ void finish_part(float (&acc)[M][32 / LPB], const float (&corr)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float c8 = 8.0f * corr[m];
#pragma unroll
    for (int c = 0; c < 32 / LPB; c += 2) {
      acc[m][c] = acc[m][c] - c8;
      acc[m][c + 1] = acc[m][c + 1] * 0.0625f - c8;
    }
  }
}

// Split-K completion ticket. Every workgroup of a tile group calls this after
// storing its partial results; it returns true in exactly one workgroup (the
// last to arrive), which may then read all partials of the group. The counter
// is reset by that workgroup so the workspace is zero again after the kernel.
__device__ __forceinline__ bool arrive_last(unsigned* __restrict__ counter, unsigned expected,
                                            unsigned* lds_flag) {
  __threadfence();  // release this workgroup's partial stores (agent scope)
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(counter, 1u);
    const bool last = (prev == expected - 1u);
    if (last) *counter = 0u;
    *lds_flag = last ? 1u : 0u;
  }
  __syncthreads();
  const bool last = (*lds_flag != 0u);
  if (last) __threadfence();  // acquire the other workgroups' partials
  return last;
}

}  // namespace q4

namespace q4 {

constexpr int kThreads = 256;             // lanes per workgroup of the decode kernels
constexpr int kRedStride = kThreads + 1;  // LDS stride of the row-phase reduction

// LDS stride (floats per k) of staged activations for M rows.
template <int M>
constexpr int x_stride() {
  return M == 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8));
}

// Geometry of one decode tile: Jt block columns starting at j0, rows
// [k0, k0 + rows) of a matrix with NB blocks per row; P row phases of Lr lanes.
struct TileGeom {
  const uint8_t* B;  // matrix base
  int NB, j0, k0, rows, Lr, P;
};

// Accumulate this lane's share of a tile. Lane t is row phase r = t / Lr and
// block column jj = (t % Lr) / LPB, part (t % Lr) % LPB; it walks rows
// k0 + r, k0 + r + P, ... in increasing order. xs holds the staged activations
// (k-major, stride x_stride<M>()). Inactive lanes leave acc/corr at zero.
template <int M, int LPB, int U>
__device__ __forceinline__ void tile_accumulate(const TileGeom& g, const float* xs,
                                                float (&acc)[M][32 / LPB], float (&corr)[M]) {
  constexpr int XS = x_stride<M>();
  const int t = threadIdx.x;
  const int r = t / g.Lr;
  const int v = t - r * g.Lr;
  const int jj = v / LPB;
  const int part = v - jj * LPB;
  const int j = g.j0 + jj;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    corr[m] = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 32 / LPB; ++cc) acc[m][cc] = 0.0f;
  }
  if (r >= g.P || j >= g.NB || r >= g.rows) return;

  const size_t row_bytes = (size_t)g.NB * kBlockBytes;
  const uint8_t* __restrict__ base = g.B + (size_t)g.k0 * row_bytes + (size_t)j * kBlockBytes;
  const int step = g.P * U;
  const int rows = g.rows;
  const int P = g.P;
  BlockPart<LPB> b0[U], b1[U];

  auto load_batch = [&](BlockPart<LPB>(&b)[U], int kk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(kk + u * P, rows - 1);
      load_part<LPB>(base + (size_t)k * row_bytes, part, b[u]);
    }
  };
  auto compute_batch = [&](BlockPart<LPB>(&b)[U], int kk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kk + u * P;
      const bool ok = k < rows;
      float xv[M];
      const float* xr = xs + (ok ? k : 0) * XS;
#pragma unroll
      for (int m = 0; m < M; ++m) xv[m] = ok ? xr[m] : 0.0f;
      if (!ok) b[u].d = 0u;  // rows past the end contribute exactly zero
      fma_part<M, LPB>(xv, b[u], acc, corr);
    }
  };

  int kk = r;
  load_batch(b0, kk);
  while (true) {
    const bool more1 = kk + step < rows;
    if (more1) load_batch(b1, kk + step);
    compute_batch(b0, kk);
    if (!more1) break;
    kk += step;
    const bool more0 = kk + step < rows;
    if (more0) load_batch(b0, kk + step);
    compute_batch(b1, kk);
    if (!more0) break;
    kk += step;
  }
}

// Sum the P row phases of a tile through LDS in phase order 0..P-1, one
// activation row at a time, and hand each tile output (m, o) to store(m, o, v),
// o in [0, ncols). smem needs (32/LPB) * kRedStride floats; the caller must
// have finished every other use of smem. Ends with a barrier.
template <int M, int LPB, class Store>
__device__ __forceinline__ void reduce_phases(float (&acc)[M][32 / LPB], float* smem, int Lr,
                                              int P, int ncols, Store store) {
  constexpr int CPL = 32 / LPB;
  const int t = threadIdx.x;
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) smem[cc * kRedStride + t] = acc[m][cc];
    __syncthreads();
    for (int o = t; o < ncols; o += kThreads) {
      const int ob = o / kBlockWeights;
      const int c32 = o - ob * kBlockWeights;
      const int pp = c32 / CPL;
      const int cc = c32 - pp * CPL;
      const int vv = ob * LPB + pp;
      float sum = 0.0f;
      for (int rr = 0; rr < P; ++rr) sum += smem[cc * kRedStride + rr * Lr + vv];
      store(m, o, sum);
    }
    __syncthreads();
  }
}

}  // namespace q4
