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
constexpr int kThreads = 256;  // lanes per workgroup of the decode tiles

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
    uint32_t lo = b.q[w] & 0x0f0f0f0fu;
    uint32_t hi = b.q[w] & 0xf0f0f0f0u;
    // Hide the masks from the optimizer: otherwise it folds each
    // (masked >> 8n) & 0xff into a 4-bit field extract plus a convert, instead
    // of one v_cvt_f32_ubyteN per nibble.
    asm volatile("" : "+v"(lo), "+v"(hi));
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

// Sum of S values src[0], src[stride], ... in index order, with the loads
// issued in groups of 8 so that they overlap.
__device__ __forceinline__ float sum_strided(const float* __restrict__ src, size_t stride, int S) {
  float v = 0.0f;
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = src[(size_t)(s + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += t[u];
  }
  for (; s < S; ++s) v += src[(size_t)s * stride];
  return v;
}

}  // namespace q4

namespace q4 {

// Buffer resource over [base, base + bytes) (raw buffer, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Load lane share `part` of a block through a buffer resource: vofs is the
// lane's byte offset of the block, sofs a workgroup-uniform byte offset.
template <int LPB>
__device__ __forceinline__ void load_part_buf(__amdgpu_buffer_rsrc_t r, uint32_t vofs, uint32_t sofs,
                                              int part, BlockPart<LPB>& out) {
  out.d = __builtin_amdgcn_raw_buffer_load_b16(r, vofs, sofs, 0);
  const uint32_t qo = vofs + 2 + part * (16 / LPB);
  if constexpr (LPB == 1) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, qo, sofs, 0);
    out.q[0] = v[0];
    out.q[1] = v[1];
    out.q[2] = v[2];
    out.q[3] = v[3];
  } else if constexpr (LPB == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, qo, sofs, 0);
    out.q[0] = v[0];
    out.q[1] = v[1];
  } else {
    out.q[0] = __builtin_amdgcn_raw_buffer_load_b32(r, qo, sofs, 0);
  }
}

// ---------------------------------------------------------------------------
// Split-K tile. A workgroup of T lanes owns Jt consecutive block columns
// (j0 .. j0+Jt-1) and the rows [k0, k0 + rows) of a K x NB-block matrix. Its
// lanes form P = T / (Jt*LPB) row phases of Lr = Jt*LPB lanes; lane t is row
// phase r = t / Lr, block column j0 + (t % Lr) / LPB, share (t % Lr) % LPB, and
// walks rows k0 + r, k0 + r + P, ... . The Lr lanes of a row phase read one
// contiguous 18*Jt-byte row segment, so a wave's loads are coalesced row
// segments. All rows of a lane (at most RB) are loaded before any is used:
// one memory round trip per tile. Weights and activations are read through
// buffer resources (one 32-bit lane offset, uniform per-row scalar offsets).
//   x, x_bytes : activations; row m of the tile's activations is x + xoff[m]
//                floats, indexed by the matrix row k
// ---------------------------------------------------------------------------
struct SplitTile {
  const uint8_t* B;
  int NB, K;        // blocks per row, rows of the whole matrix
  int j0, Jt;       // first block column, block columns of the tile
  int k0, rows;     // row range of the tile
  int Lr, P;        // lanes per row phase, row phases
};

template <int M, int LPB, int RB>
__device__ __forceinline__ void tile_accumulate(const SplitTile& g, const float* __restrict__ x,
                                                uint32_t x_bytes, const int (&xoff)[M],
                                                float (&acc)[M][32 / LPB], float (&corr)[M]) {
  const int t = threadIdx.x;
  const int r = t / g.Lr;
  const int v = t - r * g.Lr;
  const int jj = v / LPB;
  const int part = v - jj * LPB;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    corr[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < 32 / LPB; ++c) acc[m][c] = 0.0f;
  }
  if (r >= g.P || jj >= g.Jt || g.j0 + jj >= g.NB) return;
  const uint32_t row_bytes = (uint32_t)g.NB * kBlockBytes;
  const uint32_t mat_bytes = (uint32_t)g.K * row_bytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.B, mat_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, x_bytes);
  // lane part of the offsets: its block column and its row phase r
  const uint32_t vw = (uint32_t)(g.j0 + jj) * kBlockBytes + (uint32_t)r * row_bytes;
  const uint32_t vx = (uint32_t)r * 4u;
  for (int base = 0; base < g.rows; base += g.P * RB) {  // uniform trip count
    // this lane's rows in the batch: k0 + base + r + i*P, i < nv
    const int nv = min(RB, (g.rows - base - r + g.P - 1) / g.P);
    BlockPart<LPB> b[RB];
    float xv[RB][M];
    if (nv == RB) {
      // Full batch: no branches between the loads and their uses, and the
      // loads are issued in row order (scheduling barriers), so each row's
      // FMAs wait only for that row's loads (loads complete in issue order).
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint32_t row = (uint32_t)(g.k0 + base + i * g.P);  // uniform
        load_part_buf<LPB>(rw, vw, row * row_bytes, part, b[i]);
#pragma unroll
        for (int m = 0; m < M; ++m)
          xv[i][m] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rx, vx, (row + (uint32_t)xoff[m]) * 4u, 0));
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        fma_part<M, LPB>(xv[i], b[i], acc, corr);
        __builtin_amdgcn_sched_barrier(0);  // keep rows in load order
      }
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (i < nv) {
          const uint32_t row = (uint32_t)(g.k0 + base + i * g.P);
          load_part_buf<LPB>(rw, vw, row * row_bytes, part, b[i]);
#pragma unroll
          for (int m = 0; m < M; ++m)
            xv[i][m] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rx, vx, (row + (uint32_t)xoff[m]) * 4u, 0));
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i)
        if (i < nv) fma_part<M, LPB>(xv[i], b[i], acc, corr);
    }
  }
}

// LDS floats needed by reduce_phases.
template <int LPB>
constexpr int phase_lds_floats() {
  return (32 / LPB) * (256 + 1);
}

// Sum a split-K tile over its P row phases through LDS, in phase order 0..P-1,
// one activation row at a time, and hand each tile output (m, o), o in
// [0, ncols), to store(m, o, v). Needs 256 lanes and phase_lds_floats<LPB>()
// floats of smem; contains workgroup barriers; ends with a barrier.
template <int M, int LPB, class Store>
__device__ __forceinline__ void reduce_phases(float (&acc)[M][32 / LPB], float* smem, int Lr,
                                              int P, int ncols, Store store) {
  constexpr int CPL = 32 / LPB;
  constexpr int kStride = 256 + 1;
  const int t = threadIdx.x;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) smem[cc * kStride + t] = acc[m][cc];
    __syncthreads();
    for (int o = t; o < ncols; o += 256) {
      const int ob = o / kBlockWeights;
      const int c32 = o - ob * kBlockWeights;
      const int pp = c32 / CPL;
      const int cc = c32 - pp * CPL;
      const int vv = ob * LPB + pp;
      float sum = 0.0f;
      for (int rr = 0; rr < P; ++rr) sum += smem[cc * kStride + rr * Lr + vv];
      store(m, o, sum);
    }
  }
  __syncthreads();
}

}  // namespace q4
