// Device-side building blocks shared by the Q4_0 decode kernels (gfx950).
//
// Q4_0 block ("2000-line C++ DeepSeek inference engine" article, §2.2): 18
// bytes, binary16 scale d then 16 bytes qs; weight 2i is the low nibble of
// qs[i], weight 2i+1 the high nibble; value (q - 8) * d.
//
// Arithmetic used on the GPU for one block and one activation value a:
//   s       = a * d                      (one fp32 multiply per block and row)
//   acc[2i]   += s * lo_i                (lo_i = q & 0x0F, exact)
//   acc[2i+1] += s * (16 * hi_i)         (the byte masked with 0xF0, exact; the
//                                         factor 16 is removed at the end,
//                                         which is exact in binary32)
//   corr      += s
//   result    = acc - 8 * corr           (so each weight costs one FMA per
//                                         activation row, plus its share of a
//                                         few bit operations: fma_part)
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
constexpr int kMaxLdsBytes = 160 * 1024;  // LDS of one workgroup on gfx950

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
// Even columns accumulate s * q, odd ones s * 16q (the high nibble left in
// place), with s = x * d; corr sums s. The nibbles are not converted one by
// one: a masked field q (or 16q) in the low bits of a 16-bit half is the
// binary16 subnormal q * 2^-24, which v_fma_mix_f32 takes as an fp16 operand
// and widens exactly. With s' = s * 2^24 (exact), s' * (q * 2^-24) is the same
// real number as s * q, so every FMA rounds exactly as fma(s, q, acc) would.
// Unpacking costs five bit operations per dword (eight weights) instead of
// two masks and eight byte conversions.
template <int M, int LPB>
__device__ __forceinline__ void fma_part(const float (&xv)[M], const BlockPart<LPB>& b,
                                         float (&acc)[M][32 / LPB], float (&corr)[M]) {
  const float d = half_bits_to_float(b.d);
  float s[M], sw[M];
  {
    // corr must sum exactly the rounded s that the FMAs below use, so that
    // acc - 8 * corr cancels exactly when every nibble is 8: no contraction
    // of s into the corr addition.
#pragma clang fp contract(off)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      s[m] = xv[m] * d;
      corr[m] += s[m];
      sw[m] = s[m] * 16777216.0f;  // 2^24
    }
  }
#pragma unroll
  for (int w = 0; w < BlockPart<LPB>::kWords; ++w) {
    const uint32_t q = b.q[w];
    const uint32_t q8 = q >> 8;
    // halves (low, high): bytes 0 and 2, then bytes 1 and 3, of the dword;
    // columns 2*byte (low nibble) and 2*byte + 1 (16 x high nibble)
    const uint32_t h[4] = {q & 0x000f000fu, q & 0x00f000f0u, q8 & 0x000f000fu,
                           q8 & 0x00f000f0u};
    constexpr int kCol[4][2] = {{0, 4}, {1, 5}, {2, 6}, {3, 7}};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v0 = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h[k]));
      const float v1 = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(h[k] >> 16)));
      const int c0 = 8 * w + kCol[k][0], c1 = 8 * w + kCol[k][1];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        acc[m][c0] = __builtin_fmaf(sw[m], v0, acc[m][c0]);
        acc[m][c1] = __builtin_fmaf(sw[m], v1, acc[m][c1]);
      }
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
// Block formats of the vector split-K tiles. Every format stores blocks of 32
// weights along N, a binary16 scale d first; LPB lanes split a block, each
// holding 32 / LPB consecutive columns. A format supplies:
//   kBlockBytes             bytes per block;
//   kOffset                 whether weights carry the "- 8" offset that the
//                           tile folds into one correction sum per row;
//   Part<LPB>               the raw bytes of one lane's share (the scale bits
//                           and kWords dwords of values);
//   load<LPB>(...)          load a share through a buffer resource (vofs: the
//                           lane's byte offset of the block, sofs: uniform);
//   accumulate<M, LPB>(...) unpack a share and add s * value into acc[m][c]
//                           (c = column within the share) for M rows;
//   finish(sum, c, csum)    turn column c's summed accumulator into output;
// and its tile shape: kJt block columns per workgroup, lanes_per_block(M),
// rows_per_batch(M) (rows per lane in one pipelined batch) and
// grid_target(M) (workgroups the split-K plan aims at). The tile walk, the
// activation staging, the phase sums, the split-K plan and the reduction are
// shared, so a format is a template parameter of one kernel.
// ---------------------------------------------------------------------------

// Q4_0 ("2000-line C++ DeepSeek inference engine" article, §2.2): 18 bytes,
// 16 bytes of nibbles after the scale, value (q - 8) * d; arithmetic as set
// out at the top of this file.
struct Q4_0Format {
  static constexpr int kBlockBytes = 18;
  static constexpr bool kOffset = true;
  static constexpr int kJt = 16;
  template <int LPB>
  using Part = BlockPart<LPB>;
  __host__ __device__ static constexpr int lanes_per_block(int M) { return M == 1 ? 1 : 2; }
  __host__ __device__ static constexpr int rows_per_batch(int M) { return M <= 4 ? 8 : 4; }
  __host__ __device__ static constexpr int grid_target(int) { return 512; }
  template <int LPB>
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t vofs,
                                              uint32_t sofs, int part, Part<LPB>& out) {
    load_part_buf<LPB>(r, vofs, sofs, part, out);
  }
  template <int M, int LPB>
  __device__ __forceinline__ static void accumulate(const float (&xv)[M], const Part<LPB>& b,
                                                    float (&acc)[M][32 / LPB],
                                                    float (&corr)[M]) {
    fma_part<M, LPB>(xv, b, acc, corr);
  }
  // even columns hold sum(s * lo), odd ones sum(s * 16 * hi): both minus 8 * sum(s)
  __device__ __forceinline__ static float finish(float sum, int c, float csum) {
    return ((c & 1) ? sum * 0.0625f : sum) - 8.0f * csum;
  }
};

// Q8_0: the article (§2.2) weighs it against Q4_0 (twice the bytes, about 60 %
// of Q4_0's token rate on the author's CPU) without defining it; read as 34
// little-endian bytes, the scale then 32 signed bytes q, weight l = q[l] * d.
// One convert (sign-extended byte to fp32) and one FMA per weight and row,
// s = x * d formed once per block and row.
template <int LPB>
struct Q8Part {
  static constexpr int kWords = 8 / LPB;
  uint32_t d;
  uint32_t q[kWords];
};

struct Q8_0Format {
  static constexpr int kBlockBytes = 34;
  static constexpr bool kOffset = false;
  static constexpr int kJt = 8;
  template <int LPB>
  using Part = Q8Part<LPB>;
  __host__ __device__ static constexpr int lanes_per_block(int M) { return M == 1 ? 2 : 4; }
  __host__ __device__ static constexpr int rows_per_batch(int) { return 4; }
  __host__ __device__ static constexpr int grid_target(int M) { return M >= 2 ? 512 : 352; }
  template <int LPB>
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t vofs,
                                              uint32_t sofs, int part, Part<LPB>& out) {
    out.d = __builtin_amdgcn_raw_buffer_load_b16(r, vofs, sofs, 0);
    const uint32_t qo = vofs + 2 + part * (32 / LPB);  // 2-byte aligned: unaligned loads
    if constexpr (LPB == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, qo, sofs, 0);
      out.q[0] = v[0];
      out.q[1] = v[1];
      out.q[2] = v[2];
      out.q[3] = v[3];
    } else {
      static_assert(LPB == 4, "half or quarter blocks");
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, qo, sofs, 0);
      out.q[0] = v[0];
      out.q[1] = v[1];
    }
  }
  template <int M, int LPB>
  __device__ __forceinline__ static void accumulate(const float (&xv)[M], const Part<LPB>& b,
                                                    float (&acc)[M][32 / LPB], float (&)[M]) {
    const float d = half_bits_to_float(b.d);
    float s[M];
#pragma unroll
    for (int m = 0; m < M; ++m) s[m] = xv[m] * d;
#pragma unroll
    for (int w = 0; w < Part<LPB>::kWords; ++w)
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        const float f = static_cast<float>(static_cast<int8_t>(b.q[w] >> (8 * by)));
        const int c = 4 * w + by;
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m][c] = __builtin_fmaf(s[m], f, acc[m][c]);
      }
  }
  __device__ __forceinline__ static float finish(float sum, int, float) { return sum; }
};

// ---------------------------------------------------------------------------
// Split-K tile. A workgroup of 256 lanes owns Jt consecutive block columns
// (j0 .. j0+Jt-1) and the rows [k0, k0 + rows) of a K x NB-block matrix. Its
// lanes form P = 256 / (Jt*LPB) row phases of Lr = Jt*LPB lanes; lane t is row
// phase r = t / Lr, block column j0 + (t % Lr) / LPB, share (t % Lr) % LPB, and
// walks tile rows r, r + P, r + 2P, ... . The Lr lanes of a row phase read one
// contiguous 18*Jt-byte row segment, so a wave's loads are coalesced row
// segments.
//
// Pipeline: a lane's rows go in batches of RB. Two register sets hold two
// batches; while one batch is unpacked and accumulated, the loads of the next
// are in flight (the loop is unrolled by two so the sets alternate without
// register copies). Loads are never predicated, so the compiler's memory
// waits count only the loads of the batch in use: a row past the tile end
// (and every row of an idle lane) is given a lane offset of 2^31, beyond the
// buffer's range (matrices are smaller than 2 GiB, and offset plus scalar
// offset stays below 2^32), so the load returns zeros without a memory
// access. Rows past the busiest lane's last row are skipped; a lane whose last
// row is past the tile adds zeros (zero scale, zero activation).
//
// Activations: the tile's activation rows are staged in LDS as
// xs[row * XW + m] (XW = M rounded up to 1, 2, 4 or 8; rows_pad = rows
// rounded up to whole batches, the padding zeroed) by LDS-DMA loads
// (buffer_load_dword ... lds): no registers, all issued before the weight
// batches, one round trip. A row's M values are one or two aligned LDS reads,
// the same address for all lanes of a row phase (broadcast).
//   x, x_bytes : activations; activation row m of the tile is x + xoff[m]
//                floats, indexed by the matrix row k
//   xs         : LDS of tile_x_floats<M>(rows, P, RB) floats
//                (may alias the scratch of reduce_phases, which starts with a
//                barrier)
// ---------------------------------------------------------------------------
struct SplitTile {
  const uint8_t* B;
  int NB, K;        // blocks per row, rows of the whole matrix
  int j0, Jt;       // first block column, block columns of the tile
  int k0, rows;     // row range of the tile
  int Lr, P;        // lanes per row phase, row phases
};

// Tile rows rounded up to whole batches of RB rows per lane.
__host__ __device__ constexpr int tile_rows_padded(int rows, int P, int RB) {
  return ((rows + P - 1) / P + RB - 1) / RB * RB * P;
}

// Floats per staged activation row (a power of two >= M).
template <int M>
__host__ __device__ constexpr int xs_width() {
  return M <= 2 ? M : (M <= 4 ? 4 : 8);
}

// LDS floats of the staged activation tile, rounded up to whole staging
// passes of 256 words (every DMA lane of the last pass writes inside it).
template <int M>
__host__ __device__ constexpr int tile_x_floats(int rows, int P, int RB) {
  return (tile_rows_padded(rows, P, RB) * xs_width<M>() + 255) / 256 * 256;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Issue the LDS-DMA copies of an activation tile: word q = row * XW + m of
// xs holds x[xoff[m] + k0 + row] for m < M and row < rows (lane q % 256 of
// pass q / 256 loads it; the DMA writes lane l of a wave at M0 + 4*l). Other
// words read out of range (no memory access).
template <int M>
__device__ __forceinline__ void stage_x_tile(const float* __restrict__ x, uint32_t x_bytes,
                                             const int (&xoff)[M], int k0, int rows, int rows_pad,
                                             float* __restrict__ xs) {
  constexpr int XW = xs_width<M>();
  constexpr uint32_t kOutOfRange = 0x80000000u;
  const int t = threadIdx.x;
  const int wave = t / kWaveSize;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, x_bytes);
  for (int q0 = 0; q0 < XW * rows_pad; q0 += kThreads) {
    const int q = q0 + t;
    const int row = q / XW;
    const int m = q - row * XW;
    int xo = 0;
#pragma unroll
    for (int mm = 0; mm < M; ++mm)
      if (mm == m) xo = xoff[mm];
    const uint32_t off = (m < M && row < rows) ? (uint32_t)(xo + k0 + row) * 4u : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(xs + q0 + wave * kWaveSize), 4, off,
                                             0, 0, 0);
  }
}

// Zero the padding rows [rows, rows_pad) of a staged activation tile.
template <int M>
__device__ __forceinline__ void zero_x_pad(float* __restrict__ xs, int rows, int rows_pad) {
  constexpr int XW = xs_width<M>();
  for (int idx = threadIdx.x; idx < (rows_pad - rows) * XW; idx += kThreads)
    xs[rows * XW + idx] = 0.0f;
}

// The M activations of tile row `row`.
template <int M>
__device__ __forceinline__ void read_x_row(const float* __restrict__ xs, int row,
                                           float (&xv)[M]) {
  constexpr int XW = xs_width<M>();
  const float* p = xs + row * XW;
  if constexpr (XW == 1) {
    xv[0] = p[0];
  } else if constexpr (XW == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    xv[0] = v.x;
    xv[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < XW / 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(p + 4 * q);
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (4 * q + u < M) xv[4 * q + u] = e[u];
    }
  }
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wave are outstanding (n < 64); LDS and export counters are not waited on.
constexpr int vmcnt_imm(int n) {
  return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

template <int M, int LPB, int RB, class Fmt = Q4_0Format>
__device__ __forceinline__ void tile_accumulate(const SplitTile& g, const float* __restrict__ x,
                                                uint32_t x_bytes, const int (&xoff)[M],
                                                float* __restrict__ xs,
                                                float (&acc)[M][32 / LPB], float (&corr)[M]) {
  using Part = typename Fmt::template Part<LPB>;
  constexpr uint32_t kOutOfRange = 0x80000000u;
  constexpr int kLoadsPerBatch = 2 * RB;  // scale + nibble load per row
  static_assert(2 * kLoadsPerBatch < 64, "vmcnt range");
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
  const bool active = r < g.P && jj < g.Jt && g.j0 + jj < g.NB;
  const int nl = (g.rows + g.P - 1) / g.P;  // rows of the busiest lane (uniform)
  const int nb = (nl + RB - 1) / RB;         // batches (uniform)
  const int rows_pad = nb * RB * g.P;
  const uint32_t row_bytes = (uint32_t)g.NB * Fmt::kBlockBytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.B, (uint32_t)g.K * row_bytes);
  const uint32_t vcol = (uint32_t)(g.j0 + jj) * Fmt::kBlockBytes;  // lane's block in row 0
  const uint32_t sbase = (uint32_t)g.k0 * row_bytes;                // uniform
  const int rows = active ? g.rows : 0;

  stage_x_tile<M>(x, x_bytes, xoff, g.k0, g.rows, rows_pad, xs);
  // The wait below counts on every staging load being issued before the
  // weight loads.
  __builtin_amdgcn_sched_barrier(0);

  Part A[RB], Bs[RB];
  auto load_batch = [&](int b, Part(&R)[RB]) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int tr = (b * RB + i) * g.P + r;  // tile row of this lane
      const uint32_t vo = tr < rows ? vcol + (uint32_t)tr * row_bytes : kOutOfRange;
      Fmt::template load<LPB>(rw, vo, sbase, part, R[i]);
    }
  };
  auto compute_batch = [&](int b, Part(&R)[RB]) {
    float xv[RB][M];
#pragma unroll
    for (int i = 0; i < RB; ++i) read_x_row<M>(xs, (b * RB + i) * g.P + r, xv[i]);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (b * RB + i < nl) Fmt::template accumulate<M, LPB>(xv[i], R[i], acc, corr);
      __builtin_amdgcn_sched_barrier(0);  // one row's unpacked values live at a time
    }
  };

  load_batch(0, A);
  load_batch(1, Bs);
  __builtin_amdgcn_sched_barrier(0);
  // The staged activations have landed once at most the two weight batches'
  // loads are outstanding; then zero the padding rows and share the tile.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerBatch));
  zero_x_pad<M>(xs, g.rows, rows_pad);
  __syncthreads();
  if (!active) return;

  // Pairs of batches, then an odd last batch. Loads of batches past the end
  // are out of range (no memory access) rather than skipped by a branch, so
  // every iteration issues the same loads in the same order.
  int b = 0;
  for (; b + 2 <= nb; b += 2) {
    compute_batch(b, A);
    load_batch(b + 2, A);
    compute_batch(b + 1, Bs);
    load_batch(b + 3, Bs);
  }
  if (b < nb) compute_batch(b, A);
}

// ---------------------------------------------------------------------------
// Split-K tile with wave-private weight staging (same lane roles and row
// order as tile_accumulate). Requires 16-byte aligned row segments: the
// matrix base and the row pitch (18*NB bytes, NB % 8 == 0) are multiples of
// 16 and the tile is JT = 8 or 16 blocks wide (144 or 288 bytes).
//
// A wave's lanes cover WP = 64 / Lr row phases, so for one batch of RB rows
// per lane the wave consumes WP*RB row segments of CPS = 18*JT/16 chunks of
// 16 bytes. The wave copies exactly those chunks into its own LDS buffer
// with LDS-DMA loads (buffer_load_dwordx4 ... lds): consecutive lanes fetch
// consecutive 16-byte chunks of a segment, so every request is an aligned,
// contiguous piece of a row and no registers hold the data in flight. Lanes
// then read their block share (scale and nibbles) from LDS. NBUF buffers per
// wave: batches b+1 .. b+NBUF-1 stream in while batch b is computed. Producer
// and consumer are the same wave, so a vmcnt wait (in issue order) is the
// only synchronisation; a buffer is refilled only after the reads of its
// previous batch have returned. Chunks of rows past the tile (and of batches
// past the end) get an out-of-range offset: no memory access.
// LDS layout: [activation tile][4 waves][NBUF buffers][kBufBytes].
// ---------------------------------------------------------------------------
template <int LPB, int RB, int JT>
struct StageShape {
  static constexpr int Lr = JT * LPB;               // lanes per row phase
  static constexpr int WP = kWaveSize / Lr;         // row phases per wave
  static constexpr int CPS = JT * kBlockBytes / 16; // chunks per row segment
  static constexpr int NCH = WP * RB * CPS;         // chunks per wave and batch
  static constexpr int NI = (NCH + kWaveSize - 1) / kWaveSize;  // DMA instructions
  // buffer: the DMA slots plus at least 4 bytes of read slack
  // (read_block_part_lds reads one dword past a share)
  static constexpr int kBufBytes = (NCH * 16 + 4 + 1023) / 1024 * 1024;
  static_assert(JT == 8 || JT == 16, "segments of whole 16-byte chunks");
  static_assert(kWaveSize % Lr == 0, "row phases must not straddle waves");
};

// LDS bytes of the staged tile: activation tile plus NBUF weight buffers per
// wave.
template <int M, int LPB, int RB, int JT, int NBUF>
__host__ __device__ constexpr int staged_lds_bytes(int rows) {
  return tile_x_floats<M>(rows, kThreads / (JT * LPB), RB) * 4 +
         (kThreads / kWaveSize) * NBUF * StageShape<LPB, RB, JT>::kBufBytes;
}

// Read lane share `part` of the block at byte offset blk of a staged buffer.
// The nibble bytes sit at a 2-byte but not always 4-byte aligned offset, and
// unaligned LDS reads stall, so the covering dwords are read at 4-byte
// aligned addresses and shifted into place (v_alignbyte_b32, shift 0 or 2).
// Reads up to 4 bytes past the share (staging buffers have that slack).
template <int LPB>
__device__ __forceinline__ void read_block_part_lds(const uint8_t* __restrict__ buf, uint32_t blk,
                                                    int part, BlockPart<LPB>& bp) {
  constexpr int NW = BlockPart<LPB>::kWords;
  bp.d = *reinterpret_cast<const uint16_t*>(__builtin_assume_aligned(buf + blk, 2));
  const uint32_t o = blk + 2 + (uint32_t)part * (16 / LPB);
  const uint32_t sh = o & 3u;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(buf + (o - sh), 4));
  uint32_t t[NW + 1];
#pragma unroll
  for (int k = 0; k <= NW; ++k) t[k] = w[k];
#pragma unroll
  for (int k = 0; k < NW; ++k) bp.q[k] = __builtin_amdgcn_alignbyte(t[k + 1], t[k], sh);
}

// Activations computed from split-K partial sums of a gate and an up
// projection instead of copied: x[i] = SiLU(g) * u with g = sum over s of
// part[s][i] and u = sum over s of part[S + s][i], each in split order from
// +0.0 (part: [2][S][slab] floats; x index i = xoff[m] + k0 + row as for a
// copied tile). At most kActMaxSplits splits and kActMaxVals tile words per
// lane (XW * rows_pad <= kActMaxVals * 256).
struct ActSource {
  const float* part;
  uint32_t part_bytes;
  uint32_t slab;
  int S;
};
constexpr int kActMaxSplits = 16;
constexpr int kActMaxVals = 2;

template <int M, int LPB, int RB, int JT, int NBUF>
__device__ __forceinline__ void tile_accumulate_staged(const SplitTile& g,
                                                       const float* __restrict__ x,
                                                       uint32_t x_bytes, const int (&xoff)[M],
                                                       uint8_t* __restrict__ lds,
                                                       float (&acc)[M][32 / LPB],
                                                       float (&corr)[M],
                                                       ActSource act = ActSource{nullptr, 0, 0, 0}) {
  using SS = StageShape<LPB, RB, JT>;
  constexpr uint32_t kOutOfRange = 0x80000000u;
  static_assert(NBUF >= 2 && NBUF * SS::NI < 64, "vmcnt range");
  const int t = threadIdx.x;
  const int lane = t % kWaveSize;
  const int wave = t / kWaveSize;
  const int P = kThreads / SS::Lr;
  const int r = t / SS::Lr;
  const int v = t - r * SS::Lr;
  const int jj = v / LPB;
  const int part = v - jj * LPB;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    corr[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < 32 / LPB; ++c) acc[m][c] = 0.0f;
  }
  const int nl = (g.rows + P - 1) / P;  // rows of the busiest lane (uniform)
  const int nb = (nl + RB - 1) / RB;     // batches (uniform)
  const int rows_pad = nb * RB * P;
  float* xs = reinterpret_cast<float*>(lds);
  uint8_t* wbuf = lds + tile_x_floats<M>(g.rows, P, RB) * 4 + wave * NBUF * SS::kBufBytes;
  const uint32_t row_bytes = (uint32_t)g.NB * kBlockBytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.B, (uint32_t)g.K * row_bytes);

  // Chunk q = 64*i + lane of a batch: segment s = q / CPS (row phase
  // wave*WP + s % WP, batch row s / WP), piece q % CPS. Its tile row in batch
  // b is b*RB*P + trow[i]; the scalar offset carries the batch.
  int trow[SS::NI];
  uint32_t voff[SS::NI];
#pragma unroll
  for (int i = 0; i < SS::NI; ++i) {
    const int q = i * kWaveSize + lane;
    const int sg = q / SS::CPS;
    const int pc = q - sg * SS::CPS;
    trow[i] = q < SS::NCH ? (sg / SS::WP) * P + wave * SS::WP + sg % SS::WP : 0x40000000;
    voff[i] = (uint32_t)g.j0 * kBlockBytes + (uint32_t)trow[i] * row_bytes + (uint32_t)pc * 16u;
  }
  auto stage_batch = [&](int b) {
    uint8_t* buf = wbuf + (b % NBUF) * SS::kBufBytes;
    const int brow = b * RB * P;
    const uint32_t soff = (uint32_t)(g.k0 + brow) * row_bytes;
#pragma unroll
    for (int i = 0; i < SS::NI; ++i) {
      const uint32_t vo = brow + trow[i] < g.rows ? voff[i] : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (lds_void_t*)(buf + i * kWaveSize * 16), 16, vo, brow < g.rows ? soff : 0u, 0, 0);
    }
  };

  if (act.part != nullptr) {
    // Every partial-sum load is issued before the weight copies (so the
    // compiler's wait for them does not include the copies), then the
    // activations are formed and stored.
    constexpr int XW = xs_width<M>();
    constexpr uint32_t kOut = 0x80000000u;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(act.part, act.part_bytes);
    float pv[kActMaxVals][2][kActMaxSplits];
#pragma unroll
    for (int v = 0; v < kActMaxVals; ++v) {
      const int q = v * kThreads + t;
      const int row = q / XW;
      const int m = q - row * XW;
      int xo = 0;
#pragma unroll
      for (int mm = 0; mm < M; ++mm)
        if (mm == m) xo = xoff[mm];
      const bool valid = m < M && row < g.rows;
      const uint32_t base = (uint32_t)(xo + g.k0 + row);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int sp = 0; sp < kActMaxSplits; ++sp) {
          const uint32_t o = (valid && sp < act.S)
                                 ? ((uint32_t)(h * act.S + sp) * act.slab + base) * 4u
                                 : kOut;
          pv[v][h][sp] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, o, 0, 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NBUF; ++b) stage_batch(b);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < kActMaxVals; ++v) {
      const int q = v * kThreads + t;
      if (q < XW * rows_pad) {
        float gs = 0.0f, us = 0.0f;  // out-of-range splits load +0.0: the sums are unchanged
#pragma unroll
        for (int sp = 0; sp < kActMaxSplits; ++sp) {
          gs += pv[v][0][sp];
          us += pv[v][1][sp];
        }
        const int row = q / XW;
        const int m = q - row * XW;
        xs[q] = (m < M && row < g.rows) ? gs / (1.0f + expf(-gs)) * us : 0.0f;
      }
    }
  } else {
    stage_x_tile<M>(x, x_bytes, xoff, g.k0, g.rows, rows_pad, xs);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NBUF; ++b) stage_batch(b);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NBUF * SS::NI));  // activations landed
    zero_x_pad<M>(xs, g.rows, rows_pad);
  }
  // Share the activation tile. A plain __syncthreads() would also wait for
  // the weight copies in flight (its release fence waits on every memory
  // operation); the tile's own copies have landed (vmcnt above), so only the
  // LDS stores need a wait before the barrier.
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // lane's block share inside a staged segment, and its segment in a batch
  const int seg0 = (lane / SS::Lr);  // row phase within the wave
  const int in_seg = jj * kBlockBytes;
  for (int b = 0; b < nb; ++b) {
    // batch b landed (b+1 .. b+NBUF-1 in flight)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 1) * SS::NI));
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* buf = wbuf + (b % NBUF) * SS::kBufBytes;
    // Every LDS read of the batch first (rows past the tile read the zeros
    // their copies wrote and the zero-padded activations), so the batch waits
    // once for LDS instead of once per row.
    BlockPart<LPB> bp[RB];
    float xv[RB][M];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      read_block_part_lds<LPB>(buf, (i * SS::WP + seg0) * (SS::CPS * 16) + in_seg, part, bp[i]);
      read_x_row<M>(xs, (b * RB + i) * P + r, xv[i]);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i)
      if (b * RB + i < nl) fma_part<M, LPB>(xv[i], bp[i], acc, corr);  // uniform
    // every read of this buffer has returned before it is refilled
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    stage_batch(b + NBUF);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no copy may land after the tile
}

// LDS floats needed by reduce_phases: the larger of its two paths. Full
// 16-block tiles: one activation row's wave sums (4 waves x 16 block columns x
// kPhaseBlockPitch) and, for formats with the offset, the wave sums of the
// corrections of all rows. Narrower tiles: one row's accumulators of all
// phases and, with the offset, the raw corrections and their phase sums.
constexpr int kPhaseBlockPitch = 36;  // floats per block column: 16-byte rows, banks spread
template <int M, int LPB, class Fmt = Q4_0Format>
constexpr int phase_lds_floats() {
  constexpr int tree = 4 * 16 * kPhaseBlockPitch + (Fmt::kOffset ? 4 * M * 16 * LPB : 0);
  constexpr int flat = (32 / LPB) * (256 + 1) + (Fmt::kOffset ? M * (256 + 1) + M * 256 : 0);
  return tree > flat ? tree : flat;
}

// a + b where a comes from this lane and b from the lane 32 (or 16) away:
// lanes below the distance return a_lo + a_hi, lanes above it b_lo + b_hi.
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                  __builtin_bit_cast(uint32_t, b), false, false);
  const uint32_t r0 = r[0];
  const uint32_t r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                  __builtin_bit_cast(uint32_t, b), false, false);
  const uint32_t r0 = r[0];
  const uint32_t r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// Sum a split-K tile over its P row phases, then finish each output once with
// Fmt::finish. For Q4_0: even columns sum - 8*csum, odd columns sum/16 -
// 8*csum (csum = the phase sum of the corrections; both rescalings are exact).
// The phase sum is linear, so finishing after it equals finishing every lane
// first, at 1/P of the work; the corrections run through the same order as
// the accumulators, so acc - 8*corr still cancels exactly when every nibble is
// 8 (8 and 128 are powers of two). Formats without the offset skip the
// corrections. Hands each tile output (m, o), o in [0, ncols) with ncols <=
// 512, to store(m, o, v). Needs 256 lanes and phase_lds_floats<M, LPB>()
// floats of smem; contains workgroup barriers; ends with a barrier.
//
// Full tiles (16 block columns, Lr = 16*LPB lanes per phase, P = 16/LPB):
// lane l of wave w holds row phase 4w/LPB + l/Lr. Inside the wave the phases
// are summed by reduce-scatter lane swaps (distance 32, then 16 for LPB = 1),
// which leaves each lane 8 columns of its block share; the 4 waves' sums then
// meet in LDS once. The order is fixed: with p the 16 phases at LPB = 1, wave w
// gives W_w = (p[4w] + p[4w+2]) + (p[4w+1] + p[4w+3]) and the tile sum is
// ((W_0 + W_1) + W_2) + W_3 (at LPB = 2, W_w = p[2w] + p[2w+1]; at LPB = 4,
// W_w = p[w]). The MoE matrix-core tiles sum their 16 phases in the same order.
// Narrower tiles (fewer block columns, or Q8_0's 8) sum the phases through LDS
// in phase order 0..P-1.
template <int M, int LPB, class Fmt = Q4_0Format, class Store>
__device__ __forceinline__ void reduce_phases_full(const float (&acc)[M][32 / LPB],
                                                   const float (&corr)[M], float* smem,
                                                   int ncols, Store store) {
  constexpr int CPL = 32 / LPB;  // columns per lane share
  constexpr int PW = 4 / LPB;    // row phases per wave
  constexpr int NV = CPL / PW;   // columns per lane after the in-wave sums
  constexpr int Lr = 16 * LPB;
  static_assert(NV == 8 && kThreads == 256, "16 block columns, 4 waves");
  float* W = smem;                                   // [wave][block][kPhaseBlockPitch]
  float* CW = W + 4 * 16 * kPhaseBlockPitch;         // [wave][m][Lr] corrections
  const int t = threadIdx.x;
  const int lane = t & (kWaveSize - 1);
  const int wave = t / kWaveSize;
  const int v = lane & (Lr - 1);  // block share: block v / LPB, part v % LPB
  const int g = lane / Lr;        // phase within the wave
  float* wdst = W + (wave * 16 + v / LPB) * kPhaseBlockPitch + (v % LPB) * CPL + NV * g;

  // corrections: wave sums of all rows (every lane of a phase group gets them)
  float cw[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float c = corr[m];
    if constexpr (PW >= 2) c += __shfl_xor(c, 32);
    if constexpr (PW == 4) c += __shfl_xor(c, 16);
    cw[m] = c;
  }
  __syncthreads();  // smem may still hold the tile's staging
  if constexpr (Fmt::kOffset) {
    if (g == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) CW[(wave * M + m) * Lr + v] = cw[m];
    }
  }
  // this thread's outputs o = t and t + 256: block, column, lane share
  int bo_[2], c32_[2], vv_[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = t + 256 * k;
    bo_[k] = o / kBlockWeights;
    c32_[k] = o - bo_[k] * kBlockWeights;
    vv_[k] = bo_[k] * LPB + c32_[k] / CPL;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float R[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) R[c] = acc[m][c];
    if constexpr (PW >= 2) {
#pragma unroll
      for (int u = 0; u < CPL / 2; ++u) R[u] = swap_sum32(R[u], R[u + CPL / 2]);
    }
    if constexpr (PW == 4) {
#pragma unroll
      for (int u = 0; u < CPL / 4; ++u) R[u] = swap_sum16(R[u], R[u + CPL / 4]);
    }
    *reinterpret_cast<float4*>(wdst) = float4{R[0], R[1], R[2], R[3]};
    *reinterpret_cast<float4*>(wdst + 4) = float4{R[4], R[5], R[6], R[7]};
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int o = t + 256 * k;
      if (o < ncols) {
        const float* src = W + bo_[k] * kPhaseBlockPitch + c32_[k];
        float sum = src[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) sum += src[w * 16 * kPhaseBlockPitch];
        float csum = 0.0f;
        if constexpr (Fmt::kOffset) {
          const float* cs = CW + m * Lr + vv_[k];
          csum = cs[0];
#pragma unroll
          for (int w = 1; w < 4; ++w) csum += cs[w * M * Lr];
        }
        store(m, o, Fmt::finish(sum, c32_[k] % CPL, csum));
      }
    }
    __syncthreads();
  }
}

template <int M, int LPB, class Fmt = Q4_0Format, class Store>
__device__ __forceinline__ void reduce_phases(const float (&acc)[M][32 / LPB],
                                              const float (&corr)[M], float* smem, int Lr, int P,
                                              int ncols, Store store) {
  if (Lr == 16 * LPB) {  // uniform: full 16-block tiles
    reduce_phases_full<M, LPB, Fmt>(acc, corr, smem, ncols, store);
    return;
  }
  constexpr int CPL = 32 / LPB;
  constexpr int kStride = 256 + 1;
  float* A = smem;                  // [CPL][kStride] accumulators of one row m
  float* C = A + CPL * kStride;     // [M][kStride] corrections
  float* CS = C + M * kStride;      // [M][256] phase sums of the corrections
  const int t = threadIdx.x;
  __syncthreads();
  if constexpr (Fmt::kOffset) {
#pragma unroll
    for (int m = 0; m < M; ++m) C[m * kStride + t] = corr[m];
    __syncthreads();
    for (int q = t; q < M * Lr; q += 256) {
      const int m = q / Lr;
      const int v = q - m * Lr;
      float sum = 0.0f;
      for (int rr = 0; rr < P; ++rr) sum += C[m * kStride + rr * Lr + v];
      CS[m * 256 + v] = sum;
    }
  }
  // this thread's outputs o = t and t + 256
  int cc_[2], vv_[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = t + 256 * k;
    const int ob = o / kBlockWeights;
    const int c32 = o - ob * kBlockWeights;
    const int pp = c32 / CPL;
    cc_[k] = c32 - pp * CPL;
    vv_[k] = ob * LPB + pp;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) A[cc * kStride + t] = acc[m][cc];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int o = t + 256 * k;
      if (o < ncols) {
        const float* src = A + cc_[k] * kStride + vv_[k];
        float sum = 0.0f;
        for (int rr = 0; rr < P; ++rr) sum += src[rr * Lr];
        const float csum = Fmt::kOffset ? CS[m * 256 + vv_[k]] : 0.0f;
        store(m, o, Fmt::finish(sum, cc_[k], csum));
      }
    }
    __syncthreads();
  }
}

}  // namespace q4
