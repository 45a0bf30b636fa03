// Matrix-core (fp32 v_mfma_f32_4x4x1_16b_f32) tile of a Q4_0 GEMV, shared by the
// decode GEMV at batch 3..8 and the MoE expert tiles of 3..8 pairs.
//
// One MFMA "block" b (4 lanes, lane = 4b + q) is one Q4_0 block (row k, block
// column j). Lane q holds
//   A operand: s = x[q + 4h][k] * d[k][j]      (activation row q + 4h)
//   B operand: nibble i of qs dword q          (column 32j + 8q + i)
// so the 4x4 product adds s * nibble to output (m = q' + 4h, n = 32j + 8q + i)
// of every lane pair (q', q): one weight per lane per instruction (one convert
// per weight, as in the vector kernels) against 4 activation rows (8 with the
// two h halves). The instruction rounds exactly like v_fma_f32 (one rounding;
// checked bit for bit on MI355X), so each accumulator is the same fp32 FMA
// chain a vector lane would form. The -8 offset is folded out: acc = sum of
// s * nibble, corr = sum of s, y = acc - 8 * corr; odd nibbles come from the
// byte masked with 0xF0 (16x) and are rescaled at the end, which is exact.
//
// Tile: a workgroup of NW waves owns JW block columns and the rows
// [k0, k0 + rows) of one matrix. The 16 MFMA blocks of a wave are JW columns
// x PW = 16/JW row phases; the waves are further phases, PT = NW*PW in all
// (phase myph = wave*PW + ph), and phase p takes rows p, p + PT, ... in order.
// Each lane loads its 4-byte qs dword and 2-byte scale per row with buffer
// loads from a buffer over the tile's rows only (rows past the tile read zeros
// with no memory access), kMfmaRB rows per batch, kMfmaSets batches in flight
// in a register ring. Each wave copies the activations of its own rows batch
// by batch into a private LDS ring (LDS-DMA, issued with the batch's weight
// loads), so no wave waits for a workgroup-wide activation tile before its
// first products and the loop needs no barrier.
#pragma once

#include "q4_device.hpp"

namespace q4 {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMfmaRB = 4;      // rows per lane and batch
constexpr int kMfmaSets = 2;    // batches in flight (measured: 3 or 4 are slower)

template <int MH, int JW, int NW>
struct MfmaShape {
  static constexpr int PW = 16 / JW;        // row phases inside a wave
  static constexpr int PT = NW * PW;        // row phases of the workgroup (NW waves)
  static constexpr int NT = NW * kWaveSize; // lanes per workgroup
  static constexpr int XW = 4 * MH;         // staged activation floats per row
  static constexpr int NE = 8 * MH / PW;    // accumulator quads per lane after the wave sum
  static constexpr int TW = JW * 32;        // tile columns
  static constexpr int OUT = TW * 4 * MH;   // tile outputs (rows 0 .. 4*MH-1)
  static constexpr int XB = kMfmaRB * PW * XW;                 // activations of a wave's batch
  static constexpr int XI = (XB + kWaveSize - 1) / kWaveSize;  // LDS-DMA copies per batch
  static constexpr int XSLOT = XI * kWaveSize;                 // ring slot (whole copies)
  static_assert(JW == 4 || JW == 8, "tile widths of 4 or 8 blocks");
};

// LDS bytes of the activation rings of a workgroup (kMfmaSets slots per wave).
template <int MH, int JW, int NW>
__host__ __device__ constexpr int mfma_ring_bytes() {
  return NW * kMfmaSets * MfmaShape<MH, JW, NW>::XSLOT * 4;
}

// One row of the lane: s = x * d (and its correction sum) and the 8 nibbles
// of its qs dword as floats (low nibbles 0..15, high nibbles 16x).
template <int MH>
struct MfmaRowOps {
  float s[MH];
  float f[8];
};
template <int MH>
__device__ __forceinline__ void mfma_row_prep(const float (&xv)[MH], uint32_t dbits, uint32_t qs,
                                              MfmaRowOps<MH>& r, float (&corr)[MH]) {
  const float d = half_bits_to_float(dbits);
  {
    // corr sums exactly the rounded s the products use (all-8 nibbles cancel)
#pragma clang fp contract(off)
#pragma unroll
    for (int h = 0; h < MH; ++h) {
      r.s[h] = xv[h] * d;
      corr[h] += r.s[h];
    }
  }
  uint32_t lo = qs & 0x0f0f0f0fu;
  uint32_t hi = qs & 0xf0f0f0f0u;
  asm volatile("" : "+v"(lo), "+v"(hi));  // keep one v_cvt_f32_ubyteN per nibble
#pragma unroll
  for (int by = 0; by < 4; ++by) {
    r.f[2 * by] = static_cast<float>((lo >> (8 * by)) & 0xffu);
    r.f[2 * by + 1] = static_cast<float>((hi >> (8 * by)) & 0xffu);
  }
}
// The row's products: nibble i against the MH activation halves.
template <int MH>
__device__ __forceinline__ void mfma_row_products(const MfmaRowOps<MH>& r, v4f (&acc)[MH][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int h = 0; h < MH; ++h)
      acc[h][i] = __builtin_amdgcn_mfma_f32_4x4x1f32(r.s[h], r.f[i], acc[h][i], 0, 0, 0);
}

// Geometry of one tile.
struct MfmaTileGeom {
  const uint8_t* B;  // the matrix (K rows of NB blocks)
  int NB;            // blocks per row
  int j0;            // first block column of the tile
  int k0, rows;      // row range of the tile
};

// Accumulate one tile (raw acc and corr per lane; see above). Activation row m
// of the tile is x + xoff[m] floats, indexed by the matrix row, for m < M;
// rows m >= M are zero. x_bytes bounds every activation read. smem must hold
// mfma_ring_bytes<MH, JW, NW>() bytes; every copy into it has landed when the
// function returns (callers that reuse it for phase sums start with a barrier).
template <int MH, int JW, int NW>
__device__ __forceinline__ void mfma_tile_accumulate(const MfmaTileGeom& g,
                                                     const float* __restrict__ x,
                                                     uint32_t x_bytes, const int (&xoff)[4 * MH],
                                                     int M, float* smem, v4f (&acc)[MH][8],
                                                     float (&corr)[MH]) {
  using SH = MfmaShape<MH, JW, NW>;
  constexpr int PW = SH::PW, PT = SH::PT, XW = SH::XW, RB = kMfmaRB;
  constexpr int XI = SH::XI, XSLOT = SH::XSLOT;
  constexpr uint32_t kOut = 0x80000000u;
  const int t = threadIdx.x;
  const int lane = t % kWaveSize;
  const int wave = t / kWaveSize;
  const int q = lane & 3;
  const int blk = lane >> 2;
  const int jj = blk % JW;
  const int ph = blk / JW;
  const int k0 = g.k0;
  const int rows = g.rows;
  const int nl = (rows + PT - 1) / PT;  // rows of the busiest lane (uniform)
  const int nb = (nl + RB - 1) / RB;     // batches (uniform)
  const int myph = wave * PW + ph;
  const int j0 = g.j0;
  constexpr int NSET = kMfmaSets;

  // Activation ring of this wave: slot k holds batch b (b % NSET == k) as
  // [row i][phase p][e], e = 2q + h holding row m = q + 4h (MH = 2) or e = q
  // holding m = q (MH = 1), so a lane reads a row's values with one LDS load.
  // DMA lane c of copy u fills element u*64 + c: its matrix row and activation
  // row are fixed per lane, the batch moves the row by RB*PT. Lanes past the
  // batch, rows m >= M and rows past the tile read zeros.
  float* ring = smem + wave * NSET * XSLOT;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, x_bytes);
  uint32_t xo[XI];
  int xrow[XI];
#pragma unroll
  for (int u = 0; u < XI; ++u) {
    const int l = u * kWaveSize + lane;
    const int i = l / (PW * XW);
    const int rem = l - i * (PW * XW);
    const int p = rem / XW;
    const int e = rem - p * XW;
    const int m = MH == 2 ? (e >> 1) + 4 * (e & 1) : e;
    int xm = 0;
#pragma unroll
    for (int mm = 0; mm < 4 * MH; ++mm)
      if (mm == m) xm = xoff[mm];
    xrow[u] = i * PT + wave * PW + p;
    const bool ok = l < SH::XB && m < M;
    xo[u] = ok ? (uint32_t)(xm + k0 + xrow[u]) * 4u : kOut;
    if (!ok) xrow[u] = 0x40000000;
  }

  // Weights: a buffer over this tile's rows, so rows past the tile are out of
  // range; blocks past the matrix's last column get bit 31 (out of range too).
  const uint32_t pitch = (uint32_t)g.NB * kBlockBytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.B + (size_t)k0 * pitch, (uint32_t)rows * pitch);
  const bool colok = j0 + jj < g.NB;
  const uint32_t lane0 = (uint32_t)myph * pitch + (uint32_t)(j0 + jj) * kBlockBytes;
  const uint32_t vs0 = colok ? lane0 : kOut;
  const uint32_t vq0 = colok ? lane0 + 2u + 4u * (uint32_t)q : kOut;
  const uint32_t step = (uint32_t)PT * pitch;  // bytes between a lane's rows

  // Register sets of NSET batches in a ring: batch b lives in set b % NSET.
  // A batch issues its activation copies first, then its weight loads.
  uint32_t Q[NSET][RB], D[NSET][RB];
  auto load = [&](int b, int k) {
    const int brow = b * RB * PT;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const uint32_t o = brow + xrow[u] < rows ? xo[u] + (uint32_t)brow * 4u : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_void_t*)(ring + k * XSLOT + u * kWaveSize), 4, o, 0, 0, 0);
    }
    const uint32_t bo = (uint32_t)(b * RB) * step;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      Q[k][i] = __builtin_amdgcn_raw_buffer_load_b32(rw, vq0 + bo + (uint32_t)i * step, 0, 0);
      D[k][i] = __builtin_amdgcn_raw_buffer_load_b16(rw, vs0 + bo + (uint32_t)i * step, 0, 0);
    }
  };
#pragma unroll
  for (int h = 0; h < MH; ++h) {
    corr[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // Rows past the tile load zeros (zero scale) against zero activations, so
  // every batch runs whole. Batch b's copies have landed once at most its own
  // weight loads and the NSET - 1 batches issued after it are outstanding (the
  // loop issues batches in order, also past the last one).
  auto compute = [&](int b, int k) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * RB + (NSET - 1) * (XI + 2 * RB)));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const float* xs = ring + k * XSLOT;
    float xv[RB][MH];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int tr = i * PW + ph;
      if constexpr (MH == 2) {
        const float2 v = *reinterpret_cast<const float2*>(xs + tr * XW + 2 * q);
        xv[i][0] = v.x;
        xv[i][1] = v.y;
      } else {
        xv[i][0] = xs[tr * XW + q];
      }
    }
    // All conversions of the batch first, then its products: no product waits
    // on the conversion just before it, and one wave's products run on the
    // matrix core while another wave converts. Measured against conversions
    // interleaved with the products (each product right after its convert):
    // dense decode step 165.8 -> 154.3 us, 32-token MoE call 346 -> 344 us.
    MfmaRowOps<MH> ops[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) mfma_row_prep<MH>(xv[i], D[k][i], Q[k][i], ops[i], corr);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < RB; ++i) mfma_row_products<MH>(ops[i], acc);
  };

#pragma unroll
  for (int k = 0; k < NSET; ++k) load(k, k);
  __builtin_amdgcn_sched_barrier(0);

  // The scheduling barriers keep each batch's loads in issue order, so the
  // waits before a batch count only that batch's loads. A slot is refilled
  // only after the batch that read it has used its values (the LDS reads are
  // waited for before the products that follow them).
  int b = 0;
  for (; b + NSET <= nb; b += NSET) {
#pragma unroll
    for (int k = 0; k < NSET; ++k) {
      compute(b + k, k);
      __builtin_amdgcn_sched_barrier(0);
      load(b + k + NSET, k);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  static_assert(NSET == 2, "the tail's wait assumes one batch issued after it");
#pragma unroll
  for (int k = 0; k < NSET - 1; ++k)
    if (b + k < nb) compute(b + k, k);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

}  // namespace q4
