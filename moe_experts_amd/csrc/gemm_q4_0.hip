// Prefill GEMM over Q4_0 weights on the gfx950 matrix cores:
//   Y[M x N] (fp32) = X[M x K] (fp16) . deq(B[K x N]) with fp32 accumulation.
//
// The batched prompt matmul of the "2000-line C++ DeepSeek inference engine"
// article (§5.2: all prompt tokens in one large matmul) and the quantized
// tensor-core GEMM the KTransformers DeepSeek-V2 tutorial uses for prefill
// ("Optimization 2", Marlin). This is a dense contraction, so it runs on MFMA
// (v_mfma_f32_32x32x16_f16). The weights keep the pages' layout (blocks of
// 32 along N within a row), so a column's K values sit in different rows and
// the B operand is dequantized into LDS transposed ([n][k]).
//
// gemm_q4_0_kernel (K % 64 == 0, N % 128 == 0, X 16-byte and B 4-byte aligned):
//   * workgroup tile 256 x 128 and 512 lanes: 4 consumer waves, each 64 rows
//     x all 128 columns (eight 32 x 32 accumulators), only issue MFMAs; 4
//     producer waves issue the copies and dequantize, so the VALU work runs
//     beside the MFMAs on each SIMD; K steps of 64. The dequantization per
//     step scales with the tile's columns and the MFMA work with its area,
//     so the tall tile halves the dequant per MFMA of a 128 x 256 tile at
//     the same LDS traffic and grid size (measured: the dequant, not the
//     MFMAs, set the pace of the 128 x 256 tile);
//   * X tiles (16-byte chunks) and raw Q4_0 row segments (4 blocks = 72
//     bytes per row, in dwords) are copied global -> LDS by LDS-DMA loads (no
//     registers), X three and B four steps deep, issued two and three steps
//     ahead;
//   * each step the lanes dequantize the next step's raw B into an fp16 tile
//     [n][k]: w = fp16((q - 8) * d) with packed half arithmetic, one rounding;
//   * both LDS tiles are XOR-swizzled in 16-byte chunks, so the MFMA operand
//     reads (16 bytes per lane, 32 rows) and the dequant stores spread over
//     the LDS banks; for X the swizzle is applied on the source side of the
//     copy;
//   * one barrier per step, preceded by explicit waits for this wave's copies
//     and LDS stores (a plain __syncthreads would also drain the copies that
//     are meant to stay in flight).
// gemm_q4_0_generic_kernel handles every other shape: 128 x 128 tiles, K
// steps of 32, X through registers, B read block by block.
#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kPad = 8;                 // halves of padding per LDS row
constexpr int LDA = BK + kPad;          // halves per A row in LDS
constexpr int LDB = BK + kPad;          // halves per B column in LDS
constexpr int kGemmThreads = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const uint16_t* __restrict__ X;
  const uint8_t* __restrict__ B;
  float* __restrict__ Y;
  int M, N, K, NB, tiles_n;
};

// Registers carrying one K step of global data for one lane.
struct Stage {
  uint4 a[2];        // two 8-half chunks of X
  uint32_t dq[2];    // scale bits of rows k, k+1
  uint32_t q[2];     // 4 qs bytes (8 columns) of rows k, k+1
};

__device__ __forceinline__ void load_stage(const GemmArgs& g, int m0, int n0, int k0, Stage& st) {
  const int t = threadIdx.x;
  // X: 128 rows x 32 halves = 512 chunks of 8 halves, two per lane.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + i * kGemmThreads;
    const int row = q >> 2;
    const int kc = (q & 3) * 8;
    const int m = m0 + row;
    const int k = k0 + kc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < g.M) {
      const uint16_t* src = g.X + (size_t)m * g.K + k;
      if (k + 8 <= g.K && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
        v = *reinterpret_cast<const uint4*>(src);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (k + e < g.K) ? src[e] : (uint16_t)0;
        __builtin_memcpy(&v, h, 16);
      }
    }
    st.a[i] = v;
  }
  // B: 32 rows x 4 blocks; lane -> row pair kp (0..15), block column jb, quarter qq.
  const int kp = t >> 4;
  const int jb = (t >> 2) & 3;
  const int qq = t & 3;
  const int j = (n0 >> 5) + jb;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int k = k0 + 2 * kp + r;
    if (k < g.K && j < g.NB) {
      const uint8_t* blk = g.B + ((size_t)k * g.NB + j) * kBlockBytes;
      st.dq[r] = *reinterpret_cast<const uint16_t*>(blk);
      __builtin_memcpy(&st.q[r], blk + 2 + 4 * qq, 4);
    } else {
      st.dq[r] = 0u;      // zero scale: the padded weights are exactly zero
      st.q[r] = 0x88888888u;
    }
  }
}

__device__ __forceinline__ void store_stage(const Stage& st, _Float16* As, _Float16* Bs) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + i * kGemmThreads;
    const int row = q >> 2;
    const int kc = (q & 3) * 8;
    *reinterpret_cast<uint4*>(As + row * LDA + kc) = st.a[i];
  }
  const int kp = t >> 4;
  const int jb = (t >> 2) & 3;
  const int qq = t & 3;
  // Packed (row k, row k+1) scales.
  const uint32_t dpair = (st.dq[0] & 0xffffu) | (st.dq[1] << 16);
  const half2v d2 = __builtin_bit_cast(half2v, dpair);
  const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int by = 0; by < 4; ++by) {
    const uint32_t b0 = (st.q[0] >> (8 * by)) & 0xffu;
    const uint32_t b1 = (st.q[1] >> (8 * by)) & 0xffu;
    // binary16 0x6400 | v has the value 1024 + v (v < 1024): exact nibble values.
    const uint32_t lo = 0x64006400u | (b0 & 0xfu) | ((b1 & 0xfu) << 16);
    const uint32_t hi = 0x64006400u | (b0 >> 4) | ((b1 >> 4) << 16);
    const half2v wlo = (__builtin_bit_cast(half2v, lo) - off) * d2;  // (q - 8) * d, one rounding
    const half2v whi = (__builtin_bit_cast(half2v, hi) - off) * d2;
    const int n = jb * 32 + qq * 8 + 2 * by;
    *reinterpret_cast<half2v*>(Bs + n * LDB + 2 * kp) = wlo;
    *reinterpret_cast<half2v*>(Bs + (n + 1) * LDB + 2 * kp) = whi;
  }
}

__global__ __launch_bounds__(kGemmThreads) void gemm_q4_0_generic_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * LDB];

  const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int tm = L / g.tiles_n;
  const int tn = L - tm * g.tiles_n;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (g.K + BK - 1) / BK;
  Stage st;
  load_stage(g, m0, n0, 0, st);
  store_stage(st, As[0], Bs[0]);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) load_stage(g, m0, n0, (ks + 1) * BK, st);
    const _Float16* as = As[cur];
    const _Float16* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      const int kl = kk + 8 * (lane >> 5);
      half8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8*>(as + (wm * 64 + i * 32 + (lane & 31)) * LDA + kl);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8*>(bs + (wn * 64 + j * 32 + (lane & 31)) * LDB + kl);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) store_stage(st, As[cur ^ 1], Bs[cur ^ 1]);
    __syncthreads();
  }

  // Accumulator layout of a 32 x 32 fp32 MFMA result: lane l holds column
  // l % 32; register r holds row 8*(r/4) + 4*(l/32) + r%4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < g.M) g.Y[(size_t)row * g.N + col] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------
// Aligned-shape kernel
// ---------------------------------------------------------------------------
namespace fast {
// Tile heights: 256 rows for a plain GEMM, 96 for expert-grouped m-tiles
// (a prefill expert has tens to hundreds of rows: about 77 for DeepSeek-V2
// at 2048 tokens, which fill a 96-row tile 80 % and a 128-row tile 60 %).
constexpr int kDenseBM = 256, kGroupedBM = kGemmRows;
constexpr int BN = 128, BK = 64;
constexpr int kXStages = 3, kRStages = 4;
constexpr int kRowBytes = (BN / kBlockWeights) * kBlockBytes;  // 72 bytes of raw row segment
constexpr int kRowWords = kRowBytes / 4;                  // 18 dwords (copied 4 bytes at a time)
constexpr int kRowPitch = kRowBytes + 4;                  // LDS row pitch: one pad dword
constexpr int kRWords = BK * (kRowWords + 1);             // 1216 dword slots, pads included
constexpr int kRInstr = (kRWords + kGemmThreads - 1) / kGemmThreads;  // 5
constexpr int kRBytes = kRInstr * kGemmThreads * 4;       // 5 KiB
constexpr int kBBytes = BN * BK * 2;                      // 16 KiB fp16 tile
constexpr int kUnits = BN * BK / 16;                      // dequant units (2 rows x 8 columns)
constexpr int kUL = kUnits / kGemmThreads;                // 2 per producer lane

// The X stage and what depends on the tile height BM and on the number NM
// of weight matrices a workgroup contracts with the same X tile (2: an
// expert's gate and up matrices). LDS: [X stages][matrix 0: raw stages, B
// tiles][matrix 1: ...].
template <int BM, int NM>
struct XCfg {
  static constexpr int kXChunks = BM * BK / 8;            // 16-byte chunks per stage: 2048 at 256
  static constexpr int kXBytes = kXChunks * 16;           // 32 KiB at 256 rows
  static constexpr int kXInstr = kXChunks / kGemmThreads; // 8 at 256 rows
  static constexpr int kGroup = kXInstr + NM * kRInstr;   // copies issued per step
  static constexpr int kMatBytes = kRStages * kRBytes + 2 * kBBytes;
  static constexpr int kLdsBytes = kXStages * kXBytes + NM * kMatBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(BM % 32 == 0 && kXChunks % kGemmThreads == 0, "32-row bands, whole copy passes");
};

typedef __attribute__((address_space(3))) void lds_void_t;

struct Args {
  const uint16_t* X;  // M rows of K halves
  const uint8_t* B;
  float* Y;
  int M, N, K, NB, tiles_n, nk;
  // Expert-grouped mode (tiles != null): m-tile i is tiles[i] = (expert e,
  // first output row, rows <= BM); its weights are the e-th of consecutive
  // K x N matrices of mat_bytes; output row q reads X row src[q] (src null:
  // row q). Only the first *n_tiles m-tiles exist.
  const int4* tiles;
  const int* n_tiles;
  const int32_t* src;
  size_t mat_bytes;
  // Two matrices per workgroup. With H set (gate B and up B1, same shape) the
  // output is H = fp16(SiLU(X . B) * (X . B1)) instead of Y. With H null, B1
  // is B shifted by one column tile (128 columns) and the workgroup writes
  // two adjacent column tiles of Y (cpw = 2 column tiles per workgroup).
  const uint8_t* B1;
  _Float16* H;
  int cpw;
};

constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

template <int BM, int NM>
__device__ __forceinline__ uint8_t* xstage(uint8_t* lds, int s) {
  return lds + s * XCfg<BM, NM>::kXBytes;
}
template <int BM, int NM>
__device__ __forceinline__ uint8_t* rstage(uint8_t* lds, int m, int s) {
  return lds + kXStages * XCfg<BM, NM>::kXBytes + m * XCfg<BM, NM>::kMatBytes + s * kRBytes;
}
template <int BM, int NM>
__device__ __forceinline__ uint8_t* bstage(uint8_t* lds, int m, int s) {
  return lds + kXStages * XCfg<BM, NM>::kXBytes + m * XCfg<BM, NM>::kMatBytes +
         kRStages * kRBytes + s * kBBytes;
}

// LDS tiles hold rows of 64 halves (128 bytes = 8 chunks of 16 bytes); chunk
// c of row r is stored at position c ^ swz(r). A 16-byte read is served 16
// lanes at a time: with rows of 32 banks, lanes on consecutive rows hit
// disjoint banks when the even rows and the odd rows each take 8 different
// positions, which (r >> 1) & 7 gives. The B tile adds r >> 5 (the block
// column), which spreads the dequant stores of one instruction (4 blocks of
// the same column offset) over the banks too.
__device__ __forceinline__ int swz_x(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_b(int n) { return ((n >> 1) ^ (n >> 5)) & 7; }

// Byte offset of the fp16 pair (k, k+1), k = 2*kp, of column n in a B tile.
__device__ __forceinline__ uint32_t bpos(int n, int kp) {
  return (uint32_t)n * (BK * 2) + (uint32_t)(((kp >> 2) ^ swz_b(n)) << 4) +
         (uint32_t)((kp & 3) << 2);
}

// Dequantization units: unit u = t + 256*i (2 per producer lane) covers row pair
// kp (rows 2kp, 2kp+1), block jb and quarter qq (8 columns), with bits
// u[0:3] = kp % 16, u[4] = qq % 2, u[5] = kp / 16, u[6:7] = jb, u[8] = qq / 2:
// the 64 lanes of a wave span 32 row pairs x 2 quarters of one block. With
// raw rows 76 bytes apart in LDS (a pad dword per row) this spreads the raw
// reads and the tile stores over the LDS banks (chosen by a search over bit
// assignments with a bank model of both operations).
__device__ __forceinline__ int unit_kp(int u) { return (u & 15) | (((u >> 5) & 1) << 4); }
__device__ __forceinline__ int unit_jb(int u) { return (u >> 6) & 3; }
__device__ __forceinline__ int unit_qq(int u) { return ((u >> 4) & 1) | (((u >> 8) & 1) << 1); }

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A producer lane's loop-invariant offsets. Copies: lane byte offsets of its
// chunks at K step 0 (the step goes into the scalar offset; chunks past M or
// past the tile read out of range), and the wave's LDS slot offsets.
// Dequant: per unit, the offsets of the scale and of the aligned nibble
// dwords inside a raw stage, the alignbyte shift, and the store offsets of
// its four column pairs inside a B tile (column n+1 is 128 bytes after n).
template <int BM, int NM>
struct Producer {
  static constexpr int kXInstr = XCfg<BM, NM>::kXInstr;
  __amdgpu_buffer_rsrc_t rx, rb[NM];
  uint32_t xoff[kXInstr], roff[kRInstr];
  uint32_t wslot;                 // wave's first DMA slot byte offset (uniform)
  uint32_t x_step, r_step;        // bytes per K step in X and B (uniform)
  uint32_t rd[kUL], rw[kUL], sh[kUL];
  uint32_t st[kUL][4];
  int nk;

  __device__ __forceinline__ void init(const Args& g, const uint8_t* const (&B)[NM], int m0,
                                       int rows, int j0, int t) {
    constexpr uint32_t kOut = 0x80000000u;
    nk = g.nk;
    rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(g.X), (short)0,
                                           (int)((uint32_t)g.M * (uint32_t)g.K * 2u), 0x00020000);
#pragma unroll
    for (int m = 0; m < NM; ++m)
      rb[m] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(B[m]), (short)0,
                                           (int)((uint32_t)g.K * (uint32_t)g.NB * kBlockBytes),
                                           0x00020000);
    const uint32_t row_bytes = (uint32_t)g.NB * kBlockBytes;
    x_step = BK * 2;
    r_step = BK * row_bytes;
    wslot = (uint32_t)__builtin_amdgcn_readfirstlane(t >> 6) * (kWaveSize * 16);
#pragma unroll
    for (int i = 0; i < kXInstr; ++i) {
      const int slot = i * kGemmThreads + t;  // row r = slot / 8, stored position slot % 8
      const int r = slot >> 3;
      const int c = (slot & 7) ^ swz_x(r);   // source chunk landing in that position
      const int xr = r < rows ? (g.src ? g.src[m0 + r] : m0 + r) : 0;
      xoff[i] = r < rows ? ((uint32_t)xr * (uint32_t)g.K + 8u * c) * 2u : kOut;
    }
#pragma unroll
    for (int i = 0; i < kRInstr; ++i) {
      const int q = i * kGemmThreads + t;  // LDS slot: raw row q / 19, dword q % 19
      const int row = q / (kRowWords + 1);
      const int pc = q - row * (kRowWords + 1);
      roff[i] = (q < kRWords && pc < kRowWords)
                    ? (uint32_t)row * row_bytes + (uint32_t)j0 * kBlockBytes + 4u * pc
                    : kOut;
    }
#pragma unroll
    for (int i = 0; i < kUL; ++i) {
      const int u = t + i * kGemmThreads;
      const int kp = unit_kp(u), jb = unit_jb(u), qq = unit_qq(u);
      rd[i] = (uint32_t)(2 * kp) * kRowPitch + jb * kBlockBytes;
      const uint32_t o = rd[i] + 2 + 4 * qq;  // 2-byte aligned; row 2kp+1 is 76 bytes on
      sh[i] = o & 3u;
      rw[i] = o - sh[i];
      const int nb = jb * 32 + qq * 8;
#pragma unroll
      for (int by = 0; by < 4; ++by) st[i][by] = bpos(nb + 2 * by, kp);
    }
  }

  // Copies of K step ks: X into stage ks % 3, raw B into stage ks % 4. The
  // copies issued past the last step (ks >= nk) repeat step nk - 1: they land
  // in an X stage of a step that is never computed, or in a raw stage whose
  // B tile is never read, so no lane needs a select to keep its offset in
  // range.
  __device__ __forceinline__ void issue_x(uint8_t* lds, int ks) const {
    const uint32_t so = (uint32_t)min(ks, nk - 1) * x_step;
    uint8_t* dst = xstage<BM, NM>(lds, ks % kXStages) + wslot;
#pragma unroll
    for (int i = 0; i < kXInstr; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + i * kGemmThreads * 16), 16,
                                               xoff[i], so, 0, 0);
  }
  __device__ __forceinline__ void issue_r(uint8_t* lds, int ks) const {
    const uint32_t so = (uint32_t)min(ks, nk - 1) * r_step;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      uint8_t* dst = rstage<BM, NM>(lds, m, ks % kRStages) + wslot / 4;
#pragma unroll
      for (int i = 0; i < kRInstr; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[m], (lds_void_t*)(dst + i * kGemmThreads * 4),
                                                 4, roff[i], so, 0, 0);
    }
  }

  // Raw stage -> fp16 B tile, w = fp16((q - 8) * d).
  __device__ __forceinline__ void dequant(const uint8_t* __restrict__ rsb,
                                          uint8_t* __restrict__ bsb) const {
    const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
    uint32_t d0[kUL], d1[kUL], q0[kUL], q1[kUL];
#pragma unroll
    for (int i = 0; i < kUL; ++i) {
      const uint8_t* pd = rsb + rd[i];
      const uint8_t* pw = rsb + rw[i];
      d0[i] = *reinterpret_cast<const uint16_t*>(pd);
      d1[i] = *reinterpret_cast<const uint16_t*>(pd + kRowPitch);
      const uint32_t a0 = *reinterpret_cast<const uint32_t*>(pw);
      const uint32_t a1 = *reinterpret_cast<const uint32_t*>(pw + 4);
      const uint32_t b0 = *reinterpret_cast<const uint32_t*>(pw + kRowPitch);
      const uint32_t b1 = *reinterpret_cast<const uint32_t*>(pw + kRowPitch + 4);
      q0[i] = __builtin_amdgcn_alignbyte(a1, a0, sh[i]);
      q1[i] = __builtin_amdgcn_alignbyte(b1, b0, sh[i]);
    }
#pragma unroll
    for (int i = 0; i < kUL; ++i) {
      const half2v d2 = __builtin_bit_cast(half2v, d0[i] | (d1[i] << 16));
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        // bytes [q0.by, 0, q1.by, 0]: row 2kp's byte in the low half, row
        // 2kp+1's in the high half (v_perm_b32; selector 0x0c gives zero)
        const uint32_t sel = 0x0c000c00u | ((4u + by) << 16) | by;
        const uint32_t pair = __builtin_amdgcn_perm(q1[i], q0[i], sel);
        // binary16 0x6400 | v is 1024 + v exactly (v < 1024)
        const uint32_t lo = (pair & 0x000f000fu) | 0x64006400u;
        const uint32_t hi = ((pair >> 4) & 0x000f000fu) | 0x64006400u;
        const half2v wlo = (__builtin_bit_cast(half2v, lo) - off) * d2;  // one rounding
        const half2v whi = (__builtin_bit_cast(half2v, hi) - off) * d2;
        uint8_t* pst = bsb + st[i][by];
        *reinterpret_cast<half2v*>(pst) = wlo;
        *reinterpret_cast<half2v*>(pst + BK * 2) = whi;
      }
    }
  }
};

// 512 lanes: waves 0-3 contract (MFMA only), waves 4-7 produce (copies and
// dequantization). Both roles pass one barrier per K step, so a step's
// dequant (VALU) runs on the same SIMDs while the matrix cores run the MFMAs.
template <int BM, int NM>
__global__ __launch_bounds__(2 * kGemmThreads) void gemm_q4_0_kernel(Args g) {
  static_assert(NM == 1 || (NM == 2 && BM != 256), "gate and up together in grouped tiles");
  constexpr int kGroup = XCfg<BM, NM>::kGroup;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int m0, rows, tn;
  const uint8_t* B[NM];
  B[0] = g.B;
  if constexpr (NM == 2) B[1] = g.B1;
  if (g.tiles) {
    // grouped: all column tiles of an m-tile on one XCD (they read the same X
    // rows, and neighbouring 72-byte row segments of the weights share 128-byte
    // lines, so that XCD's L2 fetches both once), m-tiles round robin over the
    // 8 XCDs (the live m-tiles come first in the list). Workgroup b runs on XCD
    // b % 8 as that XCD's (b / 8)-th workgroup. With plain dispatch order the
    // column tiles of an m-tile landed on different XCDs and the gate/up pass
    // read 2.9x its algorithmic bytes from HBM.
    const int i = blockIdx.x / kNumXcd;
    const int tile = (int)(blockIdx.x % kNumXcd) + kNumXcd * (i / g.tiles_n);
    tn = i % g.tiles_n;
    if (tile >= *g.n_tiles) return;  // the whole workgroup, before any barrier
    const int4 tl = g.tiles[tile];
#pragma unroll
    for (int m = 0; m < NM; ++m) B[m] += (size_t)tl.x * g.mat_bytes;
    m0 = tl.y;
    rows = tl.z;
  } else {
    const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
    const int tm = L / g.tiles_n;
    tn = L - tm * g.tiles_n;
    m0 = tm * BM;
    rows = g.M - m0;
  }
  const int j0 = tn * g.cpw * (BN / kBlockWeights);
  const int wave = threadIdx.x >> 6;

  if (wave >= 4) {
    // ------------------------------------------------------------ producer
    Producer<BM, NM> pr;
    pr.init(g, B, m0, rows, j0, (int)threadIdx.x - kGemmThreads);
    // Prologue: X(0), raw(0), raw(1) | X(1), raw(2); then raw(0) -> B(0).
    pr.issue_x(lds, 0);
    pr.issue_r(lds, 0);
    pr.issue_r(lds, 1);
    pr.issue_x(lds, 1);
    pr.issue_r(lds, 2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGroup + NM * kRInstr));  // X(0), raw(0) landed
    lds_barrier();                                           // barrier A
#pragma unroll
    for (int m = 0; m < NM; ++m) pr.dequant(rstage<BM, NM>(lds, m, 0), bstage<BM, NM>(lds, m, 0));
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGroup) & ~0x0f00);  // raw(1); B(0) stores done
    lds_barrier();                                           // barrier B: X(0), B(0) ready
    for (int ks = 0; ks < g.nk; ++ks) {
      // X two steps ahead, raw B three (the stages they overwrite were last
      // read before the previous barrier)
      pr.issue_x(lds, ks + 2);
      pr.issue_r(lds, ks + 3);
      __builtin_amdgcn_sched_barrier(0);
      // B(ks+1) from raw(ks+1); on the last step the raw stage holds a
      // repeat of the last step and the tile is never read
#pragma unroll
      for (int m = 0; m < NM; ++m)
        pr.dequant(rstage<BM, NM>(lds, m, (ks + 1) % kRStages),
                   bstage<BM, NM>(lds, m, (ks + 1) & 1));
      // X(ks+1), raw(ks+2) (issued one step ago) landed; B(ks+1) stores done
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGroup) & ~0x0f00);
      lds_barrier();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no copy lands after the workgroup ends
    return;
  }

  // -------------------------------------------------------------- consumer
  const int lane = threadIdx.x & 63;
  // Consumer wave tiles: 256-row tiles give each wave 64 rows x all 128
  // columns; 128-row tiles a 2 x 2 grid of 64 x 64 (each wave then reads half
  // the B tile instead of all of it: 64 instead of 80 KB of LDS reads per step);
  // 96-row tiles give each wave all 96 rows x 32 columns.
  constexpr int WGR = BM == 256 ? 4 : (BM == 128 ? 2 : 1);  // waves along the rows
  constexpr int WR = BM / WGR;            // rows per wave (64 or 96)
  constexpr int WC = BN / (4 / WGR);      // columns per wave (128, 64 or 32)
  constexpr int MI = WR / 32, NJ = WC / 32;
  const int wm = wave % WGR;
  const int wn = wave / WGR;
  float16v acc[NM][MI][NJ];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.0f;
  lds_barrier();  // barrier A
  lds_barrier();  // barrier B
  for (int ks = 0; ks < g.nk; ++ks) {
    const uint8_t* xs = xstage<BM, NM>(lds, ks % kXStages);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kc = 2 * kk + (lane >> 5);  // 16-byte k chunk of this lane
      half8 af[MI], bf[NM][NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * WR + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const half8*>(xs + (r * 8 + (kc ^ swz_x(r))) * 16);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint8_t* bs = bstage<BM, NM>(lds, m, ks & 1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = wn * WC + j * 32 + (lane & 31);
          bf[m][j] = *reinterpret_cast<const half8*>(bs + n * (BK * 2) + ((kc ^ swz_b(n)) << 4));
        }
      }
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[m][i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[m][j], acc[m][i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS reads done before the stage is reused
    lds_barrier();
  }

  // Accumulator layout of a 32 x 32 fp32 MFMA result: lane l holds column
  // l % 32; register r holds row 8*(r/4) + 4*(l/32) + r%4.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = j0 * kBlockWeights + wn * WC + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = wm * WR + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (rr >= rows) continue;
        if constexpr (NM == 1) {
          g.Y[(size_t)(m0 + rr) * g.N + col] = acc[0][i][j][r];
        } else if (g.H) {
          // gate and up of one expert: h = fp16(SiLU(gate) * up)
          const float gt = acc[0][i][j][r];
          g.H[(size_t)(m0 + rr) * g.N + col] =
              (_Float16)(gt / (1.0f + expf(-gt)) * acc[1][i][j][r]);
        } else {
          // two adjacent column tiles
          g.Y[(size_t)(m0 + rr) * g.N + col] = acc[0][i][j][r];
          g.Y[(size_t)(m0 + rr) * g.N + col + BN] = acc[1][i][j][r];
        }
      }
    }
}
}  // namespace fast

}  // namespace

hipError_t launch_gemm(const uint16_t* X, const uint8_t* B, float* Y, int M, int N, int K,
                       hipStream_t st) {
  GemmArgs g;
  g.X = X;
  g.B = B;
  g.Y = Y;
  g.M = M;
  g.N = N;
  g.K = K;
  g.NB = N / kBlockWeights;
  g.tiles_n = (N + BN - 1) / BN;
  // X rows are copied in 16-byte chunks, raw B rows in dwords
  const bool aligned = (reinterpret_cast<uintptr_t>(X) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(B) & 3) == 0;
  if (K % fast::BK == 0 && N % fast::BN == 0 && aligned) {
    fast::Args f;
    f.X = X;
    f.B = B;
    f.Y = Y;
    f.M = M;
    f.N = N;
    f.K = K;
    f.NB = N / kBlockWeights;
    f.tiles_n = N / fast::BN;
    f.nk = (K + fast::BK - 1) / fast::BK;
    f.tiles = nullptr;
    f.n_tiles = nullptr;
    f.src = nullptr;
    f.mat_bytes = 0;
    f.B1 = nullptr;
    f.H = nullptr;
    f.cpw = 1;
    constexpr int BM = fast::kDenseBM;
    const long long tiles = (long long)((M + BM - 1) / BM) * f.tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fast::gemm_q4_0_kernel<BM, 1>), dim3((unsigned)tiles),
                       dim3(2 * kGemmThreads), (fast::XCfg<BM, 1>::kLdsBytes), st, f);
    return hipGetLastError();
  }
  const int tiles_m = (M + BM - 1) / BM;
  const long long tiles = (long long)tiles_m * g.tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_q4_0_generic_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, st,
                     g);
  return hipGetLastError();
}

bool gemm_grouped_supported(int N, int K) { return K % fast::BK == 0 && N % fast::BN == 0; }

// Expert-grouped launches: the gate and up matrices together (B1 set:
// H = fp16(SiLU(X . B) * (X . B1))), or one matrix into fp32 Y, two adjacent
// column tiles per workgroup when N % 256 == 0.
hipError_t launch_gemm_grouped(const uint16_t* X, int x_rows, const uint8_t* B, const uint8_t* B1,
                               size_t mat_bytes, float* Y, _Float16* H, int N, int K,
                               const int4* tiles, const int* n_tiles, int max_tiles,
                               const int32_t* src, hipStream_t st) {
  fast::Args f;
  f.X = X;
  f.B = B;
  f.Y = Y;
  f.M = x_rows;
  f.N = N;
  f.K = K;
  f.NB = N / kBlockWeights;
  f.tiles_n = N / fast::BN;
  f.nk = K / fast::BK;
  f.tiles = tiles;
  f.n_tiles = n_tiles;
  f.src = src;
  f.mat_bytes = mat_bytes;
  f.B1 = B1;
  f.H = H;
  f.cpw = 1;
  if (!B1 && N % (2 * fast::BN) == 0) {
    f.B1 = B + (fast::BN / kBlockWeights) * kBlockBytes;  // the next 128 columns of each row
    f.cpw = 2;
    f.tiles_n = N / (2 * fast::BN);
  }
  // every XCD gets ceil(max_tiles / 8) m-tile slots of tiles_n workgroups
  const long long grid = (long long)((max_tiles + kNumXcd - 1) / kNumXcd) * kNumXcd * f.tiles_n;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (grid == 0) return hipSuccess;
  constexpr int BM = fast::kGroupedBM;
  if (f.B1)
    hipLaunchKernelGGL((fast::gemm_q4_0_kernel<BM, 2>), dim3((unsigned)grid),
                       dim3(2 * kGemmThreads), (fast::XCfg<BM, 2>::kLdsBytes), st, f);
  else
    hipLaunchKernelGGL((fast::gemm_q4_0_kernel<BM, 1>), dim3((unsigned)grid),
                       dim3(2 * kGemmThreads), (fast::XCfg<BM, 1>::kLdsBytes), st, f);
  return hipGetLastError();
}

}  // namespace q4
