// Prefill GEMM over Q4_0 weights on the gfx950 matrix cores:
//   Y[M x N] (fp32) = X[M x K] (fp16) . deq(B[K x N]) with fp32 accumulation.
//
// The batched prompt matmul of the "2000-line C++ DeepSeek inference engine"
// article (§5.2: all prompt tokens in one large matmul) and the quantized
// tensor-core GEMM the KTransformers DeepSeek-V2 tutorial uses for prefill
// ("Optimization 2", Marlin). This is a dense contraction, so it runs on MFMA
// (v_mfma_f32_32x32x16_f16):
//
//   * workgroup tile BM x BN = 128 x 128, 4 waves in a 2 x 2 grid, each wave
//     a 64 x 64 block of four 32 x 32 accumulators;
//   * per K step of BK = 32: the X tile is copied to LDS ([m][k], k contiguous);
//     the B tile is read as Q4_0 (each lane: two rows x one 8-column quarter
//     block) and dequantized in registers to fp16 with packed half arithmetic,
//     w = fp16((q - 8) * d) rounded once, then written to LDS transposed
//     ([n][k], k contiguous) so that both MFMA operands are 16-byte LDS reads;
//   * two LDS stages: the next tile's global loads are in flight while the
//     current one is contracted; one barrier per K step.
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

__global__ __launch_bounds__(kGemmThreads) void gemm_q4_0_kernel(GemmArgs g) {
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
  const int tiles_m = (M + BM - 1) / BM;
  const long long tiles = (long long)tiles_m * g.tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_q4_0_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace q4
