// Decode GEMV over Q4_0 weights: y[M x N] = x[M x K] . deq(B[K x N]), M <= 8.
//
// The fused dequantize-inside-the-inner-loop matmul of the "2000-line C++
// DeepSeek inference engine" article (§3.4 matmul_q4_0), re-designed for
// gfx950. B is row-major with blocks along N, so a column's weights are spread
// over all K rows while each 128-byte cache line holds ~7 consecutive blocks of
// one row. To keep memory requests full, a workgroup reads whole 16-block row
// segments (288 bytes), and to still have hundreds of workgroups on a 4096-row
// matrix it owns only a K range of those columns (split-K):
//
//   1. gemv_q4_0_kernel: workgroup (c, s) owns block columns 16c..16c+15 and
//      rows [s*Kt, (s+1)*Kt). Its lanes form row phases of 16 (or 32) lanes;
//      each lane loads every one of its rows (one 16-byte or 8-byte unaligned
//      buffer load plus the 2-byte scale, and the activations) before using
//      any, unpacks the nibbles in registers (masked bytes, v_cvt_f32_ubyteN)
//      and accumulates one fp32 FMA per weight and activation row. The row
//      phases are summed through LDS in a fixed order; the workgroup writes its
//      partial sums to the workspace (or y directly when K is not split).
//   2. gemv_q4_0_reduce_kernel: y[m][n] = sum over the K splits, in split order.
// Cross-workgroup hand-off at agent scope costs an L2 write-back per workgroup
// on this GPU, so the split-K sum is a second kernel instead: no atomics, no
// fences, deterministic results.
#include <cstdlib>

#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

struct GemvArgs {
  const float* __restrict__ x;
  const uint8_t* __restrict__ B;
  float* __restrict__ y;
  float* __restrict__ part;  // [S][M][N] split-K partials
  int M, N, K, NB;
  int Jt, Lr, P, C, Kt, S;
};

// Rows per lane in one pipelined batch (two batches are held in registers).
template <int M, int LPB>
constexpr int rows_per_batch() {
  return M <= 2 ? 8 : (M <= 4 ? (LPB == 1 ? 6 : 8) : 4);
}

// Rows per lane in one batch of the staged path, and weight buffers per wave.
template <int M, int LPB>
constexpr int staged_rows_per_batch() {
  return LPB == 1 ? 4 : 8;
}
template <int M, int LPB>
constexpr int staged_buffers() {
  return 2;
}
constexpr int kStagedJt = 16;

template <int M, int LPB, bool STAGED>
__global__ __launch_bounds__(kThreads) void gemv_q4_0_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int c = L % a.C;
  const int s = L / a.C;
  SplitTile g;
  g.B = a.B;
  g.NB = a.NB;
  g.K = a.K;
  g.j0 = c * a.Jt;
  g.Jt = a.Jt;
  g.k0 = s * a.Kt;
  g.rows = min(a.Kt, a.K - g.k0);
  g.Lr = a.Lr;
  g.P = a.P;
  int xoff[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xoff[m] = m * a.K;
  float acc[M][32 / LPB];
  float corr[M];
  if constexpr (STAGED)
    tile_accumulate_staged<M, LPB, staged_rows_per_batch<M, LPB>(), kStagedJt,
                           staged_buffers<M, LPB>()>(
        g, a.x, (uint32_t)(4 * M * a.K), xoff, reinterpret_cast<uint8_t*>(smem), acc, corr);
  else
    tile_accumulate<M, LPB, rows_per_batch<M, LPB>()>(g, a.x, (uint32_t)(4 * M * a.K), xoff,
                                                       smem, acc, corr);
  const int n0 = g.j0 * kBlockWeights;
  const int ncols = min(a.Jt, a.NB - g.j0) * kBlockWeights;
  float* dst = (a.S == 1) ? a.y : a.part + (size_t)s * M * a.N;
  reduce_phases<M, LPB>(acc, corr, smem, a.Lr, a.P, ncols,
                        [&](int m, int o, float v) { dst[(size_t)m * a.N + n0 + o] = v; });
}

// y[i] = part[0][i] + part[1][i] + ... + part[S-1][i], in split order. With
// SMAX > 0 (S <= SMAX) all SMAX loads are issued before the first add, so the
// sum costs one memory round trip: split indices past S - 1 are clamped (the
// repeated values are loaded but not added; adding +0.0 instead leaves the
// sum bitwise unchanged, since a sum started at +0.0 is never -0.0). SMAX = 0
// takes any S in groups of 8.
template <int SMAX>
__global__ __launch_bounds__(256) void gemv_q4_0_reduce_kernel(const float* __restrict__ part,
                                                               float* __restrict__ y, int MN,
                                                               int S) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  if constexpr (SMAX == 0) {
    y[i] = sum_strided(part + i, (size_t)MN, S);
  } else {
    __builtin_assume(S >= 1);
    float t[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) t[s] = part[(size_t)min(s, S - 1) * MN + i];
    float v = 0.0f;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) v += s < S ? t[s] : 0.0f;
    y[i] = v;
  }
}

template <int M, int LPB>
hipError_t launch_one(const GemvArgs& a, bool staged, hipStream_t st) {
  const int rf = 4 * phase_lds_floats<M, LPB>();
  int lds;
  if (staged) {
    const int sb = staged_lds_bytes<M, LPB, staged_rows_per_batch<M, LPB>(), kStagedJt,
                                    staged_buffers<M, LPB>()>(a.Kt);
    lds = sb > rf ? sb : rf;
    hipLaunchKernelGGL((gemv_q4_0_kernel<M, LPB, true>), dim3(a.C * a.S), dim3(kThreads), lds, st,
                       a);
  } else {
    const int xf = 4 * tile_x_floats<M>(a.Kt, a.P, rows_per_batch<M, LPB>());
    lds = xf > rf ? xf : rf;
    hipLaunchKernelGGL((gemv_q4_0_kernel<M, LPB, false>), dim3(a.C * a.S), dim3(kThreads), lds,
                       st, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.S == 1) return err;
  return launch_gemv_reduce(a.part, a.y, M * a.N, a.S, st);
}

template <int M>
hipError_t launch_m(const GemvArgs& a, int lpb, bool staged, hipStream_t st) {
  if constexpr (M == 1) {
    if (lpb == 1) return launch_one<1, 1>(a, staged, st);
  }
  return launch_one<M, 2>(a, staged, st);
}

}  // namespace

hipError_t launch_gemv_reduce(const float* part, float* y, int MN, int S, hipStream_t st) {
  const dim3 grid((MN + 255) / 256), block(256);
  if (S <= 8)
    hipLaunchKernelGGL(gemv_q4_0_reduce_kernel<8>, grid, block, 0, st, part, y, MN, S);
  else if (S <= 16)
    hipLaunchKernelGGL(gemv_q4_0_reduce_kernel<16>, grid, block, 0, st, part, y, MN, S);
  else if (S <= 32)
    hipLaunchKernelGGL(gemv_q4_0_reduce_kernel<32>, grid, block, 0, st, part, y, MN, S);
  else if (S <= 64)
    hipLaunchKernelGGL(gemv_q4_0_reduce_kernel<64>, grid, block, 0, st, part, y, MN, S);
  else
    hipLaunchKernelGGL(gemv_q4_0_reduce_kernel<0>, grid, block, 0, st, part, y, MN, S);
  return hipGetLastError();
}

namespace {

// Dynamic LDS bytes of a vector tile of Kt rows with P row phases (as
// launch_one sizes it); with 16-block tiles the larger of the staged and the
// per-lane variant, since the matrix alignment decides between them at launch.
template <int M, int LPB>
int vector_lds_bytes_t(int Kt, int P, bool wide) {
  const int rf = 4 * phase_lds_floats<M, LPB>();
  int m = 4 * tile_x_floats<M>(Kt, P, rows_per_batch<M, LPB>());
  if (wide) {
    const int sb = staged_lds_bytes<M, LPB, staged_rows_per_batch<M, LPB>(), kStagedJt,
                                    staged_buffers<M, LPB>()>(Kt);
    m = m > sb ? m : sb;
  }
  return m > rf ? m : rf;
}

int vector_lds_bytes(int M, int LPB, int Kt, int P, bool wide) {
  switch (M) {
    case 1:
      return LPB == 1 ? vector_lds_bytes_t<1, 1>(Kt, P, wide) : vector_lds_bytes_t<1, 2>(Kt, P, wide);
    case 2: return vector_lds_bytes_t<2, 2>(Kt, P, wide);
    case 3: return vector_lds_bytes_t<3, 2>(Kt, P, wide);
    case 4: return vector_lds_bytes_t<4, 2>(Kt, P, wide);
    case 5: return vector_lds_bytes_t<5, 2>(Kt, P, wide);
    case 6: return vector_lds_bytes_t<6, 2>(Kt, P, wide);
    case 7: return vector_lds_bytes_t<7, 2>(Kt, P, wide);
    default: return vector_lds_bytes_t<8, 2>(Kt, P, wide);
  }
}

}  // namespace

// Tile plan: 16-block column tiles; whole blocks per lane for a single row,
// half blocks for M >= 2 (half the accumulator registers, so more waves per
// SIMD: measured 4-10 % faster than whole blocks at M = 2..4). The K split S
// sets the grid size C*S. Measured on MI355X over the dense 7B shapes, the
// best grid is at most one full round of resident workgroups, up to 512 (two
// per CU), for every batch: at M = 1 a sweep of the cap over 256..1024 gave
// 11.85 us at 512 against 12.4 at 352 (4096 x 11008) and 12.5 against 13.3
// (11008 x 4096); a grid just past a round costs a whole second round. Tiles
// keep at least 128 rows (8 or 16 per lane), or their fixed cost dominates.
// S is the largest split within both.
GemvPlan plan_gemv(int M, int N, int K) {
  GemvPlan p{};
  if (plan_gemv_mfma(M, N, K, p)) return p;
  constexpr int kMinTileRows = 128;
  const int NB = N / kBlockWeights;
  p.LPB = (M == 1) ? 1 : 2;
  p.Jt = NB < 16 ? NB : 16;
  p.Lr = p.Jt * p.LPB;
  p.P = kThreads / p.Lr;
  p.C = (NB + p.Jt - 1) / p.Jt;
  auto kt_for = [&](int s) {
    const int kt = (K + s - 1) / s;
    return (kt + p.P - 1) / p.P * p.P;
  };
  constexpr int target = 512;
  int best_kt = kt_for(1);  // S = 1
  int last_S = -1;
  for (int s = 2; s <= K; ++s) {
    const int kt = kt_for(s);
    const int S = (K + kt - 1) / kt;
    if (S == last_S) continue;
    last_S = S;
    if (kt < kMinTileRows || p.C * S > target) break;
    best_kt = kt;
  }
  // The activation tile grows with the rows of a tile: split K further when
  // the tile would not fit in LDS (wide matrices, where the grid target alone
  // gives few splits), even past the grid target.
  const bool wide = p.Jt == kStagedJt;
  for (int s = (K + best_kt - 1) / best_kt;
       vector_lds_bytes(M, p.LPB, best_kt, p.P, wide) > kMaxLdsBytes; ++s)
    best_kt = kt_for(s);
  p.Kt = best_kt;
  p.S = (K + p.Kt - 1) / p.Kt;
  p.ws_bytes = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemv(const float* x, const uint8_t* B, float* y, int M, int N, int K, void* ws,
                       const GemvPlan& p, hipStream_t st) {
  GemvArgs a;
  a.x = x;
  a.B = B;
  a.y = y;
  a.part = static_cast<float*>(ws);
  a.M = M;
  a.N = N;
  a.K = K;
  a.NB = N / kBlockWeights;
  a.Jt = p.Jt;
  a.Lr = p.Lr;
  a.P = p.P;
  a.C = p.C;
  a.Kt = p.Kt;
  a.S = p.S;
  if (p.mfma) return launch_gemv_mfma(x, B, y, M, N, K, ws, p, st);
  // Wave-private staging needs 16-byte aligned 16-block row segments.
  const bool staged = p.Jt == kStagedJt && a.NB % 8 == 0 &&
                      (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  switch (M) {
    case 1: return launch_m<1>(a, p.LPB, staged, st);
    case 2: return launch_m<2>(a, p.LPB, staged, st);
    case 3: return launch_m<3>(a, p.LPB, staged, st);
    case 4: return launch_m<4>(a, p.LPB, staged, st);
    case 5: return launch_m<5>(a, p.LPB, staged, st);
    case 6: return launch_m<6>(a, p.LPB, staged, st);
    case 7: return launch_m<7>(a, p.LPB, staged, st);
    case 8: return launch_m<8>(a, p.LPB, staged, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4
