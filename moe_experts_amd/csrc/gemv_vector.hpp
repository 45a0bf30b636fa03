// Split-K vector GEMV over a block format: y[M x N] = x[M x K] . deq(B[K x N]),
// M <= 8, for any format of q4_device.hpp (Q4_0Format, Q8_0Format).
//
// The fused dequantize-inside-the-inner-loop matmul of the "2000-line C++
// DeepSeek inference engine" article (§3.4 matmul_q4_0), re-designed for
// gfx950. B is row-major with blocks along N, so a column's weights are spread
// over all K rows while each 128-byte cache line holds several consecutive
// blocks of one row. To keep memory requests full, a workgroup reads whole
// row segments of Jt blocks, and to still have hundreds of workgroups on a
// 4096-row matrix it owns only a K range of those columns (split-K):
//
//   1. gemv_vector_kernel: workgroup (c, s) owns block columns Jt*c ..
//      Jt*c+Jt-1 and rows [s*Kt, (s+1)*Kt). Its lanes form row phases of
//      Jt*LPB lanes; each lane loads every one of its rows (its block share
//      plus the 2-byte scale, and the activations) before using any, unpacks
//      the values in registers and accumulates one fp32 FMA per weight and
//      activation row (Fmt::accumulate). The row phases are summed through
//      LDS in a fixed order and finished by the format (Fmt::finish); the
//      workgroup writes its partial sums to the workspace (or y directly when
//      K is not split).
//   2. the split-K reduce kernel (launch_gemv_reduce): y[m][n] = sum over the
//      K splits, in split order.
// Cross-workgroup hand-off at agent scope costs an L2 write-back per workgroup
// on this GPU, so the split-K sum is a second kernel instead: no atomics, no
// fences, deterministic results.
//
// Q4_0 matrices whose 16-block row segments are 16-byte aligned take a
// variant that stages the weights in LDS with LDS-DMA copies
// (tile_accumulate_staged); the plan sizes LDS for either variant.
#pragma once

#include <type_traits>

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

// The LDS-staged weight path reads Q4_0 blocks out of 16-block segments.
constexpr int kStagedJt = 16;
template <class Fmt>
constexpr bool stages_in_lds() {
  return std::is_same<Fmt, Q4_0Format>::value;
}
// Rows per lane in one batch of the staged path, and weight buffers per wave.
template <int LPB>
constexpr int staged_rows_per_batch() {
  return LPB == 1 ? 4 : 8;
}
constexpr int kStagedBuffers = 2;

template <class Fmt, int M, int LPB, bool STAGED>
__global__ __launch_bounds__(kThreads) void gemv_vector_kernel(GemvArgs a) {
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
  if constexpr (STAGED) {
    static_assert(stages_in_lds<Fmt>(), "the staged path reads Q4_0 blocks");
    tile_accumulate_staged<M, LPB, staged_rows_per_batch<LPB>(), kStagedJt, kStagedBuffers>(
        g, a.x, (uint32_t)(4 * M * a.K), xoff, reinterpret_cast<uint8_t*>(smem), acc, corr);
  } else {
    tile_accumulate<M, LPB, Fmt::rows_per_batch(M), Fmt>(g, a.x, (uint32_t)(4 * M * a.K), xoff,
                                                         smem, acc, corr);
  }
  const int n0 = g.j0 * kBlockWeights;
  const int ncols = min(a.Jt, a.NB - g.j0) * kBlockWeights;
  float* dst = (a.S == 1) ? a.y : a.part + (size_t)s * M * a.N;
  reduce_phases<M, LPB, Fmt>(acc, corr, smem, a.Lr, a.P, ncols,
                             [&](int m, int o, float v) { dst[(size_t)m * a.N + n0 + o] = v; });
}

// Dynamic LDS bytes of a tile of Kt rows with P row phases: the activation
// tile or the phase sums, whichever is larger; for staged-capable tiles the
// larger of the staged and the register variant, since the matrix alignment
// decides between them at launch.
template <class Fmt, int M>
int vector_lds_bytes_t(int Kt, int P, bool staged_possible) {
  constexpr int LPB = Fmt::lanes_per_block(M);
  const int rf = 4 * phase_lds_floats<M, LPB, Fmt>();
  int m = 4 * tile_x_floats<M>(Kt, P, Fmt::rows_per_batch(M));
  if constexpr (stages_in_lds<Fmt>()) {
    if (staged_possible) {
      const int sb = staged_lds_bytes<M, LPB, staged_rows_per_batch<LPB>(), kStagedJt,
                                      kStagedBuffers>(Kt);
      m = m > sb ? m : sb;
    }
  }
  return m > rf ? m : rf;
}

template <class Fmt>
int vector_lds_bytes(int M, int Kt, int P, bool staged_possible) {
  switch (M) {
    case 1: return vector_lds_bytes_t<Fmt, 1>(Kt, P, staged_possible);
    case 2: return vector_lds_bytes_t<Fmt, 2>(Kt, P, staged_possible);
    case 3: return vector_lds_bytes_t<Fmt, 3>(Kt, P, staged_possible);
    case 4: return vector_lds_bytes_t<Fmt, 4>(Kt, P, staged_possible);
    case 5: return vector_lds_bytes_t<Fmt, 5>(Kt, P, staged_possible);
    case 6: return vector_lds_bytes_t<Fmt, 6>(Kt, P, staged_possible);
    case 7: return vector_lds_bytes_t<Fmt, 7>(Kt, P, staged_possible);
    default: return vector_lds_bytes_t<Fmt, 8>(Kt, P, staged_possible);
  }
}

// Tile plan: column tiles of Fmt::kJt blocks (all of them when the matrix is
// narrower), Fmt::lanes_per_block(M) lanes per block. The K split S sets the
// grid size C*S. Measured on MI355X over the dense 7B shapes, the best grid
// is at most one full round of resident workgroups, up to 512 (two per CU):
// for Q4_0 at M = 1 a sweep of the cap over 256..1024 gave 11.85 us at 512
// against 12.4 at 352 (4096 x 11008) and 12.5 against 13.3 (11008 x 4096); a
// grid just past a round costs a whole second round. Raising the cap to 768,
// 1024 or 2048 with 32- or 64-row tiles made every M = 1 call slower
// (10.0 -> 10.8-16.7 us at 4096 x 4096): the per-workgroup fixed cost
// (activation tile, phase sums, partial stores) grows with the grid. Tiles
// keep at least 128 rows. S is the largest split within both, then raised
// further if the activation tile would not fit in LDS (wide matrices, where
// the grid target alone gives few splits).
template <class Fmt>
GemvPlan plan_vector(int M, int N, int K) {
  GemvPlan p{};
  constexpr int kMinTileRows = 128;
  const int NB = N / kBlockWeights;
  p.LPB = Fmt::lanes_per_block(M);
  p.Jt = NB < Fmt::kJt ? NB : Fmt::kJt;
  p.Lr = p.Jt * p.LPB;
  p.P = kThreads / p.Lr;
  p.C = (NB + p.Jt - 1) / p.Jt;
  auto kt_for = [&](int s) {
    const int kt = (K + s - 1) / s;
    return (kt + p.P - 1) / p.P * p.P;
  };
  const int target = Fmt::grid_target(M);
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
  const bool staged_possible = stages_in_lds<Fmt>() && p.Jt == kStagedJt;
  for (int s = (K + best_kt - 1) / best_kt;
       vector_lds_bytes<Fmt>(M, best_kt, p.P, staged_possible) > kMaxLdsBytes; ++s)
    best_kt = kt_for(s);
  p.Kt = best_kt;
  p.S = (K + p.Kt - 1) / p.Kt;
  p.ws_bytes = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
  return p;
}

template <class Fmt, int M>
hipError_t launch_vector_m(const GemvArgs& a, bool staged, hipStream_t st) {
  constexpr int LPB = Fmt::lanes_per_block(M);
  const int rf = 4 * phase_lds_floats<M, LPB, Fmt>();
  int lds;
  bool use_staged = false;
  if constexpr (stages_in_lds<Fmt>()) use_staged = staged;
  if (use_staged) {
    if constexpr (stages_in_lds<Fmt>()) {
      const int sb =
          staged_lds_bytes<M, LPB, staged_rows_per_batch<LPB>(), kStagedJt, kStagedBuffers>(a.Kt);
      lds = sb > rf ? sb : rf;
      hipLaunchKernelGGL((gemv_vector_kernel<Fmt, M, LPB, true>), dim3(a.C * a.S),
                         dim3(kThreads), lds, st, a);
    }
  } else {
    const int xf = 4 * tile_x_floats<M>(a.Kt, a.P, Fmt::rows_per_batch(M));
    lds = xf > rf ? xf : rf;
    hipLaunchKernelGGL((gemv_vector_kernel<Fmt, M, LPB, false>), dim3(a.C * a.S), dim3(kThreads),
                       lds, st, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.S == 1) return err;
  return launch_gemv_reduce(a.part, a.y, M * a.N, a.S, st);
}

// Launch a plan of plan_vector<Fmt> (main kernel, then the split-K sum).
template <class Fmt>
hipError_t launch_vector(const float* x, const uint8_t* B, float* y, int M, int N, int K, void* ws,
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
  // Wave-private staging needs 16-byte aligned 16-block row segments.
  const bool staged = stages_in_lds<Fmt>() && p.Jt == kStagedJt && a.NB % 8 == 0 &&
                      (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  switch (M) {
    case 1: return launch_vector_m<Fmt, 1>(a, staged, st);
    case 2: return launch_vector_m<Fmt, 2>(a, staged, st);
    case 3: return launch_vector_m<Fmt, 3>(a, staged, st);
    case 4: return launch_vector_m<Fmt, 4>(a, staged, st);
    case 5: return launch_vector_m<Fmt, 5>(a, staged, st);
    case 6: return launch_vector_m<Fmt, 6>(a, staged, st);
    case 7: return launch_vector_m<Fmt, 7>(a, staged, st);
    case 8: return launch_vector_m<Fmt, 8>(a, staged, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace q4
