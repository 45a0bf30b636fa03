// Decode GEMV over Q4_0 weights: y[M x N] = x[M x K] . deq(B[K x N]), M <= 8.
//
// The fused dequantize-inside-the-inner-loop matmul of the "2000-line C++
// DeepSeek inference engine" article (§3.4 matmul_q4_0), re-designed for
// gfx950. B is row-major with blocks along N, so one output column's weights
// are spread over all K rows; the kernel therefore splits both N and K:
//
//   * a workgroup (256 lanes) owns a column tile of Jt blocks (32*Jt outputs)
//     and a K range of Kt rows; its lanes form P = 256 / (Jt*LPB) row phases,
//     and each lane owns one block column (LPB = 1) or half of one (LPB = 2),
//     walking rows k0+phase, k0+phase+P, ...;
//   * each lane reads its block share with one unaligned dwordx4/dwordx2 load
//     plus one 2-byte scale load; a row's shares are adjacent, so a wave's
//     loads cover contiguous 18*Jt-byte row segments;
//   * x for the K range is staged once in LDS (k-major, M values per k);
//   * nibbles are unpacked in registers (masked bytes, v_cvt_f32_ubyteN) and
//     accumulated with one fp32 FMA per weight and activation row;
//   * the row phases are reduced through LDS in a fixed order; split-K partials
//     go to the workspace and the last workgroup of each column tile (completion
//     ticket) sums them in split order and writes y. No floating-point atomics:
//     results are deterministic.
//
// The tile shape depends only on (N, K), never on M, so row m of y is bitwise
// the same whatever the batch it is computed in.
#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

struct GemvArgs {
  const float* __restrict__ x;
  const uint8_t* __restrict__ B;
  float* __restrict__ y;
  float* __restrict__ part;    // [C][S][M][Jt*32] split-K partials
  unsigned* __restrict__ cnt;  // [C] completion tickets
  int N, K, NB;
  int Jt, Kt, S, C, Lr, P;
};

template <int M, int LPB, int U>
__global__ __launch_bounds__(kThreads) void gemv_q4_0_kernel(GemvArgs a) {
  constexpr int XS = x_stride<M>();
  extern __shared__ float smem[];
  __shared__ unsigned last_flag;

  const int t = threadIdx.x;
  const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int c = L % a.C;
  const int s = L / a.C;
  const int k0 = s * a.Kt;
  const int rows = min(a.Kt, a.K - k0);
  const int j0 = c * a.Jt;

  // Stage x[:, k0:k0+rows] in LDS as smem[kk*XS + m] (k-major).
  for (int idx = t; idx < M * rows; idx += kThreads) {
    const int m = idx / rows;
    const int kk = idx - m * rows;
    smem[kk * XS + m] = a.x[(size_t)m * a.K + k0 + kk];
  }
  __syncthreads();

  float acc[M][32 / LPB];
  float corr[M];
  const TileGeom g{a.B, a.NB, j0, k0, rows, a.Lr, a.P};
  tile_accumulate<M, LPB, U>(g, smem, acc, corr);
  finish_part<M, LPB>(acc, corr);

  const int width = a.Jt * kBlockWeights;  // output columns of the tile
  const int ncols = min(width, (a.NB - j0) * kBlockWeights);
  float* __restrict__ ycol = a.y + (size_t)j0 * kBlockWeights;
  __syncthreads();  // the staged x is no longer needed
  if (a.S == 1) {
    reduce_phases<M, LPB>(acc, smem, a.Lr, a.P, ncols,
                          [&](int m, int o, float v) { ycol[(size_t)m * a.N + o] = v; });
    return;
  }
  float* __restrict__ my_part = a.part + ((size_t)c * a.S + s) * (size_t)M * width;
  reduce_phases<M, LPB>(acc, smem, a.Lr, a.P, ncols,
                        [&](int m, int o, float v) { my_part[(size_t)m * width + o] = v; });

  // Split-K: the last workgroup of this column tile sums the partials in
  // split order and writes y.
  if (!arrive_last(a.cnt + c, (unsigned)a.S, &last_flag)) return;
  const float* __restrict__ tile_part = a.part + (size_t)c * a.S * (size_t)M * width;
  for (int idx = t; idx < M * ncols; idx += kThreads) {
    const int m = idx / ncols;
    const int o = idx - m * ncols;
    float sum = 0.0f;
    for (int ss = 0; ss < a.S; ++ss) sum += tile_part[((size_t)ss * M + m) * width + o];
    ycol[(size_t)m * a.N + o] = sum;
  }
}

#ifndef Q4_GEMV_UNROLL
#define Q4_GEMV_UNROLL 4
#endif

template <int M>
hipError_t launch_m(const GemvArgs& a, int lpb, size_t lds, hipStream_t st) {
  const dim3 grid(a.C * a.S), block(kThreads);
  if (lpb == 1)
    hipLaunchKernelGGL((gemv_q4_0_kernel<M, 1, Q4_GEMV_UNROLL>), grid, block, lds, st, a);
  else
    hipLaunchKernelGGL((gemv_q4_0_kernel<M, 2, Q4_GEMV_UNROLL>), grid, block, lds, st, a);
  return hipGetLastError();
}

}  // namespace

// Tile plan. Only (N, K) decide it, so every batch size uses the same
// per-column summation order.
GemvPlan plan_gemv(int M, int N, int K) {
  GemvPlan p{};
  const int NB = N / kBlockWeights;
  p.LPB = 2;
  p.Jt = NB < 16 ? NB : 16;
  p.Lr = p.Jt * p.LPB;
  p.P = kThreads / p.Lr;
  p.C = (NB + p.Jt - 1) / p.Jt;
  // K split: aim at ~512 workgroups, at least 8 rows per lane, at most 1024
  // rows per workgroup (x staging <= 32 KB of LDS for M = 8).
  const int target_wg = 512;
  int S = (target_wg + p.C - 1) / p.C;
  const int s_max = (K + 8 * p.P - 1) / (8 * p.P);
  if (S > s_max) S = s_max;
  if (S < 1) S = 1;
  int Kt = (K + S - 1) / S;
  Kt = (Kt + p.P - 1) / p.P * p.P;
  if (Kt > 1024) Kt = 1024;
  p.Kt = Kt;
  p.S = (K + Kt - 1) / Kt;
  const size_t xs_floats = (size_t)p.Kt * 8;  // sized for the widest stride
  const size_t red_floats = (size_t)(32 / p.LPB) * kRedStride;
  p.lds_bytes = 4 * (xs_floats > red_floats ? xs_floats : red_floats);
  const size_t cnt_bytes = ((size_t)p.C * 4 + 255) / 256 * 256;
  p.part_offset = cnt_bytes;
  p.ws_bytes = p.S > 1 ? cnt_bytes + (size_t)p.C * p.S * M * p.Jt * kBlockWeights * 4 : 0;
  (void)M;
  return p;
}

hipError_t launch_gemv(const float* x, const uint8_t* B, float* y, int M, int N, int K,
                       void* ws, const GemvPlan& p, hipStream_t st) {
  GemvArgs a;
  a.x = x;
  a.B = B;
  a.y = y;
  a.cnt = static_cast<unsigned*>(ws);
  a.part = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.part_offset) : nullptr;
  a.N = N;
  a.K = K;
  a.NB = N / kBlockWeights;
  a.Jt = p.Jt;
  a.Kt = p.Kt;
  a.S = p.S;
  a.C = p.C;
  a.Lr = p.Lr;
  a.P = p.P;
  switch (M) {
    case 1: return launch_m<1>(a, p.LPB, p.lds_bytes, st);
    case 2: return launch_m<2>(a, p.LPB, p.lds_bytes, st);
    case 3: return launch_m<3>(a, p.LPB, p.lds_bytes, st);
    case 4: return launch_m<4>(a, p.LPB, p.lds_bytes, st);
    case 5: return launch_m<5>(a, p.LPB, p.lds_bytes, st);
    case 6: return launch_m<6>(a, p.LPB, p.lds_bytes, st);
    case 7: return launch_m<7>(a, p.LPB, p.lds_bytes, st);
    case 8: return launch_m<8>(a, p.LPB, p.lds_bytes, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4
