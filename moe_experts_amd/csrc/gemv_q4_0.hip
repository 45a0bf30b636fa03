// Decode GEMV over Q4_0 weights (y[M x N] = x[M x K] . deq(B[K x N]), M <= 8)
// and the split-K sum shared by every decode GEMV.
//
// Batches of 1..2 rows (and shapes the matrix-core tile does not take) run the
// split-K vector tile of gemv_vector.hpp with the Q4_0 block format; batches
// of 3..8 run the matrix-core tile (gemv_mfma_q4_0.hip). Both write split-K
// partial sums that gemv_reduce_kernel adds up in split order.
#include <cstdlib>

#include "gemv_vector.hpp"
#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

// y[i] = part[0][i] + part[1][i] + ... + part[S-1][i], in split order. With
// SMAX > 0 (S <= SMAX) all SMAX loads are issued before the first add, so the
// sum costs one memory round trip: split indices past S - 1 are clamped (the
// repeated values are loaded but not added; adding +0.0 instead leaves the
// sum bitwise unchanged, since a sum started at +0.0 is never -0.0). SMAX = 0
// takes any S in groups of 8.
template <int SMAX>
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ part,
                                                          float* __restrict__ y, int MN, int S) {
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

}  // namespace

hipError_t launch_gemv_reduce(const float* part, float* y, int MN, int S, hipStream_t st) {
  const dim3 grid((MN + 255) / 256), block(256);
  if (S <= 8)
    hipLaunchKernelGGL(gemv_reduce_kernel<8>, grid, block, 0, st, part, y, MN, S);
  else if (S <= 16)
    hipLaunchKernelGGL(gemv_reduce_kernel<16>, grid, block, 0, st, part, y, MN, S);
  else if (S <= 32)
    hipLaunchKernelGGL(gemv_reduce_kernel<32>, grid, block, 0, st, part, y, MN, S);
  else if (S <= 64)
    hipLaunchKernelGGL(gemv_reduce_kernel<64>, grid, block, 0, st, part, y, MN, S);
  else
    hipLaunchKernelGGL(gemv_reduce_kernel<0>, grid, block, 0, st, part, y, MN, S);
  return hipGetLastError();
}

GemvPlan plan_gemv(int M, int N, int K) {
  GemvPlan p{};
  if (plan_gemv_mfma(M, N, K, p)) return p;
  return plan_vector<Q4_0Format>(M, N, K);
}

hipError_t launch_gemv(const float* x, const uint8_t* B, float* y, int M, int N, int K, void* ws,
                       const GemvPlan& p, hipStream_t st) {
  if (p.mfma) return launch_gemv_mfma(x, B, y, M, N, K, ws, p, st);
  return launch_vector<Q4_0Format>(x, B, y, M, N, K, ws, p, st);
}

}  // namespace q4
