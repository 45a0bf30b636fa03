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
// sum bitwise unchanged, since a sum started at +0.0 is never -0.0). The
// partials are read once, with non-temporal loads. SMAX = 0 takes any S in
// groups of 8. Workgroups of one wave spread the few outputs of a decode call
// over more CUs (same-box A/B against 256 lanes: 0.2-0.3 us per call).
constexpr int kReduceThreads = 64;
constexpr int kNonTemporal = 2;  // buffer-load cache policy: nt

template <int SMAX>
__global__ __launch_bounds__(kReduceThreads) void gemv_reduce_kernel(const float* __restrict__ part,
                                                                     float* __restrict__ y,
                                                                     int MN, int S) {
  const int i = blockIdx.x * kReduceThreads + threadIdx.x;
  if (i >= MN) return;
  if constexpr (SMAX == 0) {
    y[i] = sum_strided(part + i, (size_t)MN, S);
  } else {
    __builtin_assume(S >= 1);
    // S * MN floats of partials are below 2^30 (the plans keep tiles of at
    // least 64 rows and the matrix below 2 GiB), so byte offsets fit 32 bits.
    const __amdgpu_buffer_rsrc_t r = make_rsrc(part, (uint32_t)((size_t)S * MN * 4u));
    float t[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      t[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           r, (uint32_t)(min(s, S - 1) * MN + i) * 4u, 0,
                                           kNonTemporal));
    float v = 0.0f;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) v += s < S ? t[s] : 0.0f;
    y[i] = v;
  }
}

}  // namespace

hipError_t launch_gemv_reduce(const float* part, float* y, int MN, int S, hipStream_t st) {
  const dim3 grid((MN + kReduceThreads - 1) / kReduceThreads), block(kReduceThreads);
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
