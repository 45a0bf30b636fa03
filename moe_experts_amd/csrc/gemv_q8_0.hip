// Decode GEMV over Q8_0 weights: y[M x N] = x[M x K] . deq(B[K x N]), M <= 8.
//
// The split-K vector tile of gemv_vector.hpp with the Q8_0 block format
// (Q8_0Format in q4_device.hpp: 34-byte blocks, signed bytes times the
// scale): the same tile walk, activation staging, phase sums, split-K plan
// and reduction as the Q4_0 path, so the format is the only difference.
#include "gemv_vector.hpp"
#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {

GemvPlan plan_gemv_q8(int M, int N, int K) { return plan_vector<Q8_0Format>(M, N, K); }

hipError_t launch_gemv_q8(const float* x, const uint8_t* B, float* y, int M, int N, int K,
                          void* ws, const GemvPlan& p, hipStream_t st) {
  return launch_vector<Q8_0Format>(x, B, y, M, N, K, ws, p, st);
}

}  // namespace q4
