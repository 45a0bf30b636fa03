// Device helpers shared by the routing kernels (moe_q4_0.hip, moe_prefill.hip):
// a workgroup-wide prefix sum and an exact match of expert ids within a wave.
#pragma once

#include "q4_device.hpp"

namespace q4 {

// Bits of an expert id (ids are below Q4_MOE_MAX_E).
constexpr int kIdBits = 10;
static_assert((1 << kIdBits) >= Q4_MOE_MAX_E, "expert ids fit the ballot match");

// Inclusive prefix sum over one value per lane of the whole workgroup
// (wsum: one int per wave in LDS). Contains two workgroup barriers.
__device__ __forceinline__ int block_inclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x / kWaveSize;
#pragma unroll
  for (int o = 1; o < kWaveSize; o <<= 1) {
    const int n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == kWaveSize - 1) wsum[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += wsum[w];
  __syncthreads();
  return v + add;
}

// The lanes of this wave holding the same valid expert id as this lane (one
// ballot per id bit; lanes with valid == false match nothing). Every lane of
// the wave must call it.
__device__ __forceinline__ uint64_t same_id_lanes(int e, bool valid) {
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t set = __ballot(bit);
    same &= bit ? set : ~set;
  }
  return same;
}

}  // namespace q4
