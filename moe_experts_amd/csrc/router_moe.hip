// MoE router on the device: gate logits, top-k selection and softmax weights,
// with the shared-expert slots appended, so that a whole MoE layer runs on one
// stream without a host round trip.
//
// The KTransformers DeepSeek-V2 tutorial's YAML-injection section has the
// KDeepseekV2MoE forward run the gate first for each token's top-k expert ids
// and weights; "Optimization 3" keeps the shared experts, used by every token,
// on the GPU. The gate is a plain linear map (x . Wr^T, fp32) followed by the
// top-k choice and the softmax over the chosen logits.
//
//   1. router_logits_kernel: workgroup (g, s) owns experts 16g .. 16g+15 and
//      the K chunk [256 s, 256 s + 256). It stages that chunk of its 16 router
//      rows and of every token's activations in LDS (all loads in flight at
//      once); a wave takes 4 experts, its lanes the tokens (one token per
//      lane), and reads the 4 rows as LDS broadcasts. A single token instead
//      spreads the chunk's k over the lanes (below). Each lane forms its 4
//      dot products over the chunk in k order and writes them as K-split
//      partials, part[t][e][s]; the split
//      count is padded to a multiple of 4 by chunks past H, which write zeros.
//   2. router_topk_kernel: one workgroup per token. A thread per expert sums
//      its partials in split order (contiguous, four per load) into the logit,
//      also written out; then one wave picks the top-k with k rounds of a
//      wave-wide arg-max (larger logit first, then lower index; NaN never
//      chosen) and forms the softmax weights in fp32 (maximum subtracted,
//      terms summed in slot order).
#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int kRouterKc = 256;                      // k values per chunk: one float4 per lane
constexpr int kRouterEW = 4;                        // experts per wave
constexpr int kRouterWaves = 4;
constexpr int kRouterEG = kRouterEW * kRouterWaves; // experts per workgroup
constexpr int kRouterPitch = kRouterKc / 4 + 1;     // float4 per staged row: one pad spreads
                                                    // the lanes' rows over the LDS banks
constexpr int kTopkPer = Q4_MOE_MAX_E / kWaveSize;  // logits per lane in the top-k wave
static_assert(Q4_MOE_MAX_T <= kWaveSize, "one lane per token");

__global__ __launch_bounds__(kRouterWaves * kWaveSize) void router_logits_kernel(
    const float* __restrict__ x, const float* __restrict__ Wr, float* __restrict__ part, int T,
    int H, int E) {
  extern __shared__ float4 lds[];
  float4* ws = lds;                          // [kRouterEG][kRouterKc / 4] router rows
  float4* xs = lds + kRouterEG * (kRouterKc / 4);  // [T][kRouterPitch] activations
  const int g = blockIdx.x;
  const int s = blockIdx.y;
  const int Sp = gridDim.y;
  const int k0 = s * kRouterKc;
  const int n4 = max(0, min(kRouterKc, H - k0) / 4);  // float4 of this chunk (H % 4 == 0)
  constexpr int kThr = kRouterWaves * kWaveSize;
  if (T == 1) {
    // A single token: lane c takes float4 c of the chunk for each of the
    // wave's 4 experts (16-byte loads straight from memory, no staging) and the
    // wave adds the 64 lane sums with a fixed butterfly (every lane ends with
    // the same value), instead of one lane running all 256 FMAs. A single
    // token's logits therefore match its batched ones to rounding, not
    // bitwise, as for the single-token expert tiles. No barrier on this path.
    const int lane = threadIdx.x % kWaveSize;
    const int e0 = g * kRouterEG + (threadIdx.x / kWaveSize) * kRouterEW;
    if (e0 >= E) return;
    const bool in = lane < n4;
    const float4 xv = in ? *reinterpret_cast<const float4*>(x + k0 + 4 * lane)
                         : float4{0.0f, 0.0f, 0.0f, 0.0f};
    float4 rv[kRouterEW];
#pragma unroll
    for (int j = 0; j < kRouterEW; ++j)
      rv[j] = (in && e0 + j < E)
                  ? *reinterpret_cast<const float4*>(Wr + (size_t)(e0 + j) * H + k0 + 4 * lane)
                  : float4{0.0f, 0.0f, 0.0f, 0.0f};
    float acc[kRouterEW];
#pragma unroll
    for (int j = 0; j < kRouterEW; ++j) {
      float a = xv.x * rv[j].x;
      a = __builtin_fmaf(xv.y, rv[j].y, a);
      a = __builtin_fmaf(xv.z, rv[j].z, a);
      a = __builtin_fmaf(xv.w, rv[j].w, a);
#pragma unroll
      for (int off = kWaveSize / 2; off > 0; off >>= 1) a += __shfl_xor(a, off);
      acc[j] = a;
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < kRouterEW; ++j)
        if (e0 + j < E) part[(size_t)(e0 + j) * Sp + s] = acc[j];
    }
    return;
  }
  // one round trip: the chunk of the workgroup's router rows and of every
  // token's activations (zeros past the chunk or past E)
  for (int i = threadIdx.x; i < kRouterEG * (kRouterKc / 4); i += kThr) {
    const int r = i / (kRouterKc / 4);
    const int c = i - r * (kRouterKc / 4);
    const int e = g * kRouterEG + r;
    ws[i] = (c < n4 && e < E) ? *reinterpret_cast<const float4*>(Wr + (size_t)e * H + k0 + 4 * c)
                              : float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  for (int i = threadIdx.x; i < T * (kRouterKc / 4); i += kThr) {
    const int t = i / (kRouterKc / 4);
    const int c = i - t * (kRouterKc / 4);
    xs[t * kRouterPitch + c] = c < n4
        ? *reinterpret_cast<const float4*>(x + (size_t)t * H + k0 + 4 * c)
        : float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  __syncthreads();
  const int lane = threadIdx.x % kWaveSize;
  const int r0 = (threadIdx.x / kWaveSize) * kRouterEW;  // this wave's first row
  const int e0 = g * kRouterEG + r0;
  if (e0 >= E) return;
  const float4* xr = xs + min(lane, T - 1) * kRouterPitch;
  const float4* wr = ws + r0 * (kRouterKc / 4);
  float acc[kRouterEW] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int c = 0; c < n4; ++c) {
    const float4 v = xr[c];
#pragma unroll
    for (int j = 0; j < kRouterEW; ++j) {
      const float4 r = wr[j * (kRouterKc / 4) + c];  // same address in every lane
      acc[j] = __builtin_fmaf(v.x, r.x, acc[j]);
      acc[j] = __builtin_fmaf(v.y, r.y, acc[j]);
      acc[j] = __builtin_fmaf(v.z, r.z, acc[j]);
      acc[j] = __builtin_fmaf(v.w, r.w, acc[j]);
    }
  }
  if (lane < T) {
    float* dst = part + ((size_t)lane * E + e0) * Sp + s;
#pragma unroll
    for (int j = 0; j < kRouterEW; ++j)
      if (e0 + j < E) dst[(size_t)j * Sp] = acc[j];
  }
}

// (v, i) beats (w, k): a chosen candidate (index >= 0) beats none; then the
// larger logit; equal logits go to the lower index.
__device__ __forceinline__ bool beats(float v, int i, float w, int k) {
  return i >= 0 && (k < 0 || v > w || (v == w && i < k));
}

constexpr int kTopkThreads = 256;

__global__ __launch_bounds__(kTopkThreads) void router_topk_kernel(
    const float* __restrict__ part, float* __restrict__ logits, int32_t* __restrict__ ids,
    float* __restrict__ wts, int E, int Sp, int topk, int n_shared) {
  __shared__ float s_l[Q4_MOE_MAX_E];
  const int t = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kTopkThreads) {
    const float4* p = reinterpret_cast<const float4*>(part + ((size_t)t * E + e) * Sp);
    float l = 0.0f;
#pragma unroll 16
    for (int c = 0; c < Sp / 4; ++c) {
      const float4 q = p[c];
      l += q.x;
      l += q.y;
      l += q.z;
      l += q.w;
    }
    logits[(size_t)t * E + e] = l;
    s_l[e] = l;
  }
  __syncthreads();
  if (threadIdx.x >= kWaveSize) return;
  const int lane = threadIdx.x;
  float v[kTopkPer];
#pragma unroll
  for (int i = 0; i < kTopkPer; ++i) {
    const int e = lane + kWaveSize * i;
    v[i] = e < E ? s_l[e] : __builtin_nanf("");  // no expert: never chosen
  }
  unsigned taken = 0;
  float sv[Q4_MOE_MAX_TOPK];
  int si[Q4_MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < Q4_MOE_MAX_TOPK; ++j) {
    sv[j] = 0.0f;
    si[j] = -1;
    if (j >= topk) continue;
    // this lane's best remaining logit (its indices rise with i, so a strict
    // comparison keeps the lower index on ties), then the wave's
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < kTopkPer; ++i)
      if (!((taken >> i) & 1u) && !__builtin_isnan(v[i]) &&
          beats(v[i], lane + kWaveSize * i, bv, bi)) {
        bv = v[i];
        bi = lane + kWaveSize * i;
      }
#pragma unroll
    for (int off = kWaveSize / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    sv[j] = bv;
    si[j] = bi;
    if (bi >= 0 && bi % kWaveSize == lane) taken |= 1u << (bi / kWaveSize);
  }
  // softmax over the chosen logits (the first is their maximum)
  float ex[Q4_MOE_MAX_TOPK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < Q4_MOE_MAX_TOPK; ++j) {
    ex[j] = si[j] >= 0 ? expf(sv[j] - sv[0]) : 0.0f;
    sum += ex[j];
  }
  const int slots = topk + n_shared;
  if (lane < slots) {
    int id = E + (lane - topk);  // shared-expert slot
    float wt = 1.0f;
#pragma unroll
    for (int j = 0; j < Q4_MOE_MAX_TOPK; ++j)
      if (j == lane && j < topk) {
        id = si[j];
        wt = si[j] >= 0 ? ex[j] / sum : 0.0f;
      }
    ids[(size_t)t * slots + lane] = id;
    wts[(size_t)t * slots + lane] = wt;
  }
}

// K splits, padded to a multiple of 4 (the padding chunks contribute zeros)
int router_splits(int H) { return ((H + kRouterKc - 1) / kRouterKc + 3) / 4 * 4; }

}  // namespace

size_t router_ws_bytes(int T, int H, int E) {
  return (size_t)router_splits(H) * T * E * sizeof(float);
}

hipError_t launch_router(const float* x, const float* Wr, float* logits, int32_t* ids, float* w,
                         int T, int H, int E, int topk, int n_shared, void* ws,
                         hipStream_t st) {
  float* part = static_cast<float*>(ws);
  const int Sp = router_splits(H);
  const dim3 grid((E + kRouterEG - 1) / kRouterEG, Sp);
  const size_t lds = ((size_t)kRouterEG * (kRouterKc / 4) + (size_t)T * kRouterPitch) *
                     sizeof(float4);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(kRouterWaves * kWaveSize), lds, st, x, Wr,
                     part, T, H, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(router_topk_kernel, dim3(T), dim3(kTopkThreads), 0, st, part, logits, ids, w,
                     E, Sp, topk, n_shared);
  return hipGetLastError();
}

}  // namespace q4
