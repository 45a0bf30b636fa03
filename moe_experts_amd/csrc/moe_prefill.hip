// Routed-expert MoE at prefill: many tokens per expert, so each expert's
// gate, up and down products are GEMMs on the fp16 matrix cores.
//
// The KTransformers DeepSeek-V2 tutorial runs the prefill-stage experts on the
// GPU as batched matmuls (its injection rules give the experts separate
// prefill and generate operators, "KExpertsTorch" for prefill) and the dense
// prefill GEMMs on tensor cores ("Optimization 2", Marlin); this path combines
// the two: the decode path's expert grouping with the prefill GEMM's tiles.
//
//   1. moe_prefill_route_kernel (one workgroup): a stable counting sort of
//      the (token, slot) pairs by expert, each wave over its own run of pairs. Sorted row q holds pair perm[q]; the
//      kernel writes, per sorted row, the token it reads (src[q]), per pair its
//      sorted row (pos[p], -1 for an id outside [0, E)), and the list of
//      96-row m-tiles (expert, first row, rows) of every expert's rows.
//   2. gate and up together: the prefill GEMM kernel in its grouped mode
//      with two matrices (X rows gathered by src, the expert's gate and up
//      Q4_0 matrices against the same X tile); its epilogue writes
//      h = fp16(SiLU(gate) * up) in sorted order.
//   3. down: the grouped GEMM on h (rows in sorted order, no gather) -> D.
//   4. moe_prefill_combine_kernel: out[t] = sum over slots 0..topk-1 of
//      w[t][s] * D[pos[t * topk + s]] (slot order; invalid slots skipped).
// Precision: x is given in fp16 and h is rounded to fp16 for the down GEMM;
// each dequantized weight is rounded to fp16 (the prefill GEMM's rule); all
// sums are fp32.
#include "q4_device.hpp"
#include "q4_internal.hpp"
#include "q4_route.hpp"

namespace q4 {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWaveSize;
constexpr int kIdRun = 16;  // 64-pair groups whose ids a wave loads at once
static_assert(Q4_MOE_MAX_E <= kRouteThreads, "one lane per expert");

struct PrefillRoute {
  const int32_t* ids;
  int npairs, E, topk;
  int32_t* src;   // [npairs] token of sorted row q
  int32_t* pos;   // [npairs] sorted row of pair p (-1: invalid id)
  int4* tiles;    // [max_tiles] (expert, first row, rows, 0)
  int* counts;    // [2]: m-tiles, valid rows
};

// LDS of the route kernel: per-wave counts (later bases) [waves][E], then one
// int per wave for the scans.
size_t route_lds_bytes(int E) { return ((size_t)kRouteWaves * E + kRouteWaves) * sizeof(int); }

// Wave w owns a contiguous run of 64-pair groups and walks it twice, in pair
// order. Pass 1 counts its pairs per expert (LDS atomic adds into the wave's
// own row). Between the passes, lane e sums expert e's counts, the workgroup
// scans them into each expert's first sorted row and its m-tiles, and lane e
// turns its per-wave counts into per-wave first rows (waves in order). Pass 2
// gives each pair its sorted row: its wave's current row for the expert plus
// its rank among the group's lanes with that id (they find each other with
// one ballot per id bit); the group's lowest such lane then moves the row on.
// Pair order is kept within every expert (a stable sort), with two workgroup
// barriers around the scan instead of barriers per group. The whole sort runs
// on one CU: the second pass's id match (about 60 vector instructions per
// group) is most of its time.
__global__ __launch_bounds__(kRouteThreads) void moe_prefill_route_kernel(PrefillRoute a) {
  extern __shared__ int route_lds[];
  int* s_wc = route_lds;                         // [kRouteWaves][E]
  int* s_wsum = route_lds + kRouteWaves * a.E;   // [kRouteWaves]
  const int t = threadIdx.x;
  const int lane = t & (kWaveSize - 1);
  const int wave = t / kWaveSize;
  const uint64_t below = (1ull << lane) - 1;
  const int groups = (a.npairs + kWaveSize - 1) / kWaveSize;
  const int per_wave = (groups + kRouteWaves - 1) / kRouteWaves;
  const int g0 = wave * per_wave;
  const int g1 = min(groups, g0 + per_wave);
  int* wc = s_wc + wave * a.E;  // this wave's row: only this wave touches it in the passes
  for (int e = lane; e < a.E; e += kWaveSize) wc[e] = 0;

  // The ids of kIdRun groups are loaded at once (one memory round trip per
  // run instead of one per group), then the groups are taken in order.
  int ev[kIdRun];
  auto load_run = [&](int gr) {
#pragma unroll
    for (int u = 0; u < kIdRun; ++u) {
      const int p = (gr + u) * kWaveSize + lane;
      ev[u] = (gr + u < g1 && p < a.npairs) ? a.ids[p] : -1;
    }
  };
  // pass 1: counts per expert
  for (int gr = g0; gr < g1; gr += kIdRun) {
    load_run(gr);
    // fully unrolled (a guard, not a break): the ids stay in registers with
    // static indices and the waits count only their loads
#pragma unroll
    for (int u = 0; u < kIdRun; ++u) {
      if (gr + u < g1) {  // uniform
        const int e = ev[u];
        if (e >= 0 && e < a.E) atomicAdd(&wc[e], 1);  // counts only: no ranks needed
      }
    }
  }
  __syncthreads();

  // expert t: total rows, first sorted row, m-tiles of kGemmRows rows
  int cnt = 0;
  if (t < a.E)
    for (int w = 0; w < kRouteWaves; ++w) cnt += s_wc[w * a.E + t];
  const int nt = (cnt + kGemmRows - 1) / kGemmRows;
  const int off = block_inclusive_scan(cnt, s_wsum) - cnt;
  const int toff = block_inclusive_scan(nt, s_wsum) - nt;
  for (int i = 0; i < nt; ++i)
    a.tiles[toff + i] = make_int4(t, off + kGemmRows * i, min(kGemmRows, cnt - kGemmRows * i), 0);
  if (t == kRouteThreads - 1) {
    a.counts[0] = toff + nt;
    a.counts[1] = off + cnt;
  }
  if (t < a.E) {
    int row = off;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = s_wc[w * a.E + t];
      s_wc[w * a.E + t] = row;
      row += c;
    }
  }
  __syncthreads();

  // pass 2: sorted rows
  for (int gr = g0; gr < g1; gr += kIdRun) {
    load_run(gr);
#pragma unroll
    for (int u = 0; u < kIdRun; ++u) {
      if (gr + u < g1) {  // uniform
        const int e = ev[u];
        const int p = (gr + u) * kWaveSize + lane;
        const bool valid = e >= 0 && e < a.E;
        const uint64_t same = same_id_lanes(e, valid);
        int q = -1;
        if (valid) {
          const int row = wc[e];  // read by every lane of the id before its lowest lane moves it
          q = row + __popcll(same & below);
          if ((same & below) == 0) wc[e] = row + __popcll(same);
          a.src[q] = p / a.topk;
        }
        if (p < a.npairs) a.pos[p] = q;
      }
    }
  }
}

// Four consecutive outputs per thread (16-byte loads and stores; H % 4 == 0,
// rows and out 16-byte aligned); every slot's sorted row and weight, then
// every slot's four values, are loaded before the sum.
__global__ __launch_bounds__(256) void moe_prefill_combine_kernel(
    const float* __restrict__ D, const int32_t* __restrict__ pos, const float* __restrict__ w,
    float* __restrict__ out, int T, int H, int topk) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
  const int H4 = H / 4;
  if (i4 >= (size_t)T * H4) return;
  const int t = (int)(i4 / H4);
  const int n4 = (int)(i4 - (size_t)t * H4);
  int q[Q4_MOE_MAX_TOPK];
  float wv[Q4_MOE_MAX_TOPK];
#pragma unroll
  for (int s = 0; s < Q4_MOE_MAX_TOPK; ++s) {
    const int p = t * topk + min(s, topk - 1);
    q[s] = pos[p];
    wv[s] = w[p];
  }
  float4 d[Q4_MOE_MAX_TOPK];
#pragma unroll
  for (int s = 0; s < Q4_MOE_MAX_TOPK; ++s)
    d[s] = (s < topk && q[s] >= 0)
               ? reinterpret_cast<const float4*>(D + (size_t)q[s] * H)[n4]
               : float4{0.0f, 0.0f, 0.0f, 0.0f};
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < Q4_MOE_MAX_TOPK; ++s)
    if (s < topk && q[s] >= 0) {
      acc.x = __builtin_fmaf(wv[s], d[s].x, acc.x);
      acc.y = __builtin_fmaf(wv[s], d[s].y, acc.y);
      acc.z = __builtin_fmaf(wv[s], d[s].z, acc.z);
      acc.w = __builtin_fmaf(wv[s], d[s].w, acc.w);
    }
  reinterpret_cast<float4*>(out)[i4] = acc;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

MoePrefillPlan plan_moe_prefill(int T, int H, int I, int E, int topk) {
  MoePrefillPlan p{};
  const size_t np = (size_t)T * topk;
  p.max_tiles = (int)((np + kGemmRows - 1) / kGemmRows + (np < (size_t)E ? np : (size_t)E));
  size_t off = 0;
  p.off_src = off;
  off += align256(np * 4);
  p.off_pos = off;
  off += align256(np * 4);
  p.off_tiles = off;
  off += align256((size_t)p.max_tiles * 16);
  p.off_counts = off;
  off += 256;
  p.off_h = off;
  off += align256(np * I * 2);
  p.off_d = off;
  off += align256(np * H * 4);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_moe_prefill(const uint16_t* x16, const uint8_t* Wg, const uint8_t* Wu,
                              const uint8_t* Wd, const int32_t* ids, const float* w, float* out,
                              int T, int H, int I, int E, int topk, void* ws,
                              const MoePrefillPlan& p, hipStream_t st) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* src = reinterpret_cast<int32_t*>(base + p.off_src);
  int32_t* pos = reinterpret_cast<int32_t*>(base + p.off_pos);
  int4* tiles = reinterpret_cast<int4*>(base + p.off_tiles);
  int* counts = reinterpret_cast<int*>(base + p.off_counts);
  _Float16* h = reinterpret_cast<_Float16*>(base + p.off_h);
  float* D = reinterpret_cast<float*>(base + p.off_d);
  const int npairs = T * topk;
  const size_t mat = (size_t)H * (I / kBlockWeights) * kBlockBytes;

  PrefillRoute r{ids, npairs, E, topk, src, pos, tiles, counts};
  hipLaunchKernelGGL(moe_prefill_route_kernel, dim3(1), dim3(kRouteThreads), route_lds_bytes(E),
                     st, r);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_gemm_grouped(x16, T, Wg, Wu, mat, nullptr, h, I, H, tiles, counts, p.max_tiles,
                            src, st);
  if (err != hipSuccess) return err;
  err = launch_gemm_grouped(reinterpret_cast<const uint16_t*>(h), npairs, Wd, nullptr, mat, D,
                            nullptr, H, I, tiles, counts, p.max_tiles, nullptr, st);
  if (err != hipSuccess) return err;
  const size_t total4 = (size_t)T * H / 4;
  hipLaunchKernelGGL(moe_prefill_combine_kernel, dim3((unsigned)((total4 + 255) / 256)), dim3(256),
                     0, st, D, pos, w, out, T, H, topk);
  return hipGetLastError();
}

}  // namespace q4
