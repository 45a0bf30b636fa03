// Routed-expert MoE decode over Q4_0 expert weights (DeepSeek-V2 shape).
//
// The KTransformers DeepSeek-V2 tutorial ("Optimization 3", arithmetic-
// intensity guided offload) describes the routed experts at decode as a set of
// batched GEMVs: each token picks 6 of 160 experts, so only 3.75 % of the
// expert weights are touched per token and the work is bandwidth-bound. The
// MoE module's gate hands the experts top-k ids and weights, and the expert
// outputs are gathered on one device. Here the whole layer runs on one GPU as
// four kernels on one stream (no host round trip, capturable in a graph):
//
//   1. route    : one workgroup turns topk_ids into expert groups: the (token,
//                 slot) pairs sorted by expert (stable), and work items of at
//                 most 8 pairs of one expert; it also clears the tickets.
//   2. gate/up  : for each work item, column tile and K split, the expert's
//                 gate and up matrices are streamed once for all its pairs
//                 (GEMV tiles of the dense decode kernel); the last workgroup
//                 of a tile group applies h = SiLU(g) * u.
//   3. down     : yd = h . Wd_e per pair, split-K with a completion ticket.
//   4. combine  : out[t] = sum over slots in order 0..topk-1 of w[t][s] * yd.
//
// Tile shapes depend only on (H, I), so a token's result is bitwise the same
// whatever other tokens share the call (batch invariance).
#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kMaxChunk = 8;  // pairs per work item
constexpr int kLPB = 2;       // lanes per block in the expert GEMV tiles

struct WorkItem {
  int e, start, cnt, pad;
};

// ---------------------------------------------------------------------------
// 1. routing prologue
// ---------------------------------------------------------------------------
struct RouteArgs {
  const int32_t* __restrict__ ids;  // [T*topk]
  int npairs, E;
  int* __restrict__ pair_sorted;    // [npairs]
  WorkItem* __restrict__ items;     // [max_items]
  int* __restrict__ n_items;
  unsigned* __restrict__ tickets;   // counters to clear
  int n_tickets;
};

// Inclusive prefix sum over kRouteThreads values held one per lane.
__device__ int block_inclusive_scan(int v, int* buf) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int add = (t >= off) ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  const int r = buf[t];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(RouteArgs a) {
  __shared__ int s_ids[Q4_MOE_MAX_T * Q4_MOE_MAX_TOPK];
  __shared__ int s_rank[Q4_MOE_MAX_T * Q4_MOE_MAX_TOPK];
  __shared__ int s_count[kRouteThreads];
  __shared__ int s_scan[kRouteThreads];
  const int t = threadIdx.x;

  for (int i = t; i < a.n_tickets; i += kRouteThreads) a.tickets[i] = 0u;
  s_count[t] = 0;
  for (int p = t; p < a.npairs; p += kRouteThreads) s_ids[p] = a.ids[p];
  __syncthreads();

  // Rank of each valid pair among the earlier pairs of its expert (stable order).
  for (int p = t; p < a.npairs; p += kRouteThreads) {
    const int e = s_ids[p];
    if (e < 0 || e >= a.E) continue;
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += (s_ids[q] == e) ? 1 : 0;
    s_rank[p] = rank;
    atomicAdd(&s_count[e], 1);
  }
  __syncthreads();

  const int cnt = (t < a.E) ? s_count[t] : 0;
  const int nch = (cnt + kMaxChunk - 1) / kMaxChunk;
  const int off_incl = block_inclusive_scan(cnt, s_scan);
  const int item_incl = block_inclusive_scan(nch, s_scan);
  const int off = off_incl - cnt;
  const int item_off = item_incl - nch;
  s_count[t] = off;  // reuse as the expert's start in pair_sorted
  if (t == kRouteThreads - 1) *a.n_items = item_incl;
  __syncthreads();

  for (int p = t; p < a.npairs; p += kRouteThreads) {
    const int e = s_ids[p];
    if (e < 0 || e >= a.E) continue;
    a.pair_sorted[s_count[e] + s_rank[p]] = p;
  }
  for (int i = 0; i < nch; ++i) {
    WorkItem w;
    w.e = t;
    w.start = off + i * kMaxChunk;
    w.cnt = min(kMaxChunk, cnt - i * kMaxChunk);
    w.pad = 0;
    a.items[item_off + i] = w;
  }
}

// ---------------------------------------------------------------------------
// 2./3. expert GEMV tiles
// ---------------------------------------------------------------------------
struct ExpertArgs {
  const float* __restrict__ xin;       // activations: x [T][H] (gate/up) or h [pairs][I] (down)
  const uint8_t* __restrict__ W0;      // gate (gate/up) or down matrices
  const uint8_t* __restrict__ W1;      // up matrices (gate/up only)
  const int* __restrict__ pair_sorted;
  const WorkItem* __restrict__ items;
  const int* __restrict__ n_items;
  float* __restrict__ part;            // [nmat][C][S][npairs][width]
  unsigned* __restrict__ tickets;      // [max_items][C]
  float* __restrict__ out;             // h [pairs][I] (gate/up) or yd [pairs][H] (down)
  size_t mat_bytes;                    // bytes of one expert matrix
  int K, N, NB;                        // rows, columns, blocks per row of one matrix
  int Jt, Lr, P, C, Kt, S, nmat;
  int topk, npairs;
  int x_by_token;                      // 1: xin row = pair / topk (gate/up); 0: xin row = pair
};

template <int M>
__device__ void expert_tile(const ExpertArgs& a, const WorkItem& it, int item, int mat, int c,
                            int s, float* smem, unsigned* flag) {
  constexpr int XS = x_stride<M>();
  const int t = threadIdx.x;
  const int k0 = s * a.Kt;
  const int rows = min(a.Kt, a.K - k0);
  const int j0 = c * a.Jt;

  // Stage the activation rows of this item's pairs.
  for (int idx = t; idx < M * rows; idx += kThreads) {
    const int m = idx / rows;
    const int kk = idx - m * rows;
    const int pair = a.pair_sorted[it.start + m];
    const int xrow = a.x_by_token ? pair / a.topk : pair;
    smem[kk * XS + m] = a.xin[(size_t)xrow * a.K + k0 + kk];
  }
  __syncthreads();

  float acc[M][32 / kLPB];
  float corr[M];
  const uint8_t* W = (mat == 0 ? a.W0 : a.W1) + (size_t)it.e * a.mat_bytes;
  const TileGeom g{W, a.NB, j0, k0, rows, a.Lr, a.P};
  tile_accumulate<M, kLPB, 4>(g, smem, acc, corr);
  finish_part<M, kLPB>(acc, corr);

  const int width = a.Jt * kBlockWeights;
  const int ncols = min(width, (a.NB - j0) * kBlockWeights);
  __syncthreads();
  // partial slab of (mat, c, s), rows indexed by position in pair_sorted
  float* __restrict__ slab =
      a.part + (((size_t)mat * a.C + c) * a.S + s) * (size_t)a.npairs * width;
  reduce_phases<M, kLPB>(acc, smem, a.Lr, a.P, ncols, [&](int m, int o, float v) {
    slab[(size_t)(it.start + m) * width + o] = v;
  });

  if (!arrive_last(a.tickets + (size_t)item * a.C + c, (unsigned)(a.S * a.nmat), flag)) return;

  // Last workgroup of (item, column tile): sum the split partials in order.
  for (int idx = t; idx < M * ncols; idx += kThreads) {
    const int m = idx / ncols;
    const int o = idx - m * ncols;
    const size_t row = (size_t)(it.start + m) * width + o;
    float v0 = 0.0f;
    for (int ss = 0; ss < a.S; ++ss)
      v0 += a.part[(((size_t)0 * a.C + c) * a.S + ss) * (size_t)a.npairs * width + row];
    const int pair = a.pair_sorted[it.start + m];
    float res;
    if (a.nmat == 2) {
      float v1 = 0.0f;
      for (int ss = 0; ss < a.S; ++ss)
        v1 += a.part[(((size_t)1 * a.C + c) * a.S + ss) * (size_t)a.npairs * width + row];
      res = v0 / (1.0f + expf(-v0)) * v1;  // SiLU(gate) * up
    } else {
      res = v0;
    }
    a.out[(size_t)pair * a.N + (size_t)j0 * kBlockWeights + o] = res;
  }
}

__global__ __launch_bounds__(kThreads) void moe_expert_kernel(ExpertArgs a) {
  extern __shared__ float smem[];
  __shared__ unsigned flag;
  const int per_item = a.nmat * a.C * a.S;
  const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int item = L / per_item;
  if (item >= *a.n_items) return;
  int rest = L - item * per_item;
  const int c = rest % a.C;
  rest /= a.C;
  const int mat = rest % a.nmat;
  const int s = rest / a.nmat;
  const WorkItem it = a.items[item];
  switch (it.cnt) {
    case 1: expert_tile<1>(a, it, item, mat, c, s, smem, &flag); break;
    case 2: expert_tile<2>(a, it, item, mat, c, s, smem, &flag); break;
    case 3: expert_tile<3>(a, it, item, mat, c, s, smem, &flag); break;
    case 4: expert_tile<4>(a, it, item, mat, c, s, smem, &flag); break;
    case 5: expert_tile<5>(a, it, item, mat, c, s, smem, &flag); break;
    case 6: expert_tile<6>(a, it, item, mat, c, s, smem, &flag); break;
    case 7: expert_tile<7>(a, it, item, mat, c, s, smem, &flag); break;
    case 8: expert_tile<8>(a, it, item, mat, c, s, smem, &flag); break;
    default: break;
  }
}

// ---------------------------------------------------------------------------
// 4. slot-ordered combine
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void moe_combine_kernel(const float* __restrict__ yd,
                                                               const int32_t* __restrict__ ids,
                                                               const float* __restrict__ w,
                                                               float* __restrict__ out, int T,
                                                               int H, int E, int topk) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)T * H) return;
  const int t = (int)(idx / H);
  const int n = (int)(idx - (size_t)t * H);
  float acc = 0.0f;
  for (int s = 0; s < topk; ++s) {
    const int e = ids[t * topk + s];
    if (e < 0 || e >= E) continue;
    acc = __builtin_fmaf(w[t * topk + s], yd[(size_t)(t * topk + s) * H + n], acc);
  }
  out[idx] = acc;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

void plan_gemv_tiles(int K, int NB, int kt_target, int& Jt, int& Lr, int& P, int& C, int& Kt,
                     int& S) {
  Jt = NB < 16 ? NB : 16;
  Lr = Jt * kLPB;
  P = kThreads / Lr;
  C = (NB + Jt - 1) / Jt;
  S = (K + kt_target / 2) / kt_target;
  if (S < 1) S = 1;
  Kt = (K + S - 1) / S;
  Kt = (Kt + P - 1) / P * P;
  if (Kt > 1024) Kt = 1024;
  S = (K + Kt - 1) / Kt;
}

}  // namespace

MoePlan plan_moe(int T, int H, int I, int E, int topk) {
  MoePlan p{};
  p.T = T;
  p.H = H;
  p.I = I;
  p.E = E;
  p.topk = topk;
  const int npairs = T * topk;
  const int bound = E + npairs / kMaxChunk;
  p.max_items = npairs < bound ? npairs : bound;
  plan_gemv_tiles(H, I / kBlockWeights, 320, p.gu_Jt, p.gu_Lr, p.gu_P, p.gu_C, p.gu_Kt, p.gu_S);
  plan_gemv_tiles(I, H / kBlockWeights, 192, p.dn_Jt, p.dn_Lr, p.dn_P, p.dn_C, p.dn_Kt, p.dn_S);
  const size_t red = (size_t)(32 / kLPB) * kRedStride;
  p.gu_lds = 4 * (((size_t)p.gu_Kt * 8) > red ? (size_t)p.gu_Kt * 8 : red);
  p.dn_lds = 4 * (((size_t)p.dn_Kt * 8) > red ? (size_t)p.dn_Kt * 8 : red);
  size_t off = 0;
  p.off_route = off;
  off += align256((size_t)npairs * 4) + align256((size_t)p.max_items * sizeof(WorkItem)) + 256;
  p.off_gu_cnt = off;
  off += align256((size_t)p.max_items * p.gu_C * 4);
  p.off_dn_cnt = off;
  off += align256((size_t)p.max_items * p.dn_C * 4);
  p.off_gu_part = off;
  off += align256((size_t)2 * p.gu_C * p.gu_S * npairs * p.gu_Jt * kBlockWeights * 4);
  p.off_dn_part = off;
  off += align256((size_t)p.dn_C * p.dn_S * npairs * p.dn_Jt * kBlockWeights * 4);
  p.off_h = off;
  off += align256((size_t)npairs * I * 4);
  p.off_yd = off;
  off += align256((size_t)npairs * H * 4);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_moe(const float* x, const uint8_t* Wg, const uint8_t* Wu, const uint8_t* Wd,
                      const int32_t* ids, const float* w, float* out, void* ws,
                      const MoePlan& p, hipStream_t st) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  const int npairs = p.T * p.topk;
  int* pair_sorted = reinterpret_cast<int*>(base + p.off_route);
  WorkItem* items = reinterpret_cast<WorkItem*>(base + p.off_route + align256((size_t)npairs * 4));
  int* n_items = reinterpret_cast<int*>(base + p.off_route + align256((size_t)npairs * 4) +
                                        align256((size_t)p.max_items * sizeof(WorkItem)));
  unsigned* gu_cnt = reinterpret_cast<unsigned*>(base + p.off_gu_cnt);
  unsigned* dn_cnt = reinterpret_cast<unsigned*>(base + p.off_dn_cnt);
  float* gu_part = reinterpret_cast<float*>(base + p.off_gu_part);
  float* dn_part = reinterpret_cast<float*>(base + p.off_dn_part);
  float* h = reinterpret_cast<float*>(base + p.off_h);
  float* yd = reinterpret_cast<float*>(base + p.off_yd);

  RouteArgs ra;
  ra.ids = ids;
  ra.npairs = npairs;
  ra.E = p.E;
  ra.pair_sorted = pair_sorted;
  ra.items = items;
  ra.n_items = n_items;
  ra.tickets = gu_cnt;  // gate/up and down tickets are adjacent
  ra.n_tickets = (int)((p.off_gu_part - p.off_gu_cnt) / 4);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, st, ra);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const size_t mat_bytes = (size_t)p.H * (p.I / kBlockWeights) * kBlockBytes;
  ExpertArgs g;
  g.xin = x;
  g.W0 = Wg;
  g.W1 = Wu;
  g.pair_sorted = pair_sorted;
  g.items = items;
  g.n_items = n_items;
  g.part = gu_part;
  g.tickets = gu_cnt;
  g.out = h;
  g.mat_bytes = mat_bytes;
  g.K = p.H;
  g.N = p.I;
  g.NB = p.I / kBlockWeights;
  g.Jt = p.gu_Jt;
  g.Lr = p.gu_Lr;
  g.P = p.gu_P;
  g.C = p.gu_C;
  g.Kt = p.gu_Kt;
  g.S = p.gu_S;
  g.nmat = 2;
  g.topk = p.topk;
  g.npairs = npairs;
  g.x_by_token = 1;
  hipLaunchKernelGGL(moe_expert_kernel, dim3(p.max_items * 2 * p.gu_C * p.gu_S), dim3(kThreads),
                     p.gu_lds, st, g);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  ExpertArgs d = g;
  d.xin = h;
  d.W0 = Wd;
  d.W1 = nullptr;
  d.part = dn_part;
  d.tickets = dn_cnt;
  d.out = yd;
  d.K = p.I;
  d.N = p.H;
  d.NB = p.H / kBlockWeights;
  d.Jt = p.dn_Jt;
  d.Lr = p.dn_Lr;
  d.P = p.dn_P;
  d.C = p.dn_C;
  d.Kt = p.dn_Kt;
  d.S = p.dn_S;
  d.nmat = 1;
  d.x_by_token = 0;
  hipLaunchKernelGGL(moe_expert_kernel, dim3(p.max_items * p.dn_C * p.dn_S), dim3(kThreads),
                     p.dn_lds, st, d);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  const size_t total = (size_t)p.T * p.H;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, yd, ids, w, out, p.T, p.H, p.E, p.topk);
  return hipGetLastError();
}

}  // namespace q4
