// Routed-expert MoE decode over Q4_0 expert weights (DeepSeek-V2 shape).
//
// The KTransformers DeepSeek-V2 tutorial ("Optimization 3", arithmetic-
// intensity guided offload) describes the routed experts at decode as a set of
// batched GEMVs: each token picks 6 of 160 experts, so only 3.75 % of the
// expert weights are touched per token and the work is bandwidth-bound. The
// MoE module's gate hands the experts top-k ids and weights, and the expert
// outputs are gathered on one device. Here the whole layer runs on one GPU as
// five kernels on one stream (no host round trip, capturable in a graph):
//
//   1. route    : one workgroup groups the (token, slot) pairs by expert
//                 (stable order). An expert with 1 or 2 pairs becomes one
//                 vector work item; one with 3 or more becomes ceil(n / 8)
//                 matrix-core items of balanced sizes (3 .. 8 pairs). A single
//                 token skips it: its 6 pairs are the (vector) items.
//   2. gate/up  : split-K GEMV tiles over the routed experts' gate and up
//                 matrices, two kernels over the two item lists: the dense
//                 decode kernel's vector tiles (one or two pairs), and the
//                 fp32 matrix-core tiles (3 .. 8 pairs, one weight per lane
//                 against 4 pairs per v_mfma_f32_4x4x1). A tile streams its
//                 expert's row segments once for all pairs of its item and
//                 writes per-pair partial sums.
// At a few tokens per expert the FMA and unpack work (not HBM) bounds the
// vector tiles, so what matters there is how many waves each SIMD can
// interleave: items of at most 2 pairs keep those tiles small in registers and
// LDS. Experts chosen by more pairs (hot experts under skewed routing) go to
// the matrix cores, which take their FMAs 4 pairs at a time and stream the
// expert's weights once per 8 pairs instead of once per 2.
//   3. act      : h = SiLU(sum of gate partials) * (sum of up partials).
//   4. down     : split-K tiles of h . Wd_e, per-pair partial sums.
//   5. combine  : out[t] = sum over slots in order 0..topk-1 of
//                 w[t][s] * (sum of the slot's down partials).
// No atomics and no cross-workgroup hand-off inside a kernel: deterministic.
// For T >= 2 the K splits depend only on (H, I), never on T or on the item
// sizes, and both tile kinds form the same FMA chains in the same 16 row
// phases and sum them in the same order, so a token's result is bitwise the
// same whatever other tokens share the call (batch invariance); a single token
// uses finer K splits, so it matches its batched result to rounding, not
// bitwise.
#include "q4_device.hpp"
#include "q4_internal.hpp"
#include "q4_mfma.hpp"
#include "q4_route.hpp"

namespace q4 {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kMaxChunk = 2;  // pairs per vector work item (MC <= kMaxChunk)
constexpr int kMfmaPairs = 8;  // pairs per matrix-core work item (3 .. 8)
constexpr int kMfmaJW = 4;     // matrix-core tiles: 4 block columns, 4 waves: 16 row
constexpr int kMfmaNW = 4;     // phases, the same phases as the vector tiles
constexpr int kSplitLoads = 16;    // act: splits summed with all loads in flight
constexpr int kCombineSplits = 16;  // combine: splits it sums with every load in flight
constexpr int kLPB = 1;       // whole-block lane shares, for every item size
constexpr int kJt = 16;       // block columns per tile: 288-byte row segments

struct ItemRec {
  int e, cnt, pad0, pad1;
  int pairs[kMfmaPairs];  // pair index t * topk + slot, in stable expert order
};

// The routing table's record is the header's q4_moe_item (inspection ABI).
static_assert(sizeof(ItemRec) == sizeof(q4_moe_item) && offsetof(ItemRec, e) ==
              offsetof(q4_moe_item, expert) && offsetof(ItemRec, cnt) ==
              offsetof(q4_moe_item, count) && offsetof(ItemRec, pairs) ==
              offsetof(q4_moe_item, pairs), "routing table record layout");

constexpr int kMaxRB = 4;       // rows per lane in one pipelined batch (per-lane path)
constexpr int kStagedRB = 2;    // rows per lane in one batch of the staged path
constexpr int kStagedBufs = 2;  // weight buffers per wave of the staged path

template <int M>
constexpr int moe_rows_per_batch() {
  return kMaxRB;
}

// ---------------------------------------------------------------------------
// 1. routing prologue
// ---------------------------------------------------------------------------
struct RouteArgs {
  const int32_t* __restrict__ ids;  // [npairs]
  int npairs, E;
  ItemRec* __restrict__ items;      // vector items: an expert's 1 or 2 pairs
  int* __restrict__ n_items;
  ItemRec* __restrict__ mitems;     // matrix-core items: 3 .. 8 pairs of one expert
  int* __restrict__ n_mitems;
};

static_assert(Q4_MOE_MAX_T * Q4_MOE_MAX_TOPK <= kRouteThreads, "one lane per pair");
constexpr int kRouteWaves = Q4_MOE_MAX_T * Q4_MOE_MAX_TOPK / kWaveSize;

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(RouteArgs a) {
  __shared__ int s_cnt[Q4_MOE_MAX_E];
  __shared__ int s_off[Q4_MOE_MAX_E];
  __shared__ int s_sorted[Q4_MOE_MAX_T * Q4_MOE_MAX_TOPK];
  __shared__ int s_wcnt[kRouteWaves][Q4_MOE_MAX_E];  // pairs per expert in each wave
  __shared__ int s_wsum[kRouteThreads / kWaveSize];
  const int t = threadIdx.x;
  const int lane = t & (kWaveSize - 1);
  const int wave = t / kWaveSize;

  // Lane p holds pair p. Lanes of one wave with the same (valid) expert id
  // find each other with one ballot per id bit: the exact-match mask.
  const int e = t < a.npairs ? a.ids[t] : -1;
  const bool valid = e >= 0 && e < a.E;
  const uint64_t same = same_id_lanes(e, valid);
  const uint64_t below = (1ull << lane) - 1;
  s_cnt[t] = 0;
  for (int i = t; i < kRouteWaves * Q4_MOE_MAX_E; i += kRouteThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  // the first lane of each match group records the group's size
  if (valid && (same & below) == 0) {
    s_wcnt[wave][e] = __popcll(same);
    atomicAdd(&s_cnt[e], __popcll(same));
  }
  __syncthreads();

  // Per-expert offsets into the sorted pair list and into the two item
  // lists: an expert with 1 or 2 pairs makes one vector item; one with 3 or
  // more makes ceil(cnt / 8) matrix-core items of balanced sizes (3 .. 8).
  const int cnt = (t < a.E) ? s_cnt[t] : 0;
  const int nv = (cnt >= 1 && cnt <= kMaxChunk) ? 1 : 0;
  const int nm = cnt > kMaxChunk ? (cnt + kMfmaPairs - 1) / kMfmaPairs : 0;
  const int off = block_inclusive_scan(cnt, s_wsum) - cnt;
  const int v_incl = block_inclusive_scan(nv, s_wsum);
  const int m_incl = block_inclusive_scan(nm, s_wsum);
  s_off[t] = off;
  if (t == kRouteThreads - 1) {
    *a.n_items = v_incl;
    *a.n_mitems = m_incl;
  }
  __syncthreads();

  // Stable placement: pair p goes after the earlier pairs of its expert
  // (those of earlier waves, then the lower lanes of its own wave).
  if (valid) {
    int rank = __popcll(same & below);
    for (int w = 0; w < wave; ++w) rank += s_wcnt[w][e];
    s_sorted[s_off[e] + rank] = t;
  }
  __syncthreads();

  if (nv) {
    ItemRec r;
    r.e = t;
    r.cnt = cnt;
    r.pad0 = r.pad1 = 0;
#pragma unroll
    for (int m = 0; m < kMfmaPairs; ++m) r.pairs[m] = (m < cnt) ? s_sorted[off + m] : 0;
    a.items[v_incl - 1] = r;
  }
  int first = off;
  for (int i = 0; i < nm; ++i) {
    const int sz = cnt / nm + (i < cnt % nm ? 1 : 0);
    ItemRec r;
    r.e = t;
    r.cnt = sz;
    r.pad0 = r.pad1 = 0;
#pragma unroll
    for (int m = 0; m < kMfmaPairs; ++m) r.pairs[m] = (m < sz) ? s_sorted[first + m] : 0;
    a.mitems[m_incl - nm + i] = r;
    first += sz;
  }
}

// ---------------------------------------------------------------------------
// 2./4. expert split-K tiles
// ---------------------------------------------------------------------------
struct ExpertArgs {
  const float* __restrict__ x;        // activations: x [T][H] or h [npairs][I]
  uint32_t x_bytes;
  const uint8_t* __restrict__ W0;     // gate (or down) matrices, E consecutive
  const uint8_t* __restrict__ W1;     // up matrices (gate/up only)
  const ItemRec* __restrict__ items;
  const int* __restrict__ n_items;
  float* __restrict__ part;           // [nmat][S][npairs][N] partial sums
  size_t mat_bytes;
  int K, N, NB;                       // rows, columns, blocks per row of one matrix
  int C, Kt, S, nmat, npairs;
  int x_row_div;                      // activation row = pair / x_row_div, times K
  const int32_t* __restrict__ ids;    // [npairs] expert ids (single-token items)
  int E;
  ActSource act;                      // single-token down: activations from gate/up partials
                                      // (part null: copy x)
};

// ACT: the tile may form its activations from gate/up partials (a.act).
template <int M, bool STAGED, bool ACT>
__device__ void expert_tile(const ExpertArgs& a, const ItemRec& it, int mat, int c, int s,
                            float* smem) {
  constexpr int Lr = kJt * kLPB;
  SplitTile g;
  g.B = (mat == 0 ? a.W0 : a.W1) + (size_t)it.e * a.mat_bytes;
  g.NB = a.NB;
  g.K = a.K;
  g.j0 = c * kJt;
  g.Jt = kJt;
  g.k0 = s * a.Kt;
  g.rows = min(a.Kt, a.K - g.k0);
  g.Lr = Lr;
  g.P = kThreads / Lr;
  int xoff[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xoff[m] = (it.pairs[m] / a.x_row_div) * a.K;
  float acc[M][32 / kLPB];
  float corr[M];
  if constexpr (STAGED)
    tile_accumulate_staged<M, kLPB, kStagedRB, kJt, kStagedBufs>(
        g, a.x, a.x_bytes, xoff, reinterpret_cast<uint8_t*>(smem), acc, corr,
        ACT ? a.act : ActSource{nullptr, 0, 0, 0});
  else
    tile_accumulate<M, kLPB, moe_rows_per_batch<M>()>(g, a.x, a.x_bytes, xoff, smem, acc, corr);
  const int n0 = g.j0 * kBlockWeights;
  const int ncols = min(kJt, a.NB - g.j0) * kBlockWeights;
  float* dst = a.part + ((size_t)mat * a.S + s) * a.npairs * a.N;
  reduce_phases<M, kLPB>(acc, corr, smem, Lr, g.P, ncols, [&](int m, int o, float v) {
    dst[(size_t)it.pairs[m] * a.N + n0 + o] = v;
  });
}

// Vector tile number r of item it: column tile, matrix and K split.
template <int MC, bool STAGED>
__device__ void vector_item_tile(const ExpertArgs& a, const ItemRec& it, int r, float* smem) {
  const int c = r % a.C;
  r /= a.C;
  const int mat = r % a.nmat;
  const int s = r / a.nmat;
  if (it.cnt == 1) {
    expert_tile<1, STAGED, MC == 1>(a, it, mat, c, s, smem);
  } else if constexpr (MC > 1) {
    static_assert(MC == 2, "work items hold at most 2 pairs");
    if (it.cnt == 2) expert_tile<2, STAGED, false>(a, it, mat, c, s, smem);
  }
}

// A single token: item p is pair p, read straight from the routing ids (no
// routing table). The grid is all live tiles, so consecutive tiles (the same
// expert's row segments) are remapped onto one XCD to share its L2.
template <bool STAGED>
__global__ __launch_bounds__(kThreads) void moe_expert_kernel(ExpertArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int per_item = a.nmat * a.C * a.S;
  const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int item = L / per_item;
  if (item >= a.npairs) return;
  const int e = a.ids[item];
  if (e < 0 || e >= a.E) return;  // an invalid slot contributes nothing
  ItemRec it;
  it.e = e;
  it.cnt = 1;
  it.pairs[0] = item;
  vector_item_tile<1, STAGED>(a, it, L - item * per_item, smem);
}

// ---------------------------------------------------------------------------
// 2./4. matrix-core expert tiles (items of 3 .. 8 pairs of one expert)
//
// The same split-K tiles as above (the same K ranges, and 16 row phases that
// take rows p, p + 16, ... in order), but the products run on the fp32 matrix
// cores (mfma_tile_accumulate), one weight per lane against 4 pairs' rows per
// instruction. That instruction rounds like v_fma_f32, so every accumulator is
// the FMA chain a vector tile forms for that phase and column; the phases and
// the corrections are then summed in the vector tiles' fixed order (groups of
// four as (p0 + p2) + (p1 + p3), the groups in turn) and finished with the
// vector tiles' expression. A pair's partial sums are therefore bitwise the same
// whichever kind of item carries it: results stay independent of how many
// other pairs chose the same expert.
// LDS: the activation rings, then [16 phases][4 rows][128 columns] accumulator
// scratch (one activation half at a time) and [16][8][4] corrections.
// ---------------------------------------------------------------------------
constexpr int kMfmaPhases = kMfmaNW * (16 / kMfmaJW);
constexpr int kMfmaCols = kMfmaJW * kBlockWeights;
constexpr int kMfmaScratchFloats = kMfmaPhases * 4 * kMfmaCols + kMfmaPhases * 8 * kMfmaJW;
static_assert(kMfmaPhases == kThreads / (kJt * kLPB), "matrix-core and vector tiles share phases");

template <int MH>
__device__ void expert_mfma_tile(const ExpertArgs& a, const ItemRec& it, int mat, int c, int s,
                                 float* smem) {
  constexpr int JW = kMfmaJW, NW = kMfmaNW;
  const int lane = threadIdx.x % kWaveSize;
  const int wave = threadIdx.x / kWaveSize;
  const int q = lane & 3;
  const int jj = (lane >> 2) % JW;
  const int p = wave * (16 / JW) + (lane >> 2) / JW;  // this lane's row phase
  MfmaTileGeom g;
  g.B = (mat == 0 ? a.W0 : a.W1) + (size_t)it.e * a.mat_bytes;
  g.NB = a.NB;
  g.j0 = c * JW;
  g.k0 = s * a.Kt;
  g.rows = min(a.Kt, a.K - g.k0);
  int xoff[4 * MH];
#pragma unroll
  for (int m = 0; m < 4 * MH; ++m) xoff[m] = (it.pairs[m] / a.x_row_div) * a.K;
  v4f acc[MH][8];
  float corr[MH];
  mfma_tile_accumulate<MH, JW, NW>(g, a.x, a.x_bytes, xoff, it.cnt, smem, acc, corr);

  float* sa = smem;                                  // [phase][row r][column]
  float* sc = smem + kMfmaPhases * 4 * kMfmaCols;    // [phase][m][block]
  __syncthreads();  // every wave is done with its activation ring
#pragma unroll
  for (int h = 0; h < MH; ++h) sc[(p * 8 + q + 4 * h) * JW + jj] = corr[h];
  const int n0 = g.j0 * kBlockWeights;
  float* dst = a.part + ((size_t)mat * a.S + s) * a.npairs * a.N;
#pragma unroll
  for (int h = 0; h < MH; ++h) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* row = sa + (p * 4 + r) * kMfmaCols + jj * 32 + 8 * q;
      *reinterpret_cast<float4*>(row) =
          float4{acc[h][0][r], acc[h][1][r], acc[h][2][r], acc[h][3][r]};
      *reinterpret_cast<float4*>(row + 4) =
          float4{acc[h][4][r], acc[h][5][r], acc[h][6][r], acc[h][7][r]};
    }
    __syncthreads();
    for (int o = threadIdx.x; o < 4 * kMfmaCols; o += kThreads) {
      const int r = o / kMfmaCols;
      const int n = o - r * kMfmaCols;
      const int m = r + 4 * h;
      if (m < it.cnt && n0 + n < a.N) {
        // the 16 phases in the vector tiles' order (reduce_phases): per group
        // of four, (p0 + p2) + (p1 + p3), then the groups in order
        auto ph = [&](int pp) { return sa[(pp * 4 + r) * kMfmaCols + n]; };
        auto pc = [&](int pp) { return sc[(pp * 8 + m) * JW + n / kBlockWeights]; };
        float sum = (ph(0) + ph(2)) + (ph(1) + ph(3));
        float cs = (pc(0) + pc(2)) + (pc(1) + pc(3));
#pragma unroll
        for (int w = 1; w < kMfmaPhases / 4; ++w) {
          sum += (ph(4 * w) + ph(4 * w + 2)) + (ph(4 * w + 1) + ph(4 * w + 3));
          cs += (pc(4 * w) + pc(4 * w + 2)) + (pc(4 * w + 1) + pc(4 * w + 3));
        }
        const float c8 = 8.0f * cs;
        // the pair of row m, selected without indexing the record at run time
        // (the record then stays in scalar registers)
        int pr = 0;
#pragma unroll
        for (int mm = 0; mm < 4 * MH; ++mm)
          if (mm == m) pr = it.pairs[mm];
        dst[(size_t)pr * a.N + n0 + n] = ((n & 1) ? sum * 0.0625f : sum) - c8;
      }
    }
    __syncthreads();
  }
}

// Matrix-core tile number r of item it.
__device__ void mfma_item_tile(const ExpertArgs& a, const ItemRec& it, int r, float* smem) {
  const int c = r % a.C;
  r /= a.C;
  const int mat = r % a.nmat;
  const int s = r / a.nmat;
  if (it.cnt > 4)
    expert_mfma_tile<2>(a, it, mat, c, s, smem);
  else
    expert_mfma_tile<1>(a, it, mat, c, s, smem);
}

// A batch: the vector items (a) and the matrix-core items (am) in one grid.
// The grid is sized for the most items the routing can make; tiles past the
// live count exit at once. The live tiles are handed out in chunks of
// kTileChunk consecutive tiles of one kind: the column tiles of the same rows
// (consecutive in both kinds' tile order) share 128-byte lines at their edges,
// so a chunk runs on one XCD and those lines are fetched into its L2 once
// (at 32 tokens this cut the expert kernels' HBM reads from 1.6x to about 1.1x
// the experts' bytes).
// Chunks go round robin over the 8 XCDs (all of them get live work). The
// vector chunks come first and the matrix-core chunks after them: a vector
// tile streams 4x the bytes of a matrix-core tile and runs about twice as long
// (41 against 21 us at 32 tokens), so with the short tiles last the grid's
// tail is about half as long. Against chunks of both kinds interleaved
// through the grid (same box, alternating builds): 32-token call 334.2 ->
// 313.2 us, skewed routing 260.5 -> 250.5 us, whole layer 387.8 -> 373.4 us.
// Two kernels would run one after the other on the stream, each with its own
// ramp and tail.
// 12: the gate/up column tiles of one matrix-core row run, or four vector
// ones (3 each); same-box sweep at 32 tokens: 12 / 24 / 48 tiles gave
// 341 / 343 / 346 us (smaller chunks spread the live tiles more evenly).
constexpr int kTileChunk = 12;

// Workgroups to launch for Lv vector and Lm matrix-core tiles at most: every
// XCD needs a whole number of chunk slots for the chunks it can be given.
inline long long mixed_grid(long long Lv, long long Lm) {
  const long long chunks = (Lv + kTileChunk - 1) / kTileChunk + (Lm + kTileChunk - 1) / kTileChunk;
  return (chunks + kNumXcd - 1) / kNumXcd * kNumXcd * kTileChunk;
}

template <bool STAGED>
__global__ __launch_bounds__(kThreads) void moe_expert_mixed_kernel(ExpertArgs a, ExpertArgs am) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int pv = a.nmat * a.C * a.S;
  const int pm = am.nmat * am.C * am.S;
  const int Lv = *a.n_items * pv;
  const int Lm = *am.n_items * pm;
  constexpr int G = kTileChunk;
  const int Cv = (Lv + G - 1) / G;
  const int Cm = (Lm + G - 1) / G;
  const int Ct = Cv + Cm;
  // Workgroup b runs on XCD b % 8 as that XCD's (b / 8)-th workgroup: there it
  // takes tile o of chunk q, the XCD's (b / 8 / G)-th chunk.
  const int x = blockIdx.x % kNumXcd;
  const int i = blockIdx.x / kNumXcd;
  const int q = x + kNumXcd * (i / G);
  const int o = i % G;
  if (q >= Ct) return;
  if (q >= Cv) {
    const int m = (q - Cv) * G + o;
    if (m >= Lm) return;
    const int item = m / pm;
    const ItemRec it = am.items[item];
    mfma_item_tile(am, it, m - item * pm, smem);
  } else {
    const int v = q * G + o;
    if (v >= Lv) return;
    const int item = v / pv;
    const ItemRec it = a.items[item];
    vector_item_tile<kMaxChunk, STAGED>(a, it, v - item * pv, smem);
  }
}

// ---------------------------------------------------------------------------
// 3. h = SiLU(gate) * up from the split-K partials (split order)
// ---------------------------------------------------------------------------
// One-wave workgroups and non-temporal loads of the partials (read once), as
// in the decode GEMV's split-K sum; the combine below does the same.
constexpr int kSumThreads = 64;

__global__ __launch_bounds__(kSumThreads) void moe_act_kernel(const float* __restrict__ part,
                                                              float* __restrict__ h, int npairs,
                                                              int I, int S) {
  const size_t idx = (size_t)blockIdx.x * kSumThreads + threadIdx.x;
  if (idx >= (size_t)npairs * I) return;
  // Pairs with an invalid expert id have no partial sums; their h is never
  // read, so they are not filtered here (no dependent id load).
  const size_t slab = (size_t)npairs * I;
  float g, u;
  if (S <= kSplitLoads) {
    // all 2S loads in flight at once (indices clamped; extra values unused)
    float tg[kSplitLoads], tu[kSplitLoads];
#pragma unroll
    for (int k = 0; k < kSplitLoads; ++k) {
      const size_t sk = (size_t)min(k, S - 1);
      tg[k] = __builtin_nontemporal_load(part + sk * slab + idx);
      tu[k] = __builtin_nontemporal_load(part + ((size_t)S + sk) * slab + idx);
    }
    g = 0.0f;
    u = 0.0f;
#pragma unroll
    for (int k = 0; k < kSplitLoads; ++k)
      if (k < S) {
        g += tg[k];
        u += tu[k];
      }
  } else {
    g = sum_strided(part + idx, slab, S);
    u = sum_strided(part + (size_t)S * slab + idx, slab, S);
  }
  h[idx] = g / (1.0f + expf(-g)) * u;
}

// ---------------------------------------------------------------------------
// 5. combine: slot order 0..topk-1, split order inside each slot
// ---------------------------------------------------------------------------
template <int SMAX>
__global__ __launch_bounds__(kSumThreads) void moe_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ ids, const float* __restrict__ w,
    float* __restrict__ out, int T, int H, int E, int topk, int S) {
  const size_t idx = (size_t)blockIdx.x * kSumThreads + threadIdx.x;
  if (idx >= (size_t)T * H) return;
  const int t = (int)(idx / H);
  const int n = (int)(idx - (size_t)t * H);
  const size_t slab = (size_t)T * topk * H;
  float acc = 0.0f;
  if (SMAX > 0) {
    // ids, weights and every split partial of every slot in flight at once
    // (indices clamped; values of invalid slots are loaded but not used)
    constexpr int SM = SMAX > 0 ? SMAX : 1;
    int ev[Q4_MOE_MAX_TOPK];
    float wv[Q4_MOE_MAX_TOPK], pv[Q4_MOE_MAX_TOPK][SM];
#pragma unroll
    for (int sl = 0; sl < Q4_MOE_MAX_TOPK; ++sl) {
      const int p = t * topk + min(sl, topk - 1);
      ev[sl] = ids[p];
      wv[sl] = w[p];
#pragma unroll
      for (int k = 0; k < SM; ++k)
        pv[sl][k] =
            __builtin_nontemporal_load(part + (size_t)min(k, S - 1) * slab + (size_t)p * H + n);
    }
#pragma unroll
    for (int sl = 0; sl < Q4_MOE_MAX_TOPK; ++sl) {
      if (sl >= topk || ev[sl] < 0 || ev[sl] >= E) continue;
      float yd = 0.0f;
#pragma unroll
      for (int k = 0; k < SM; ++k)
        if (k < S) yd += pv[sl][k];
      acc = __builtin_fmaf(wv[sl], yd, acc);
    }
  } else {
    for (int sl = 0; sl < topk; ++sl) {
      const int e = ids[t * topk + sl];
      if (e < 0 || e >= E) continue;
      const size_t o = (size_t)(t * topk + sl) * H + n;
      const float yd = sum_strided(part + o, slab, S);
      acc = __builtin_fmaf(w[t * topk + sl], yd, acc);
    }
  }
  out[idx] = acc;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

void plan_tiles(int K, int NB, int kt_target, int& C, int& Kt, int& S) {
  constexpr int P = kThreads / (kJt * kLPB);
  C = (NB + kJt - 1) / kJt;
  S = (K + kt_target - 1) / kt_target;
  if (S < 1) S = 1;
  Kt = (K + S - 1) / S;
  Kt = (Kt + P - 1) / P * P;
  S = (K + Kt - 1) / Kt;
}

// A single token's K split: the largest S (at most max_S) whose grid of
// C column tiles x nmat matrices x S splits x npairs items stays within
// kSingleGrid workgroups (two per CU). Same-box sweeps of the gate/up tile
// height: 6 experts 576 / 504 / 432 / 360 workgroups gave 30.2 / 28.5 / 29.3 /
// 30.4 us per call, 8 experts (the whole layer) 768 / 672 / 576 / 480 gave
// 45.7 / 46.1 / 47.4 / 45.4 us: about 500 workgroups either way. The down
// tiles follow the same rule (480 workgroups of 192 rows instead of 240 of
// 384: 28.45 -> 27.55 us per call, 45.0 -> 43.55 us per layer), with the
// combine summing up to kCombineSplits splits with every load in flight.
constexpr int kSingleGrid = 512;
void plan_single_tiles(int K, int NB, int nmat, int npairs, int max_S, int& C, int& Kt, int& S) {
  constexpr int P = kThreads / (kJt * kLPB);
  C = (NB + kJt - 1) / kJt;
  int s = kSingleGrid / (C * nmat * npairs);
  s = s < 1 ? 1 : (s > max_S ? max_S : s);
  plan_tiles(K, NB, (K + s - 1) / s, C, Kt, S);
  if (Kt < P) plan_tiles(K, NB, P, C, Kt, S);
}

// LDS of the vector tiles for items of up to MC pairs (activation tile or
// weight staging, then the phase sums).
template <int MC>
int vector_lds_bytes(int Kt, bool staged) {
  constexpr int P = kThreads / (kJt * kLPB);
  const int rf = 4 * phase_lds_floats<MC, kLPB>();
  const int t = staged ? staged_lds_bytes<MC, kLPB, kStagedRB, kJt, kStagedBufs>(Kt)
                       : 4 * tile_x_floats<MC>(Kt, P, kMaxRB);  // every item size M <= MC
  return t > rf ? t : rf;
}

// LDS of the matrix-core tiles: the activation rings, then the phase sums.
int mfma_item_lds_bytes() {
  const int xs = mfma_ring_bytes<2, kMfmaJW, kMfmaNW>();
  const int sc = 4 * kMfmaScratchFloats;
  return xs > sc ? xs : sc;
}

hipError_t launch_expert_single(const ExpertArgs& a, int max_items, bool staged, hipStream_t st) {
  const dim3 grid(max_items * a.nmat * a.C * a.S);
  const int lds = vector_lds_bytes<1>(a.Kt, staged);
  if (staged)
    hipLaunchKernelGGL((moe_expert_kernel<true>), grid, dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((moe_expert_kernel<false>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_expert_mixed(const ExpertArgs& a, const ExpertArgs& am, int max_items,
                               int max_mitems, bool staged, hipStream_t st) {
  const long long g = mixed_grid((long long)max_items * a.nmat * a.C * a.S,
                                 (long long)max_mitems * am.nmat * am.C * am.S);
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)g);
  const int lv = vector_lds_bytes<kMaxChunk>(a.Kt, staged);
  const int lm = max_mitems > 0 ? mfma_item_lds_bytes() : 0;
  const int lds = lv > lm ? lv : lm;
  if (staged)
    hipLaunchKernelGGL((moe_expert_mixed_kernel<true>), grid, dim3(kThreads), lds, st, a, am);
  else
    hipLaunchKernelGGL((moe_expert_mixed_kernel<false>), grid, dim3(kThreads), lds, st, a, am);
  return hipGetLastError();
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
  // One pair per item for a single token (only the M = 1 tiles are compiled
  // into that variant); up to 2 pairs of one expert per item otherwise.
  // Batches: an expert with 1 or 2 pairs is one vector item (at most one per
  // expert), one with more is matrix-core items of 3 .. 8 pairs.
  p.MC = (T == 1) ? 1 : kMaxChunk;
  p.max_items = (T == 1) ? npairs : (npairs < E ? npairs : E);
  p.max_mitems = (T == 1) ? 0 : npairs / (kMaxChunk + 1);
  // K tiles: a single token has only 6 experts' worth of tiles, so it splits
  // K finer (more workgroups, by plan_single_tiles, sized by its number of
  // items); batches use long tiles (less partial-sum traffic, fewer tile
  // epilogues) that depend only on (H, I), never on T or the routing. With the
  // vector tiles ahead of the matrix-core ones, a same-box sweep at 32 tokens
  // (gate/up rows / down rows): 1280 / 768 313.0 us, 2560 / 768 309.6 us,
  // 2560 / 1536 309.7 us (skewed 249.2 -> 245.3 us), 5120 / 768 342.4 us,
  // 640 / 768 333.4 us, 1280 / 384 330.2 us.
  const bool single = (T == 1);
  if (single)
    plan_single_tiles(H, I / kBlockWeights, 2, npairs, kActMaxSplits, p.gu_C, p.gu_Kt, p.gu_S);
  else
    plan_tiles(H, I / kBlockWeights, 2560, p.gu_C, p.gu_Kt, p.gu_S);
  if (single)
    plan_single_tiles(I, H / kBlockWeights, 1, npairs, kCombineSplits, p.dn_C, p.dn_Kt, p.dn_S);
  else
    plan_tiles(I, H / kBlockWeights, 1536, p.dn_C, p.dn_Kt, p.dn_S);
  p.gu_Cm = (I / kBlockWeights + kMfmaJW - 1) / kMfmaJW;
  p.dn_Cm = (H / kBlockWeights + kMfmaJW - 1) / kMfmaJW;
  size_t off = 0;
  p.off_items = off;
  off += align256((size_t)p.max_items * sizeof(ItemRec));
  p.off_n_items = off;  // two counters: vector items, matrix-core items
  off += 256;
  p.off_mitems = off;
  off += align256((size_t)p.max_mitems * sizeof(ItemRec));
  p.off_gu_part = off;
  off += align256((size_t)2 * p.gu_S * npairs * I * sizeof(float));
  p.off_h = off;
  off += align256((size_t)npairs * I * sizeof(float));
  p.off_dn_part = off;
  off += align256((size_t)p.dn_S * npairs * H * sizeof(float));
  p.ws_bytes = off;
  return p;
}

hipError_t launch_moe(const float* x, const uint8_t* Wg, const uint8_t* Wu, const uint8_t* Wd,
                      const int32_t* ids, const float* w, float* out, void* ws,
                      const MoePlan& p, hipStream_t st) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  ItemRec* items = reinterpret_cast<ItemRec*>(base + p.off_items);
  int* n_items = reinterpret_cast<int*>(base + p.off_n_items);
  float* gu_part = reinterpret_cast<float*>(base + p.off_gu_part);
  float* h = reinterpret_cast<float*>(base + p.off_h);
  float* dn_part = reinterpret_cast<float*>(base + p.off_dn_part);
  const int npairs = p.T * p.topk;

  ItemRec* mitems = reinterpret_cast<ItemRec*>(base + p.off_mitems);
  int* n_mitems = n_items + 1;
  RouteArgs ra;
  ra.ids = ids;
  ra.npairs = npairs;
  ra.E = p.E;
  ra.items = items;
  ra.n_items = n_items;
  ra.mitems = mitems;
  ra.n_mitems = n_mitems;
  hipError_t err = hipSuccess;
  if (p.T > 1) {  // a single token needs no route: its items are the pairs
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, st, ra);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  const size_t mat_bytes = (size_t)p.H * (p.I / kBlockWeights) * kBlockBytes;
  // Wave-private staging needs 16-byte aligned row segments: pitches of a
  // multiple of 8 blocks and 16-byte aligned matrices.
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool staged_gu = (p.I / kBlockWeights) % 8 == 0 && al16(Wg) && al16(Wu);
  const bool staged_dn = (p.H / kBlockWeights) % 8 == 0 && al16(Wd);
  ExpertArgs g;
  g.x = x;
  g.x_bytes = (uint32_t)((size_t)p.T * p.H * sizeof(float));
  g.W0 = Wg;
  g.W1 = Wu;
  g.items = items;
  g.n_items = n_items;
  g.part = gu_part;
  g.mat_bytes = mat_bytes;
  g.K = p.H;
  g.N = p.I;
  g.NB = p.I / kBlockWeights;
  g.C = p.gu_C;
  g.Kt = p.gu_Kt;
  g.S = p.gu_S;
  g.nmat = 2;
  g.npairs = npairs;
  g.x_row_div = p.topk;
  g.ids = ids;
  g.E = p.E;
  g.act = ActSource{nullptr, 0, 0, 0};
  ExpertArgs gm = g;
  gm.items = mitems;
  gm.n_items = n_mitems;
  gm.C = p.gu_Cm;
  err = (p.T == 1) ? launch_expert_single(g, p.max_items, staged_gu, st)
                   : launch_expert_mixed(g, gm, p.max_items, p.max_mitems, staged_gu, st);
  if (err != hipSuccess) return err;

  const size_t nh = (size_t)npairs * p.I;
  // A single token's down tiles form h = SiLU(gate) * up themselves from the
  // gate/up partial sums while staging their activation tile (same sums, same
  // order, same expression as moe_act_kernel), which saves a kernel launch.
  constexpr int kP = kThreads / (kJt * kLPB);
  const bool fuse_act = p.T == 1 && staged_dn && p.gu_S <= kActMaxSplits &&
                        tile_rows_padded(p.dn_Kt, kP, kStagedRB) <= kActMaxVals * kThreads;
  if (!fuse_act) {
    hipLaunchKernelGGL(moe_act_kernel, dim3((unsigned)((nh + kSumThreads - 1) / kSumThreads)),
                       dim3(kSumThreads), 0, st,
                       gu_part, h, npairs, p.I, p.gu_S);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  ExpertArgs d = g;
  d.x = h;
  d.x_bytes = (uint32_t)(nh * sizeof(float));
  d.W0 = Wd;
  d.W1 = nullptr;
  d.part = dn_part;
  d.K = p.I;
  d.N = p.H;
  d.NB = p.H / kBlockWeights;
  d.C = p.dn_C;
  d.Kt = p.dn_Kt;
  d.S = p.dn_S;
  d.nmat = 1;
  d.x_row_div = 1;
  if (fuse_act)
    d.act = ActSource{gu_part, (uint32_t)(2 * (size_t)p.gu_S * nh * sizeof(float)), (uint32_t)nh,
                      p.gu_S};
  ExpertArgs dm = d;
  dm.items = mitems;
  dm.n_items = n_mitems;
  dm.C = p.dn_Cm;
  err = (p.T == 1) ? launch_expert_single(d, p.max_items, staged_dn, st)
                   : launch_expert_mixed(d, dm, p.max_items, p.max_mitems, staged_dn, st);
  if (err != hipSuccess) return err;

  const size_t total = (size_t)p.T * p.H;
  const dim3 cgrid((unsigned)((total + kSumThreads - 1) / kSumThreads)), cblock(kSumThreads);
  if (p.dn_S <= 4)
    hipLaunchKernelGGL(moe_combine_kernel<4>, cgrid, cblock, 0, st, dn_part, ids, w, out, p.T,
                       p.H, p.E, p.topk, p.dn_S);
  else if (p.dn_S <= 8)
    hipLaunchKernelGGL(moe_combine_kernel<8>, cgrid, cblock, 0, st, dn_part, ids, w, out, p.T,
                       p.H, p.E, p.topk, p.dn_S);
  else if (p.dn_S <= kCombineSplits)
    hipLaunchKernelGGL(moe_combine_kernel<kCombineSplits>, cgrid, cblock, 0, st, dn_part, ids, w,
                       out, p.T, p.H, p.E, p.topk, p.dn_S);
  else
    hipLaunchKernelGGL(moe_combine_kernel<0>, cgrid, cblock, 0, st, dn_part, ids, w, out, p.T,
                       p.H, p.E, p.topk, p.dn_S);
  return hipGetLastError();
}

}  // namespace q4
