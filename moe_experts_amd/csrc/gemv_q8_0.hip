// Decode GEMV over Q8_0 weights: y[M x N] = x[M x K] . deq(B[K x N]), M <= 8.
//
// The "2000-line C++ DeepSeek inference engine" article (§2.2) weighs Q8_0
// against Q4_0: twice the memory, about 60 % of Q4_0's token rate on the
// author's CPU. It does not define Q8_0; read as blocks of 32 weights in 34
// little-endian bytes (a binary16 scale d, then 32 signed bytes q), weight
// l = q[l] * d, blocks along N as for Q4_0. This is the Q4_0 vector GEMV's
// structure with that block:
//   * split-K tiles: workgroup (c, s) owns block columns 8c .. 8c+7 (272-byte
//     row segments) and a K range; its lanes form row phases of 16 (one
//     token) or 32 lanes (several), each lane holding half or a quarter of a
//     block (16 or 8 signed bytes) per row;
//   * each lane loads its rows in batches (an unaligned 16- or 8-byte buffer
//     load plus the 2-byte scale per row, two batches in flight); the
//     activations are staged once per tile in LDS;
//   * per weight one convert (sign-extended byte to fp32) and one FMA per
//     activation row, with s = x * d formed once per block and row;
//   * the row phases are summed through LDS in phase order and the tile is
//     written as one split-K partial (or straight to y), summed by the same
//     reduce kernel as the Q4_0 path.
#include "q4_device.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int kQ8BlockBytes = 34;
constexpr int kQ8Jt = 8;   // block columns per tile
constexpr int kQ8RB = 4;   // rows per lane in one batch

// One lane's share of a block: the scale and 32/LPB signed bytes.
template <int LPB>
struct Q8Part {
  static constexpr int kWords = 8 / LPB;
  uint32_t d;
  uint32_t q[kWords];
};

template <int LPB>
__device__ __forceinline__ void load_q8_part(__amdgpu_buffer_rsrc_t r, uint32_t vofs,
                                             uint32_t sofs, int part, Q8Part<LPB>& out) {
  out.d = __builtin_amdgcn_raw_buffer_load_b16(r, vofs, sofs, 0);
  const uint32_t qo = vofs + 2 + part * (32 / LPB);  // 2-byte aligned: unaligned loads
  if constexpr (LPB == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, qo, sofs, 0);
    out.q[0] = v[0];
    out.q[1] = v[1];
    out.q[2] = v[2];
    out.q[3] = v[3];
  } else {
    static_assert(LPB == 4, "half or quarter blocks");
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, qo, sofs, 0);
    out.q[0] = v[0];
    out.q[1] = v[1];
  }
}

template <int M, int LPB>
__device__ __forceinline__ void fma_q8_part(const float (&xv)[M], const Q8Part<LPB>& b,
                                            float (&acc)[M][32 / LPB]) {
  const float d = half_bits_to_float(b.d);
  float s[M];
#pragma unroll
  for (int m = 0; m < M; ++m) s[m] = xv[m] * d;
#pragma unroll
  for (int w = 0; w < Q8Part<LPB>::kWords; ++w)
#pragma unroll
    for (int by = 0; by < 4; ++by) {
      const float f = static_cast<float>(static_cast<int8_t>(b.q[w] >> (8 * by)));
      const int c = 4 * w + by;
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m][c] = __builtin_fmaf(s[m], f, acc[m][c]);
    }
}

struct Q8Args {
  const float* __restrict__ x;
  const uint8_t* __restrict__ B;
  float* __restrict__ y;
  float* __restrict__ part;  // [S][M][N] split-K partials
  int M, N, K, NB;
  int Lr, P, C, Kt, S;
};

// LDS: the staged activations, then the phase sums ([32/LPB][257] per row m).
template <int M, int LPB>
constexpr int q8_reduce_floats() {
  return (32 / LPB) * (kThreads + 1);
}

template <int M, int LPB>
__global__ __launch_bounds__(kThreads) void gemv_q8_0_kernel(Q8Args a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  constexpr int CPL = 32 / LPB;
  constexpr int RB = kQ8RB;
  constexpr uint32_t kOutOfRange = 0x80000000u;
  constexpr int kLoadsPerBatch = 2 * RB;
  const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int c = L % a.C;
  const int s = L / a.C;
  const int j0 = c * kQ8Jt;
  const int k0 = s * a.Kt;
  const int trows = min(a.Kt, a.K - k0);
  const int t = threadIdx.x;
  const int r = t / a.Lr;
  const int v = t - r * a.Lr;
  const int jj = v / LPB;
  const int part = v - jj * LPB;
  float acc[M][CPL];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int q = 0; q < CPL; ++q) acc[m][q] = 0.0f;
  const bool active = r < a.P && j0 + jj < a.NB;
  const int nl = (trows + a.P - 1) / a.P;  // rows of the busiest lane (uniform)
  const int nb = (nl + RB - 1) / RB;        // batches (uniform)
  const int rows_pad = nb * RB * a.P;
  const uint32_t row_bytes = (uint32_t)a.NB * kQ8BlockBytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.B, (uint32_t)a.K * row_bytes);
  const uint32_t vcol = (uint32_t)(j0 + jj) * kQ8BlockBytes;
  const uint32_t sbase = (uint32_t)k0 * row_bytes;
  const int rows = active ? trows : 0;
  int xoff[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xoff[m] = m * a.K;
  float* xs = smem;
  stage_x_tile<M>(a.x, (uint32_t)(4 * a.M * a.K), xoff, k0, trows, rows_pad, xs);
  __builtin_amdgcn_sched_barrier(0);  // the staging loads go first (the wait below counts on it)

  Q8Part<LPB> A[RB], Bs[RB];
  auto load_batch = [&](int b, Q8Part<LPB>(&R)[RB]) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int tr = (b * RB + i) * a.P + r;
      const uint32_t vo = tr < rows ? vcol + (uint32_t)tr * row_bytes : kOutOfRange;
      load_q8_part<LPB>(rw, vo, sbase, part, R[i]);
    }
  };
  auto compute_batch = [&](int b, Q8Part<LPB>(&R)[RB]) {
    float xv[RB][M];
#pragma unroll
    for (int i = 0; i < RB; ++i) read_x_row<M>(xs, (b * RB + i) * a.P + r, xv[i]);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (b * RB + i < nl) fma_q8_part<M, LPB>(xv[i], R[i], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load_batch(0, A);
  load_batch(1, Bs);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerBatch));  // the activations have landed
  zero_x_pad<M>(xs, trows, rows_pad);
  __syncthreads();
  if (active) {
    int b = 0;
    for (; b + 2 <= nb; b += 2) {
      compute_batch(b, A);
      load_batch(b + 2, A);
      compute_batch(b + 1, Bs);
      load_batch(b + 3, Bs);
    }
    if (b < nb) compute_batch(b, A);
  }

  // Phase sums in phase order 0..P-1, one activation row at a time. Lane
  // (r, jj, part) holds columns 32 (j0 + jj) + part * CPL + q.
  constexpr int kStride = kThreads + 1;
  float* red = smem;  // [CPL][kStride]
  const int ncols = min(kQ8Jt, a.NB - j0) * kBlockWeights;
  float* out = (a.S == 1) ? a.y : a.part + (size_t)s * a.M * a.N;
  const int n0 = j0 * kBlockWeights;
  for (int m = 0; m < M; ++m) {
    __syncthreads();  // the activation tile (or the previous row's sums) is done with
#pragma unroll
    for (int q = 0; q < CPL; ++q) red[q * kStride + t] = acc[m][q];
    __syncthreads();
    for (int o = t; o < ncols; o += kThreads) {
      const int ob = o / kBlockWeights;
      const int c32 = o - ob * kBlockWeights;
      const int pp = c32 / CPL;
      const int q = c32 - pp * CPL;
      const float* src = red + q * kStride + ob * LPB + pp;
      float sum = 0.0f;
      for (int rr = 0; rr < a.P; ++rr) sum += src[rr * a.Lr];
      out[(size_t)m * a.N + n0 + o] = sum;
    }
  }
}

template <int M, int LPB>
hipError_t launch_q8_t(const Q8Args& a, hipStream_t st) {
  const int xf = 4 * tile_x_floats<M>(a.Kt, a.P, kQ8RB);
  const int rf = 4 * q8_reduce_floats<M, LPB>();
  hipLaunchKernelGGL((gemv_q8_0_kernel<M, LPB>), dim3(a.C * a.S), dim3(kThreads),
                     xf > rf ? xf : rf, st, a);
  return hipGetLastError();
}

template <int M>
hipError_t launch_q8_m(const Q8Args& a, hipStream_t st) {
  if constexpr (M == 1) return launch_q8_t<1, 2>(a, st);
  return launch_q8_t<M, 4>(a, st);
}

}  // namespace

// Plan: half blocks per lane for one activation row (16 columns), quarter
// blocks for several (8 columns, fewer accumulators); the K split keeps the
// grid within one round of resident workgroups (352 for M = 1, 512 else,
// as the Q4_0 vector tiles) with at least 128 rows per tile.
namespace {

// Dynamic LDS bytes of a tile of Kt rows (as launch_q8_t sizes it).
template <int M, int LPB>
int q8_lds_bytes_t(int Kt, int P) {
  const int xf = 4 * tile_x_floats<M>(Kt, P, kQ8RB);
  const int rf = 4 * q8_reduce_floats<M, LPB>();
  return xf > rf ? xf : rf;
}

int q8_lds_bytes(int M, int Kt, int P) {
  switch (M) {
    case 1: return q8_lds_bytes_t<1, 2>(Kt, P);
    case 2: return q8_lds_bytes_t<2, 4>(Kt, P);
    case 3: return q8_lds_bytes_t<3, 4>(Kt, P);
    case 4: return q8_lds_bytes_t<4, 4>(Kt, P);
    case 5: return q8_lds_bytes_t<5, 4>(Kt, P);
    case 6: return q8_lds_bytes_t<6, 4>(Kt, P);
    case 7: return q8_lds_bytes_t<7, 4>(Kt, P);
    default: return q8_lds_bytes_t<8, 4>(Kt, P);
  }
}

}  // namespace

GemvPlan plan_gemv_q8(int M, int N, int K) {
  GemvPlan p{};
  const int NB = N / kBlockWeights;
  p.LPB = (M == 1) ? 2 : 4;
  p.Jt = kQ8Jt;
  p.Lr = p.Jt * p.LPB;
  p.P = kThreads / p.Lr;
  p.C = (NB + p.Jt - 1) / p.Jt;
  auto kt_for = [&](int s) {
    const int kt = (K + s - 1) / s;
    return (kt + p.P - 1) / p.P * p.P;
  };
  const int target = M >= 2 ? 512 : 352;
  int best_kt = kt_for(1);  // S = 1
  int last_S = -1;
  for (int s = 2; s <= K; ++s) {
    const int kt = kt_for(s);
    const int S = (K + kt - 1) / kt;
    if (S == last_S) continue;
    last_S = S;
    if (kt < 128 || p.C * S > target) break;
    best_kt = kt;
  }
  // split K further when the activation tile would not fit in LDS
  for (int s = (K + best_kt - 1) / best_kt; q8_lds_bytes(M, best_kt, p.P) > kMaxLdsBytes; ++s)
    best_kt = kt_for(s);
  p.Kt = best_kt;
  p.S = (K + p.Kt - 1) / p.Kt;
  p.ws_bytes = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemv_q8(const float* x, const uint8_t* B, float* y, int M, int N, int K,
                          void* ws, const GemvPlan& p, hipStream_t st) {
  Q8Args a;
  a.x = x;
  a.B = B;
  a.y = y;
  a.part = static_cast<float*>(ws);
  a.M = M;
  a.N = N;
  a.K = K;
  a.NB = N / kBlockWeights;
  a.Lr = p.Lr;
  a.P = p.P;
  a.C = p.C;
  a.Kt = p.Kt;
  a.S = p.S;
  hipError_t err;
  switch (M) {
    case 1: err = launch_q8_m<1>(a, st); break;
    case 2: err = launch_q8_m<2>(a, st); break;
    case 3: err = launch_q8_m<3>(a, st); break;
    case 4: err = launch_q8_m<4>(a, st); break;
    case 5: err = launch_q8_m<5>(a, st); break;
    case 6: err = launch_q8_m<6>(a, st); break;
    case 7: err = launch_q8_m<7>(a, st); break;
    case 8: err = launch_q8_m<8>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess || p.S == 1) return err;
  return launch_gemv_reduce(a.part, y, M * N, p.S, st);
}

}  // namespace q4
