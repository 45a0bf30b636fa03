// Decode GEMV over Q4_0 weights on the fp32 matrix cores, for 3 <= M <= 8:
// y[M x N] = x[M x K] . deq(B[K x N]).
//
// The operation is the fused dequantize-inside-the-inner-loop matmul of the
// "2000-line C++ DeepSeek inference engine" article (§3.4 matmul_q4_0). With
// several activation rows the work per weight grows with M while the bytes do
// not, and the fp32 FMA rate of the vector ALU sets the pace. Here the M-fold
// part runs on v_mfma_f32_4x4x1_16b_f32: sixteen independent 4x4 outer
// products per instruction, 64 multiply-adds per SIMD cycle, twice the vector
// FMA rate and with no rounding change (fp32 operands, fp32 accumulation).
//
// The tile (operands, phases, loads) is mfma_tile_accumulate in q4_mfma.hpp.
// Here a workgroup of NW = 4 or 8 waves owns JW = 4 or 8 block columns and a
// K range of Kt rows. The row phases are summed inside the wave with lane
// swaps (v_permlane32/16_swap, a fixed order) and across the waves through
// LDS, then the tile is written as one split-K partial (or straight to y when
// K is not split); the split-K sum is the same second kernel as the vector path.
#include "q4_internal.hpp"
#include "q4_mfma.hpp"

namespace q4 {
namespace {

// LDS of the GEMV tile: the activation rings, then the waves' phase sums
// (after the rings, so a wave that finishes early writes its sums at once).
template <int MH, int JW, int NW>
constexpr int mfma_lds_bytes() {
  return mfma_ring_bytes<MH, JW, NW>() + NW * MfmaShape<MH, JW, NW>::OUT * 4;
}

struct MfmaArgs {
  const float* __restrict__ x;
  const uint8_t* __restrict__ B;
  float* __restrict__ y;
  float* __restrict__ part;  // [S][M][N]
  int M, N, K, NB;
  int C, Kt, S;
};

// Sum the tile over its row phases and store it. Inside the wave the PW
// phases sit 16 lanes apart (PW = 4: lane bits 4 and 5; PW = 2: bit 5); a
// reduce-scatter with lane swaps leaves each lane NE accumulator quads, summed
// as (p0 + p2) + (p1 + p3), and the corrections are summed in the same order.
// Each wave then finishes its values (odd columns / 16, minus 8 * corr) into
// LDS, and the workgroup adds its NW waves in wave order.
template <int MH, int JW, int NW>
__device__ __forceinline__ void mfma_tile_store(v4f (&acc)[MH][8], float (&corr)[MH],
                                                float* smem, const MfmaArgs& a, int s, int j0,
                                                int lane, int wave, int q, int jj) {
  using SH = MfmaShape<MH, JW, NW>;
  constexpr int PW = SH::PW;
  // step 1 (distance 32): MH = 2 keeps h = lane bit 5, MH = 1 keeps i / 4
  float S1[4 * MH][4];
#pragma unroll
  for (int u = 0; u < 4 * MH; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S1[u][r] = MH == 2 ? swap_sum32(acc[0][u][r], acc[MH - 1][u][r])
                         : swap_sum32(acc[0][u][r], acc[0][(u + 4) & 7][r]);
  float R[SH::NE][4];
  if constexpr (PW == 2) {
#pragma unroll
    for (int u = 0; u < SH::NE; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) R[u][r] = S1[u][r];
  } else {
    // step 2 (distance 16): lane bit 4 keeps the lower or upper half of the
    // remaining i range (MH = 2: i vs i + 4; MH = 1: u vs u + 2)
    constexpr int D2 = MH == 2 ? 4 : 2;
#pragma unroll
    for (int u = 0; u < SH::NE; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) R[u][r] = swap_sum16(S1[u][r], S1[u + D2][r]);
  }
#pragma unroll
  for (int h = 0; h < MH; ++h) {
    corr[h] += __shfl_xor(corr[h], 32);
    if constexpr (PW == 4) corr[h] += __shfl_xor(corr[h], 16);
  }
  // this lane's activation half and first column: i = ibase + u
  const int hsel = MH == 2 ? (lane >> 5) : 0;
  int ibase;
  if constexpr (PW == 2) ibase = MH == 2 ? 0 : 4 * (lane >> 5);
  else ibase = MH == 2 ? 4 * ((lane >> 4) & 1) : 4 * (lane >> 5) + 2 * ((lane >> 4) & 1);
  // corrections of rows m = r + 4 * hsel for this block: lane q = r of the quad
  const float ch = hsel ? corr[MH - 1] : corr[0];
  float cb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) cb[r] = __shfl(ch, (lane & ~3) | r);

  float* sums = smem + mfma_ring_bytes<MH, JW, NW>() / 4;
  float* red = sums + wave * SH::OUT;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = r + 4 * hsel;
    float v[SH::NE];
#pragma unroll
    for (int u = 0; u < SH::NE; ++u)
      v[u] = ((u & 1) ? R[u][r] * 0.0625f : R[u][r]) - 8.0f * cb[r];
    float* dst = red + m * SH::TW + jj * 32 + 8 * q + ibase;
    if constexpr (SH::NE == 2) {
      *reinterpret_cast<float2*>(dst) = float2{v[0], v[1]};
    } else {
#pragma unroll
      for (int u = 0; u < SH::NE; u += 4)
        *reinterpret_cast<float4*>(dst + u) = float4{v[u], v[u + 1], v[u + 2], v[u + 3]};
    }
  }
  __syncthreads();
  // Every LDS read of the sum is issued before the first store.
  constexpr int IT = SH::OUT / SH::NT;
  static_assert(IT * SH::NT == SH::OUT, "whole passes over the tile");
  float* out = (a.S == 1) ? a.y : a.part + (size_t)s * a.M * a.N;
  const int n0 = j0 * kBlockWeights;
  float sum[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int o = it * SH::NT + threadIdx.x;
    sum[it] = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum[it] += sums[w * SH::OUT + o];
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int o = it * SH::NT + threadIdx.x;
    const int m = o / SH::TW;
    const int n = o - m * SH::TW;
    if (m < a.M && n0 + n < a.N) out[(size_t)m * a.N + n0 + n] = sum[it];
  }
}

template <int MH, int JW, int NW>
__global__ __launch_bounds__(NW * kWaveSize) void gemv_q4_0_mfma_kernel(MfmaArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int L = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int c = L % a.C;
  const int s = L / a.C;
  const int lane = threadIdx.x % kWaveSize;
  const int wave = threadIdx.x / kWaveSize;
  const int q = lane & 3;
  const int jj = (lane >> 2) % JW;
  const int j0 = c * JW;
  const int k0 = s * a.Kt;
  const int rows = min(a.Kt, a.K - k0);
  int xoff[4 * MH];
#pragma unroll
  for (int m = 0; m < 4 * MH; ++m) xoff[m] = m * a.K;
  MfmaTileGeom g{a.B, a.NB, j0, k0, rows};
  v4f acc[MH][8];
  float corr[MH];
  mfma_tile_accumulate<MH, JW, NW>(g, a.x, (uint32_t)(4 * a.M * a.K), xoff, a.M, smem, acc, corr);

  mfma_tile_store<MH, JW, NW>(acc, corr, smem, a, s, j0, lane, wave, q, jj);
}

template <int MH, int JW, int NW>
hipError_t launch_mfma_t(const MfmaArgs& a, hipStream_t st) {
  constexpr int lds = mfma_lds_bytes<MH, JW, NW>();
  hipLaunchKernelGGL((gemv_q4_0_mfma_kernel<MH, JW, NW>), dim3(a.C * a.S), dim3(NW * kWaveSize),
                     lds, st, a);
  return hipGetLastError();
}

template <int MH>
hipError_t launch_mfma_m(const MfmaArgs& a, int JW, int NW, hipStream_t st) {
  if (NW == 8) return JW == 4 ? launch_mfma_t<MH, 4, 8>(a, st) : launch_mfma_t<MH, 8, 8>(a, st);
  return JW == 4 ? launch_mfma_t<MH, 4, 4>(a, st) : launch_mfma_t<MH, 8, 4>(a, st);
}

// Bytes between the tile start and the furthest row offset a lane forms
// (rows of kMfmaSets batches past the tile's last batch): must stay below 2^31.
uint64_t mfma_offset_span(int Kt, int JW, int NW, uint32_t pitch) {
  const int PT = NW * (16 / JW);
  const int rows_pad = ((Kt + PT - 1) / PT + kMfmaRB - 1) / kMfmaRB * kMfmaRB * PT;
  return (uint64_t)(rows_pad + kMfmaSets * kMfmaRB * PT) * pitch;
}

}  // namespace

// Plan: block-column width JW (4 or 8), waves per workgroup NW (4 or 8) and
// K split S, for n = C*S workgroups. Workgroups share the CUs evenly only in
// whole rounds of 256, so the plan takes the largest fraction of a whole round
// used, n / (256 * ceil(n / 256)), over the candidates with at most 2048
// waves in all (two per SIMD; measured: more waves only add partial sums) and
// at least 64 rows per tile; ties go to more waves, then to fewer splits (less
// partial-sum traffic).
bool plan_gemv_mfma(int M, int N, int K, GemvPlan& p) {
  if (M < 3 || M > 8) return false;
  const int NB = N / kBlockWeights;
  const uint32_t pitch = (uint32_t)NB * kBlockBytes;
  double best = -1.0;
  for (int NW : {4, 8})
    for (int JW : {4, 8}) {
      // 8-block tiles (144-byte row segments) read faster than 4-block ones:
      // same-box A/B on the dense shapes, 11008 x 4096 at batch 4 13.9 -> 12.5
      // us and at batch 8 17.0 -> 16.1 us; so when the matrix splits into whole
      // 8-block tiles only those are planned
      if (NB % 8 == 0 && JW != 8) continue;
      const int PT = NW * (16 / JW);
      const int C = (NB + JW - 1) / JW;
      int last_S = -1;
      for (int s = 1; s <= K; ++s) {
        int kt = (K + s - 1) / s;
        kt = (kt + PT - 1) / PT * PT;
        const int S = (K + kt - 1) / kt;
        if (S == last_S) continue;
        last_S = S;
        const long long n = (long long)C * S;
        if (n * NW > 2048) break;
        if (S > 1 && kt < 64) break;
        if (mfma_offset_span(kt, JW, NW, pitch) >= (1ull << 31)) continue;
        const double rounds = (double)((n + 255) / 256);
        const double score = (double)n / (256.0 * rounds) + 1e-7 * (double)(n * NW) - 1e-9 * S;
        if (score > best) {
          best = score;
          p.JW = JW;
          p.NW = NW;
          p.C = C;
          p.Kt = kt;
          p.S = S;
        }
      }
    }
  if (best < 0.0) return false;
  p.mfma = true;
  p.LPB = 0;
  p.Jt = p.JW;
  p.Lr = 0;
  p.P = p.NW * (16 / p.JW);
  p.ws_bytes = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
  return true;
}

hipError_t launch_gemv_mfma(const float* x, const uint8_t* B, float* y, int M, int N, int K,
                            void* ws, const GemvPlan& p, hipStream_t st) {
  MfmaArgs a;
  a.x = x;
  a.B = B;
  a.y = y;
  a.part = static_cast<float*>(ws);
  a.M = M;
  a.N = N;
  a.K = K;
  a.NB = N / kBlockWeights;
  a.C = p.C;
  a.Kt = p.Kt;
  a.S = p.S;
  const hipError_t err =
      M > 4 ? launch_mfma_m<2>(a, p.JW, p.NW, st) : launch_mfma_m<1>(a, p.JW, p.NW, st);
  if (err != hipSuccess || p.S == 1) return err;
  return launch_gemv_reduce(a.part, y, M * N, p.S, st);
}

}  // namespace q4
