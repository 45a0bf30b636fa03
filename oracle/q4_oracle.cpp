/*
 * CPU oracle for Q4_0 fused-dequantization matmul and routed-expert MoE decode.
 * TEST INFRASTRUCTURE ONLY: see q4_oracle.h for scope, sources and pins.
 *
 * Built with g++ -O2 (no -ffast-math, single-threaded). Every step is the
 * plain definition from the pages, in double precision:
 *   - binary16 decode from the IEEE-754 bit layout (the article's
 *     fp16_to_fp32 is left undefined there; this is the exact map it names);
 *   - the §2.2 dequantize rule of the "2000-line C++ DeepSeek inference
 *     engine" article, element l of a block = (nibble(l) - 8) * d;
 *   - the §3.2/§3.4 (i, k, j) loop: for each output row i, for each k,
 *     C[i][:] += A[i][k] * w[k][:], with C cleared first;
 *   - SiLU(z) = z / (1 + exp(-z)) for the expert FFN (DeepSeek-V2 experts,
 *     KTransformers tutorial, "Optimization 3").
 */
#include "q4_oracle.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

constexpr int kBlockBytes = 18;   // 2-byte scale + 16 bytes of nibbles
constexpr int kBlockWeights = 32;
constexpr int kQ8BlockBytes = 34;  // 2-byte scale + 32 signed bytes

// Row v (length K, double) times the dequantized K x N matrix B, accumulated
// over k in ascending order: acc[n] = sum_k v[k] * w[k][n] and, when bnd is
// given, bnd[n] = sum_k |v[k] * w[k][n]|. Each product v[k] * w[k][n] is exact
// in double when v[k] came from a binary32 or binary16 value.
// Dequantizes one block of either format into 32 doubles.
typedef void (*DequantFn)(const uint8_t*, double*);

void row_times_matrix_fmt(const double* v, const uint8_t* B, int N, int K, double* acc,
                          double* bnd, DequantFn dequant, int block_bytes);

void row_times_matrix(const double* v, const uint8_t* B, int N, int K,
                      double* acc, double* bnd) {
  row_times_matrix_fmt(v, B, N, K, acc, bnd, oracle_dequant_block, kBlockBytes);
}

void row_times_matrix_fmt(const double* v, const uint8_t* B, int N, int K, double* acc,
                          double* bnd, DequantFn dequant, int block_bytes) {
  const int nb = N / kBlockWeights;
  for (int n = 0; n < N; ++n) {
    acc[n] = 0.0;
    if (bnd) bnd[n] = 0.0;
  }
  double w32[kBlockWeights];
  for (int k = 0; k < K; ++k) {
    const double a = v[k];
    const uint8_t* row = B + (size_t)k * (size_t)nb * block_bytes;
    for (int jb = 0; jb < nb; ++jb) {
      dequant(row + (size_t)jb * block_bytes, w32);
      double* accb = acc + (size_t)jb * kBlockWeights;
      double* bndb = bnd ? bnd + (size_t)jb * kBlockWeights : nullptr;
      for (int l = 0; l < kBlockWeights; ++l) {
        const double p = a * w32[l];
        accb[l] += p;
        if (bndb) bndb[l] += std::fabs(p);
      }
    }
  }
}

bool bad_matmul_args(const void* x, const uint8_t* B, int M, int N, int K,
                     const float* y) {
  return x == nullptr || B == nullptr || y == nullptr || M < 1 || N < 32 ||
         K < 1 || (N % kBlockWeights) != 0;
}

}  // namespace

extern "C" {

double oracle_fp16_to_double(uint16_t bits) {
  // binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
  const int sign = (bits >> 15) & 1;
  const int expo = (bits >> 10) & 0x1f;
  const int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = std::ldexp((double)frac, -24);  // zero or subnormal: 0.f * 2^-14
  } else if (expo == 31) {
    mag = (frac == 0) ? INFINITY : NAN;
  } else {
    mag = std::ldexp((double)(1024 + frac), expo - 25);  // 1.f * 2^(e-15)
  }
  return sign ? -mag : mag;
}

void oracle_dequant_block(const uint8_t* block18, double* out32) {
  // Little-endian scale in bytes 0..1, packed nibbles in bytes 2..17.
  const uint16_t dbits = (uint16_t)(block18[0] | (block18[1] << 8));
  const double d = oracle_fp16_to_double(dbits);
  const uint8_t* qs = block18 + 2;
  for (int l = 0; l < kBlockWeights; ++l) {
    const uint8_t packed = qs[l / 2];
    const int q = (l % 2 == 0) ? (packed & 0x0f) : (packed >> 4);
    out32[l] = (double)(q - 8) * d;
  }
}

int oracle_dequant_rows(const uint8_t* B, int N, int k0, int k1, float* out) {
  if (B == nullptr || out == nullptr || N < 32 || (N % kBlockWeights) != 0 ||
      k0 < 0 || k1 < k0)
    return -1;
  const int nb = N / kBlockWeights;
  double w32[kBlockWeights];
  for (int k = k0; k < k1; ++k) {
    for (int jb = 0; jb < nb; ++jb) {
      oracle_dequant_block(B + ((size_t)k * nb + jb) * kBlockBytes, w32);
      for (int l = 0; l < kBlockWeights; ++l)
        out[(size_t)(k - k0) * N + (size_t)jb * kBlockWeights + l] = (float)w32[l];
    }
  }
  return 0;
}

int oracle_q4_0_matmul(const float* x, const uint8_t* B, int M, int N, int K,
                       float* y, double* bound) {
  if (bad_matmul_args(x, B, M, N, K, y)) return -1;
  std::vector<double> v(K), acc(N), bnd(bound ? N : 0);
  for (int i = 0; i < M; ++i) {
    for (int k = 0; k < K; ++k) v[k] = (double)x[(size_t)i * K + k];
    row_times_matrix(v.data(), B, N, K, acc.data(), bound ? bnd.data() : nullptr);
    for (int n = 0; n < N; ++n) {
      y[(size_t)i * N + n] = (float)acc[n];
      if (bound) bound[(size_t)i * N + n] = bnd[n];
    }
  }
  return 0;
}

int oracle_q4_0_matmul_f16(const uint16_t* x16, const uint8_t* B, int M, int N,
                           int K, float* y, double* bound) {
  if (bad_matmul_args(x16, B, M, N, K, y)) return -1;
  std::vector<double> v(K), acc(N), bnd(bound ? N : 0);
  for (int i = 0; i < M; ++i) {
    for (int k = 0; k < K; ++k) v[k] = oracle_fp16_to_double(x16[(size_t)i * K + k]);
    row_times_matrix(v.data(), B, N, K, acc.data(), bound ? bnd.data() : nullptr);
    for (int n = 0; n < N; ++n) {
      y[(size_t)i * N + n] = (float)acc[n];
      if (bound) bound[(size_t)i * N + n] = bnd[n];
    }
  }
  return 0;
}

int oracle_moe_decode(const float* x, const uint8_t* Wg, const uint8_t* Wu,
                      const uint8_t* Wd, const int32_t* ids, const float* w,
                      int T, int H, int I, int E, int topk, float* out,
                      double* bound, double* h_out) {
  if (x == nullptr || Wg == nullptr || Wu == nullptr || Wd == nullptr ||
      ids == nullptr || w == nullptr || out == nullptr || T < 1 || H < 32 ||
      I < 32 || (H % kBlockWeights) != 0 || (I % kBlockWeights) != 0 || E < 1 ||
      topk < 1)
    return -1;
  // Bytes of one expert matrix (both H x I and I x H have H*I/32 blocks).
  const size_t mat_bytes = (size_t)H * (size_t)(I / kBlockWeights) * kBlockBytes;
  std::vector<double> xv(H), g(I), u(I), h(I), yd(H), bd(H);
  std::vector<double> acc(H), bacc(H);
  for (int t = 0; t < T; ++t) {
    for (int n = 0; n < H; ++n) { acc[n] = 0.0; bacc[n] = 0.0; }
    for (int k = 0; k < H; ++k) xv[k] = (double)x[(size_t)t * H + k];
    for (int j = 0; j < topk; ++j) {
      const int e = ids[(size_t)t * topk + j];
      double* hslot = h_out ? h_out + ((size_t)t * topk + j) * I : nullptr;
      if (e < 0 || e >= E) {  // an out-of-range id contributes nothing
        if (hslot) for (int n = 0; n < I; ++n) hslot[n] = 0.0;
        continue;
      }
      row_times_matrix(xv.data(), Wg + (size_t)e * mat_bytes, I, H, g.data(), nullptr);
      row_times_matrix(xv.data(), Wu + (size_t)e * mat_bytes, I, H, u.data(), nullptr);
      for (int n = 0; n < I; ++n) {
        const double silu = g[n] / (1.0 + std::exp(-g[n]));
        h[n] = silu * u[n];
        if (hslot) hslot[n] = h[n];
      }
      row_times_matrix(h.data(), Wd + (size_t)e * mat_bytes, H, I, yd.data(), bd.data());
      const double wt = (double)w[(size_t)t * topk + j];
      for (int n = 0; n < H; ++n) {
        acc[n] += wt * yd[n];
        bacc[n] += std::fabs(wt) * bd[n];
      }
    }
    for (int n = 0; n < H; ++n) {
      out[(size_t)t * H + n] = (float)acc[n];
      if (bound) bound[(size_t)t * H + n] = bacc[n];
    }
  }
  return 0;
}

int oracle_router_logits(const float* x, const float* Wr, int T, int H, int E,
                         float* logits, double* bound) {
  if (x == nullptr || Wr == nullptr || logits == nullptr || T < 1 || H < 1 || E < 1)
    return -1;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0, b = 0.0;
      for (int h = 0; h < H; ++h) {
        const double p = (double)x[(size_t)t * H + h] * (double)Wr[(size_t)e * H + h];
        acc += p;
        b += std::fabs(p);
      }
      logits[(size_t)t * E + e] = (float)acc;
      if (bound) bound[(size_t)t * E + e] = b;
    }
  return 0;
}

int oracle_router_topk(const float* logits, int T, int E, int topk, int n_shared,
                       int32_t* ids, float* w) {
  if (logits == nullptr || ids == nullptr || w == nullptr || T < 1 || E < 1 || topk < 1 ||
      topk > E || n_shared < 0)
    return -1;
  const int slots = topk + n_shared;
  std::vector<char> taken(E);
  std::vector<double> ex(topk);
  for (int t = 0; t < T; ++t) {
    const float* lg = logits + (size_t)t * E;
    int32_t* id = ids + (size_t)t * slots;
    float* wt = w + (size_t)t * slots;
    for (int e = 0; e < E; ++e) taken[e] = 0;
    // selection: repeatedly the largest remaining logit, lower index on ties
    for (int j = 0; j < topk; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e] || std::isnan(lg[e])) continue;
        if (best < 0 || lg[e] > lg[best]) best = e;
      }
      id[j] = best;
      if (best >= 0) taken[best] = 1;
    }
    // softmax over the chosen logits; the first chosen one is their maximum
    double sum = 0.0;
    for (int j = 0; j < topk; ++j) {
      ex[j] = id[j] >= 0 ? std::exp((double)lg[id[j]] - (double)lg[id[0]]) : 0.0;
      sum += ex[j];
    }
    for (int j = 0; j < topk; ++j) wt[j] = id[j] >= 0 ? (float)(ex[j] / sum) : 0.0f;
    for (int s = 0; s < n_shared; ++s) {
      id[topk + s] = E + s;
      wt[topk + s] = 1.0f;
    }
  }
  return 0;
}

void oracle_q8_0_dequant_block(const uint8_t* block34, double* out32) {
  const uint16_t bits = (uint16_t)(block34[0] | (block34[1] << 8));  // little-endian
  const double d = oracle_fp16_to_double(bits);
  for (int l = 0; l < kBlockWeights; ++l) {
    const int q = (int)(int8_t)block34[2 + l];  // two's complement byte
    out32[l] = (double)q * d;
  }
}

int oracle_q8_0_matmul(const float* x, const uint8_t* B, int M, int N, int K, float* y,
                       double* bound) {
  if (bad_matmul_args(x, B, M, N, K, y)) return -1;
  std::vector<double> v(K), acc(N), bnd(N);
  for (int m = 0; m < M; ++m) {
    for (int k = 0; k < K; ++k) v[k] = (double)x[(size_t)m * K + k];
    row_times_matrix_fmt(v.data(), B, N, K, acc.data(), bound ? bnd.data() : nullptr,
                         oracle_q8_0_dequant_block, kQ8BlockBytes);
    for (int n = 0; n < N; ++n) {
      y[(size_t)m * N + n] = (float)acc[n];
      if (bound) bound[(size_t)m * N + n] = bnd[n];
    }
  }
  return 0;
}

}  // extern "C"
