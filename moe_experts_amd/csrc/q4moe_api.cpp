// C ABI of libq4moe: host-side argument checks, workspace sizing and launch.
// Every entry point validates its arguments before touching the HIP runtime,
// so argument errors never enqueue work (and can be tested without a GPU).
#include "q4moe.h"

#include <hip/hip_runtime.h>

#include "q4_internal.hpp"

namespace {

// The kernels address one weight matrix and the activations with 32-bit byte
// offsets: each must stay below 2 GiB.
constexpr long long kMaxBytes = 0x7fffffffLL;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape limits of the decode GEMVs (block_bytes: 18 for Q4_0, 34 for Q8_0).
// The workspace-size functions apply them too, so a shape the entry point
// refuses never reaches a plan.
int check_gemv_shape(int M, int N, int K, int block_bytes) {
  if (M <= 0 || N <= 0 || K <= 0) return Q4_EINVAL;
  if (N % 32 != 0 || M > Q4_GEMV_MAX_M) return Q4_ESHAPE;
  if ((long long)K * (N / 32) * block_bytes > kMaxBytes || (long long)M * K * 4 > kMaxBytes ||
      (long long)M * N * 4 > kMaxBytes)
    return Q4_ETOOBIG;
  return Q4_OK;
}

int check_gemv(const float* x, const q4_0_block* B, const float* y, int M, int N, int K) {
  if (!x || !B || !y) return Q4_EINVAL;
  const int rc = check_gemv_shape(M, N, K, 18);
  if (rc != Q4_OK) return rc;
  if (!aligned(x, 4) || !aligned(y, 4) || !aligned(B, 2)) return Q4_EALIGN;
  return Q4_OK;
}

int check_gemv_q8(const float* x, const q8_0_block* B, const float* y, int M, int N, int K) {
  if (!x || !B || !y) return Q4_EINVAL;
  const int rc = check_gemv_shape(M, N, K, 34);
  if (rc != Q4_OK) return rc;
  if (!aligned(x, 4) || !aligned(y, 4) || !aligned(B, 2)) return Q4_EALIGN;
  return Q4_OK;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return Q4_OK;
  if (!ws || ws_bytes < need) return Q4_EWORKSPACE;
  if (!aligned(ws, 256)) return Q4_EALIGN;
  return Q4_OK;
}

int check_moe_shape(int T, int H, int I, int E, int topk) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return Q4_EINVAL;
  if (H % 32 != 0 || I % 32 != 0 || T > Q4_MOE_MAX_T || topk > Q4_MOE_MAX_TOPK ||
      E > Q4_MOE_MAX_E)
    return Q4_ESHAPE;
  if ((long long)H * (I / 32) * 18 > kMaxBytes) return Q4_ETOOBIG;  // one expert matrix
  return Q4_OK;
}

// The decode kernels address the activations, h and the split-K partial sums
// with 32-bit byte offsets: each must stay below 2 GiB.
int check_moe_sizes(const q4::MoePlan& p) {
  const long long np = (long long)p.T * p.topk;
  if ((long long)p.T * p.H * 4 > kMaxBytes || np * p.I * 4 > kMaxBytes ||
      2LL * p.gu_S * np * p.I * 4 > kMaxBytes || (long long)p.dn_S * np * p.H * 4 > kMaxBytes)
    return Q4_ETOOBIG;
  return Q4_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_EHIP; }

int check_router_shape(int T, int H, int E, int topk, int n_shared) {
  if (T <= 0 || H <= 0 || E <= 0 || topk <= 0 || n_shared < 0) return Q4_EINVAL;
  if (H % 4 != 0 || T > Q4_MOE_MAX_T || E > Q4_MOE_MAX_E || topk > E ||
      topk + n_shared > Q4_MOE_MAX_TOPK)
    return Q4_ESHAPE;
  if ((long long)E * H * 4 > kMaxBytes || (long long)T * H * 4 > kMaxBytes) return Q4_ETOOBIG;
  return Q4_OK;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

int check_prefill_shape(int T, int H, int I, int E, int topk) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return Q4_EINVAL;
  if (H % 128 != 0 || I % 128 != 0 || T > Q4_MOE_PREFILL_MAX_T || topk > Q4_MOE_MAX_TOPK ||
      E > Q4_MOE_MAX_E)
    return Q4_ESHAPE;
  const long long np = (long long)T * topk;
  if ((long long)H * (I / 32) * 18 > kMaxBytes || (long long)T * H * 2 > kMaxBytes ||
      np * I * 4 > kMaxBytes || np * H * 4 > kMaxBytes)
    return Q4_ETOOBIG;
  return Q4_OK;
}

// Layer workspace: router partials, logits, ids, weights, then the decode's.
struct LayerWs {
  size_t off_logits, off_ids, off_w, off_moe, bytes;
};

LayerWs layer_ws(int T, int H, int I, int E, int topk, int n_shared) {
  const int slots = topk + n_shared;
  LayerWs l;
  l.off_logits = align256(q4::router_ws_bytes(T, H, E));
  l.off_ids = l.off_logits + align256((size_t)T * E * sizeof(float));
  l.off_w = l.off_ids + align256((size_t)T * slots * sizeof(int32_t));
  l.off_moe = l.off_w + align256((size_t)T * slots * sizeof(float));
  l.bytes = l.off_moe + q4::plan_moe(T, H, I, E + n_shared, slots).ws_bytes;
  return l;
}

}  // namespace

extern "C" {

const char* q4_strerror(int status) {
  switch (status) {
    case Q4_OK: return "success";
    case Q4_EINVAL: return "invalid argument: null pointer or non-positive dimension";
    case Q4_ESHAPE: return "unsupported shape: N/H/I must be multiples of 32, M/T/topk/E within limits";
    case Q4_EALIGN:
      return "misaligned pointer (blocks 2 B, fp32/fp16 arrays 4 B, router x and Wr 16 B, "
             "workspace 256 B)";
    case Q4_EWORKSPACE: return "workspace missing or too small";
    case Q4_EHIP: return "HIP runtime error at launch";
    case Q4_ETOOBIG: return "size exceeds implementation limits";
    default: return "unknown status";
  }
}

size_t q4_0_gemv_workspace_bytes(int M, int N, int K) {
  if (check_gemv_shape(M, N, K, 18) != Q4_OK) return 0;
  return q4::plan_gemv(M, N, K).ws_bytes;
}

int q4_0_gemv(const float* x, const q4_0_block* B, float* y, int M, int N, int K, void* ws,
              size_t ws_bytes, void* stream) {
  int rc = check_gemv(x, B, y, M, N, K);
  if (rc != Q4_OK) return rc;
  const q4::GemvPlan p = q4::plan_gemv(M, N, K);
  rc = check_ws(ws, ws_bytes, p.ws_bytes);
  if (rc != Q4_OK) return rc;
  return from_hip(q4::launch_gemv(x, reinterpret_cast<const uint8_t*>(B), y, M, N, K, ws, p,
                                  static_cast<hipStream_t>(stream)));
}

size_t q8_0_gemv_workspace_bytes(int M, int N, int K) {
  if (check_gemv_shape(M, N, K, 34) != Q4_OK) return 0;
  return q4::plan_gemv_q8(M, N, K).ws_bytes;
}

int q8_0_gemv(const float* x, const q8_0_block* B, float* y, int M, int N, int K, void* ws,
              size_t ws_bytes, void* stream) {
  int rc = check_gemv_q8(x, B, y, M, N, K);
  if (rc != Q4_OK) return rc;
  const q4::GemvPlan p = q4::plan_gemv_q8(M, N, K);
  rc = check_ws(ws, ws_bytes, p.ws_bytes);
  if (rc != Q4_OK) return rc;
  return from_hip(q4::launch_gemv_q8(x, reinterpret_cast<const uint8_t*>(B), y, M, N, K, ws, p,
                                     static_cast<hipStream_t>(stream)));
}

int q4_0_gemm(const uint16_t* X, const q4_0_block* B, float* Y, int M, int N, int K,
              void* stream) {
  if (!X || !B || !Y || M <= 0 || N <= 0 || K <= 0) return Q4_EINVAL;
  if (N % 32 != 0) return Q4_ESHAPE;
  if ((long long)K * (N / 32) * 18 > kMaxBytes || (long long)M * K * 2 > kMaxBytes ||
      (long long)M * N * 4 > kMaxBytes)
    return Q4_ETOOBIG;
  if (!aligned(X, 4) || !aligned(Y, 4) || !aligned(B, 2)) return Q4_EALIGN;
  return from_hip(q4::launch_gemm(X, reinterpret_cast<const uint8_t*>(B), Y, M, N, K,
                                  static_cast<hipStream_t>(stream)));
}

size_t moe_q4_0_workspace_bytes(int T, int H, int I, int E, int topk) {
  if (check_moe_shape(T, H, I, E, topk) != Q4_OK) return 0;
  const q4::MoePlan p = q4::plan_moe(T, H, I, E, topk);
  return check_moe_sizes(p) == Q4_OK ? p.ws_bytes : 0;
}

int moe_q4_0_decode(const float* x, const q4_0_block* Wg, const q4_0_block* Wu,
                    const q4_0_block* Wd, const int32_t* topk_ids, const float* topk_w,
                    float* out, int T, int H, int I, int E, int topk, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!x || !Wg || !Wu || !Wd || !topk_ids || !topk_w || !out) return Q4_EINVAL;
  int rc = check_moe_shape(T, H, I, E, topk);
  if (rc != Q4_OK) return rc;
  if (!aligned(x, 4) || !aligned(out, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
      !aligned(Wg, 2) || !aligned(Wu, 2) || !aligned(Wd, 2))
    return Q4_EALIGN;
  const q4::MoePlan p = q4::plan_moe(T, H, I, E, topk);
  rc = check_moe_sizes(p);
  if (rc != Q4_OK) return rc;
  rc = check_ws(ws, ws_bytes, p.ws_bytes);
  if (rc != Q4_OK) return rc;
  return from_hip(q4::launch_moe(x, reinterpret_cast<const uint8_t*>(Wg),
                                 reinterpret_cast<const uint8_t*>(Wu),
                                 reinterpret_cast<const uint8_t*>(Wd), topk_ids, topk_w, out, ws,
                                 p, static_cast<hipStream_t>(stream)));
}

int moe_q4_0_route_layout(int T, int H, int I, int E, int topk, size_t* items_off,
                          size_t* counts_off, size_t* mitems_off) {
  if (!items_off || !counts_off || !mitems_off) return Q4_EINVAL;
  int rc = check_moe_shape(T, H, I, E, topk);
  if (rc != Q4_OK) return rc;
  const q4::MoePlan p = q4::plan_moe(T, H, I, E, topk);
  rc = check_moe_sizes(p);
  if (rc != Q4_OK) return rc;
  *items_off = p.off_items;
  *counts_off = p.off_n_items;
  *mitems_off = p.off_mitems;
  return Q4_OK;
}

size_t moe_router_workspace_bytes(int T, int H, int E) {
  if (check_router_shape(T, H, E, 1, 0) != Q4_OK) return 0;
  return q4::router_ws_bytes(T, H, E);
}

int moe_router_topk(const float* x, const float* Wr, float* logits, int32_t* topk_ids,
                    float* topk_w, int T, int H, int E, int topk, int n_shared, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!x || !Wr || !logits || !topk_ids || !topk_w) return Q4_EINVAL;
  int rc = check_router_shape(T, H, E, topk, n_shared);
  if (rc != Q4_OK) return rc;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(logits, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return Q4_EALIGN;
  rc = check_ws(ws, ws_bytes, q4::router_ws_bytes(T, H, E));
  if (rc != Q4_OK) return rc;
  return from_hip(q4::launch_router(x, Wr, logits, topk_ids, topk_w, T, H, E, topk, n_shared, ws,
                                    static_cast<hipStream_t>(stream)));
}

size_t moe_q4_0_layer_workspace_bytes(int T, int H, int I, int E, int topk, int n_shared) {
  if (check_router_shape(T, H, E, topk, n_shared) != Q4_OK ||
      check_moe_shape(T, H, I, E + n_shared, topk + n_shared) != Q4_OK ||
      check_moe_sizes(q4::plan_moe(T, H, I, E + n_shared, topk + n_shared)) != Q4_OK)
    return 0;
  return layer_ws(T, H, I, E, topk, n_shared).bytes;
}

int moe_q4_0_layer(const float* x, const float* Wr, const q4_0_block* Wg, const q4_0_block* Wu,
                   const q4_0_block* Wd, float* out, int T, int H, int I, int E, int topk,
                   int n_shared, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !Wr || !Wg || !Wu || !Wd || !out) return Q4_EINVAL;
  int rc = check_router_shape(T, H, E, topk, n_shared);
  if (rc != Q4_OK) return rc;
  rc = check_moe_shape(T, H, I, E + n_shared, topk + n_shared);
  if (rc != Q4_OK) return rc;
  rc = check_moe_sizes(q4::plan_moe(T, H, I, E + n_shared, topk + n_shared));
  if (rc != Q4_OK) return rc;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(out, 4) || !aligned(Wg, 2) ||
      !aligned(Wu, 2) || !aligned(Wd, 2))
    return Q4_EALIGN;
  const LayerWs l = layer_ws(T, H, I, E, topk, n_shared);
  rc = check_ws(ws, ws_bytes, l.bytes);
  if (rc != Q4_OK) return rc;
  const int slots = topk + n_shared;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* logits = reinterpret_cast<float*>(base + l.off_logits);
  int32_t* ids = reinterpret_cast<int32_t*>(base + l.off_ids);
  float* w = reinterpret_cast<float*>(base + l.off_w);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err =
      q4::launch_router(x, Wr, logits, ids, w, T, H, E, topk, n_shared, ws, st);
  if (err != hipSuccess) return Q4_EHIP;
  const q4::MoePlan p = q4::plan_moe(T, H, I, E + n_shared, slots);
  return from_hip(q4::launch_moe(x, reinterpret_cast<const uint8_t*>(Wg),
                                 reinterpret_cast<const uint8_t*>(Wu),
                                 reinterpret_cast<const uint8_t*>(Wd), ids, w, out,
                                 base + l.off_moe, p, st));
}

int moe_q4_0_prefill_route_layout(int T, int H, int I, int E, int topk, size_t* src_off,
                                  size_t* pos_off, size_t* tiles_off, size_t* counts_off) {
  if (!src_off || !pos_off || !tiles_off || !counts_off) return Q4_EINVAL;
  const int rc = check_prefill_shape(T, H, I, E, topk);
  if (rc != Q4_OK) return rc;
  const q4::MoePrefillPlan p = q4::plan_moe_prefill(T, H, I, E, topk);
  *src_off = p.off_src;
  *pos_off = p.off_pos;
  *tiles_off = p.off_tiles;
  *counts_off = p.off_counts;
  return Q4_OK;
}

size_t moe_q4_0_prefill_workspace_bytes(int T, int H, int I, int E, int topk) {
  if (check_prefill_shape(T, H, I, E, topk) != Q4_OK) return 0;
  return q4::plan_moe_prefill(T, H, I, E, topk).ws_bytes;
}

int moe_q4_0_prefill(const uint16_t* x16, const q4_0_block* Wg, const q4_0_block* Wu,
                     const q4_0_block* Wd, const int32_t* topk_ids, const float* topk_w,
                     float* out, int T, int H, int I, int E, int topk, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!x16 || !Wg || !Wu || !Wd || !topk_ids || !topk_w || !out) return Q4_EINVAL;
  int rc = check_prefill_shape(T, H, I, E, topk);
  if (rc != Q4_OK) return rc;
  if (!aligned(x16, 16) || !aligned(Wg, 4) || !aligned(Wu, 4) || !aligned(Wd, 4) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(out, 16))
    return Q4_EALIGN;
  const q4::MoePrefillPlan p = q4::plan_moe_prefill(T, H, I, E, topk);
  rc = check_ws(ws, ws_bytes, p.ws_bytes);
  if (rc != Q4_OK) return rc;
  return from_hip(q4::launch_moe_prefill(x16, reinterpret_cast<const uint8_t*>(Wg),
                                         reinterpret_cast<const uint8_t*>(Wu),
                                         reinterpret_cast<const uint8_t*>(Wd), topk_ids, topk_w,
                                         out, T, H, I, E, topk, ws, p,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
