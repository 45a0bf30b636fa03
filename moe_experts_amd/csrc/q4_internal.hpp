// Host-side plans and launchers shared between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q4moe.h"

namespace q4 {

// ---- decode GEMV ---------------------------------------------------------
struct GemvPlan {
  bool mfma;        // matrix-core kernel (3 <= M <= 8) instead of the vector tiles
  int JW;           // matrix-core kernel: block columns per tile (4 or 8)
  int NW;           // matrix-core kernel: waves per workgroup (4 or 8)
  int LPB;          // lanes per block (1: whole block per lane, 2: half)
  int Jt;           // block columns per workgroup tile
  int Lr;           // lanes per row phase (Jt * LPB)
  int P;            // row phases per workgroup
  int C;            // column tiles
  int Kt;           // rows per workgroup
  int S;            // K splits
  size_t ws_bytes;  // workspace bytes: S * M * N floats of partials (0 when S == 1)
};

GemvPlan plan_gemv(int M, int N, int K);
hipError_t launch_gemv(const float* x, const uint8_t* B, float* y, int M, int N, int K,
                       void* ws, const GemvPlan& p, hipStream_t st);
// matrix-core variant (gemv_mfma_q4_0.hip): false when the shape does not suit it
bool plan_gemv_mfma(int M, int N, int K, GemvPlan& p);
hipError_t launch_gemv_mfma(const float* x, const uint8_t* B, float* y, int M, int N, int K,
                            void* ws, const GemvPlan& p, hipStream_t st);
// Q8_0 weights (gemv_q8_0.hip): the vector tiles' plan fields (LPB, Jt, Lr, P, C, Kt, S)
GemvPlan plan_gemv_q8(int M, int N, int K);
hipError_t launch_gemv_q8(const float* x, const uint8_t* B, float* y, int M, int N, int K,
                          void* ws, const GemvPlan& p, hipStream_t st);
// y[i] = sum over s < S of part[s * MN + i], in split order
hipError_t launch_gemv_reduce(const float* part, float* y, int MN, int S, hipStream_t st);

// ---- routed-expert MoE decode -------------------------------------------
struct MoePlan {
  int T, H, I, E, topk;
  int MC;                // pairs per vector work item (1 for a single token, else 2)
  int max_items;         // upper bound on vector work items (1 or 2 pairs of one expert)
  int max_mitems;        // upper bound on matrix-core work items (3 .. 8 pairs), 0 for T = 1
  int gu_Cm, dn_Cm;      // matrix-core column tiles (4 block columns each)
  int gu_C, gu_Kt, gu_S; // gate/up tiles: column tiles, rows per tile, K splits
  int dn_C, dn_Kt, dn_S; // down tiles
  // workspace layout (byte offsets)
  size_t off_items, off_n_items, off_mitems, off_gu_part, off_h, off_dn_part;
  size_t ws_bytes;
};

MoePlan plan_moe(int T, int H, int I, int E, int topk);
hipError_t launch_moe(const float* x, const uint8_t* Wg, const uint8_t* Wu, const uint8_t* Wd,
                      const int32_t* ids, const float* w, float* out, void* ws,
                      const MoePlan& p, hipStream_t st);

// ---- MoE router (router_moe.hip) ------------------------------------------
// K-split partial logits: bytes of workspace for the router kernels
size_t router_ws_bytes(int T, int H, int E);
hipError_t launch_router(const float* x, const float* Wr, float* logits, int32_t* ids, float* w,
                         int T, int H, int E, int topk, int n_shared, void* ws, hipStream_t st);

// ---- prefill GEMM --------------------------------------------------------
hipError_t launch_gemm(const uint16_t* X, const uint8_t* B, float* Y, int M, int N, int K,
                       hipStream_t st);
// Expert-grouped mode of the aligned prefill kernel (gemm_q4_0.hip): m-tiles
// (expert, first output row, rows <= kGemmRows) from a device list, X rows
// gathered through src (null: identity), B = consecutive K x N matrices.
// With B1 (a second set of matrices of the same shape) the workgroup
// contracts the same X tile with both and writes H = fp16(SiLU(X.B) * (X.B1))
// instead of Y.
constexpr int kGemmRows = Q4_MOE_PREFILL_TILE_ROWS;  // rows of one grouped m-tile
bool gemm_grouped_supported(int N, int K);
hipError_t launch_gemm_grouped(const uint16_t* X, int x_rows, const uint8_t* B, const uint8_t* B1,
                               size_t mat_bytes, float* Y, _Float16* H, int N, int K,
                               const int4* tiles, const int* n_tiles, int max_tiles,
                               const int32_t* src, hipStream_t st);

// ---- MoE prefill (moe_prefill.hip) -----------------------------------------
struct MoePrefillPlan {
  int max_tiles;  // upper bound on m-tiles over all experts
  size_t off_src, off_pos, off_tiles, off_counts, off_h, off_d, ws_bytes;
};
MoePrefillPlan plan_moe_prefill(int T, int H, int I, int E, int topk);
hipError_t launch_moe_prefill(const uint16_t* x16, const uint8_t* Wg, const uint8_t* Wu,
                              const uint8_t* Wd, const int32_t* ids, const float* w, float* out,
                              int T, int H, int I, int E, int topk, void* ws,
                              const MoePrefillPlan& p, hipStream_t st);

}  // namespace q4
