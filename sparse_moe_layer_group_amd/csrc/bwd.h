// Internal declarations of the layer backward (bwd_kernels.hip); not part of the C ABI.
#pragma once

#include "common.h"

namespace moe {

// Buffers of the backward; rows are staged rows (routed experts in expert
// order, then the shared expert's T rows), all row-major.
struct BwdArgs {
  const bf16_t* x;            // [T][H]
  const int32_t* perm;        // [T*K] token of each routed staged row
  const int32_t* counts;      // [E]
  const int32_t* offsets;     // [E+1]
  int32_t* mt;                // [E+S+1] prefix of 128-row tiles
  int32_t* mtd;               // [E+S+1] prefix of the large-tile dgrad GEMM's row tiles, or null
  const bf16_t* w_gate;       // [E+S][I][H]
  const bf16_t* w_up;         // [E+S][I][H]
  const bf16_t* w_down;       // [E+S][H][I]
  bf16_t* xst;                // [rows][H] x in staged-row order
  bf16_t* gst;                // [rows][I] recomputed X W_gate^T (the forward's gated GEMM)
  bf16_t* ust;                // [rows][I] recomputed X W_up^T
  bf16_t* hst;                // [rows][I] recomputed SiLU(G) * U
  bf16_t* yst;                // [rows][H] recomputed expert outputs
  bf16_t* dyst;               // [rows][H] expert output gradients
  bf16_t* dgst;               // [rows][I]
  bf16_t* dust;               // [rows][I]
  bf16_t* dxst;               // [rows][H] expert input gradients
  float* dg;                  // [T*K] gate gradients
  float* dgp;                 // [I/256][rows] per-tile row sums of dH * H (gate gradients
                              // without recomputing Y), or null: dg from the recomputed Y
  float* dl;                  // [T*K] logit gradients of the chosen experts
  float* dlst;                // [T*K] the same per routed staged row
  float* wrt;                 // [E][H] W_r transposed
  float* dwrt;                // [E][H] dW_r transposed
  float* dw_gate;             // [E+S][I][H] float32 out
  float* dw_up;               // [E+S][I][H] float32 out
  float* dw_down;             // [E+S][H][I] float32 out
  int E, n_exp, T, TK, K, H, I;
  int wg_xcd;                 // decode-sized batch (at most 64 rows per routed expert): the
                              // per-tile weight-gradient kernel, else the persistent one
};

int bwd_max_row_tiles(int T, int K, int E, int S);

// One stage of the backward (0 gather x, 2 combine backward and tile prefixes,
// 3 router backward, 4 dH GEMM, 5 dX GEMM, 6 weight-gradient GEMMs, 7 dW_r,
// 8 dx; G, U and H come from the forward's gated GEMM); P / ks: router
// partials and their count.  With dgp, stage 3 runs after stage 4.
hipError_t launch_backward_kernels(const BwdArgs& g, const float* P, int ks, const int32_t* idx,
                                   const int32_t* slot, const float* gate, const float* w_router,
                                   const bf16_t* dy, bf16_t* dx, float* dw_router, hipStream_t st,
                                   int stage);

// ---- E4M3 backward (bwd_fp8_kernels.hip)

// One grouped E4M3 GEMM launch (see f8_gemm_kernel): sources 0 and 1 (the
// second only for dX), output float32 or bf16.
struct F8GemmArgs {
  const uint8_t* a0;
  const uint8_t* a1;
  const float* as0;
  const float* as1;
  const uint8_t* b0;
  const uint8_t* b1;
  const float* bs0;
  const float* bs1;
  void* out;
  const int32_t* perm;     // A rows gathered through perm (row grouping), or null
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* mt;       // [n_exp+1] prefix of 128-row tiles
  const int32_t* kp;       // [n_exp+1] prefix of rows rounded up to 128
  int E, n_exp, T, TK, M, N, K;
  int xcd;                 // K grouping: routed tiles in XCD-contiguous order
};

// Buffers of the E4M3 backward; rows are staged rows.
struct BwdArgs8 {
  const bf16_t* x;            // [T][H]
  const bf16_t* dy;           // [T][H]
  const int32_t* perm;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* slot;
  const float* gate;          // [T*K]
  const uint8_t* xq;          // [T][H] x in E4M3, scales [T][H/128]
  const float* xs;
  const uint8_t* w_gate;      // [E+S][I][H] codes, block scales [E+S][I/128][H/128]
  const uint8_t* w_up;
  const uint8_t* w_down;      // [E+S][H][I], scales [E+S][H/128][I/128]
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  float* f32a;                // [rows][I] G, then dH
  float* f32b;                // [rows][I] U
  uint8_t* gq;                // cached SwiGLU input [rows][I], scales [rows][I/128]
  float* gs;
  uint8_t* uq;
  float* us;
  uint8_t* hq;                // H for the down GEMM [rows][I], scales [rows][I/128]
  float* hs;
  bf16_t* yst;                // [rows][H] recomputed expert outputs
  uint8_t* dyq;               // [rows][H], scales [rows][H/128]
  float* dys;
  float* rowgate;             // [T*K] gate of each routed staged row
  float* dg32;                // [rows][I]
  float* du32;
  uint8_t* dgq;               // [rows][I], scales [rows][I/128]
  float* dgs;
  uint8_t* duq;
  float* dus;
  bf16_t* dxst;               // [rows][H]
  int32_t* mt;                // [E+S+1]
  int32_t* kp;                // [E+S+1]
  uint8_t* dyT;               // 128x1 operands: per expert [C][Kp_e], scales [C][Kp_e/128]
  float* dysT;
  uint8_t* xT;
  float* xsT;
  uint8_t* hT;
  float* hsT;
  uint8_t* dgT;
  float* dgsT;
  uint8_t* duT;
  float* dusT;
  float* dw_gate;
  float* dw_up;
  float* dw_down;
  int E, n_exp, T, TK, K, H, I;
};

int f8_max_row_tiles(int T, int K, int E, int S);

// One stage of the E4M3 backward: 1 prefixes, 2 G, U, H and Y, 3 Q(dY), 4 dH
// and the SwiGLU backward, 5 dX, 6 the 128x1 operands, 7 weight gradients.
hipError_t launch_backward_fp8(const BwdArgs8& g, hipStream_t st, int stage);

}  // namespace moe
