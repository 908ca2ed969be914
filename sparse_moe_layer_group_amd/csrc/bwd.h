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
  int32_t* mt;                // [E+S+1] row-tile prefix of the dgrad GEMM
  const bf16_t* w_gate;       // [E+S][I][H]
  const bf16_t* w_up;         // [E+S][I][H]
  const bf16_t* w_down;       // [E+S][H][I]
  bf16_t* xst;                // [rows][H] x in staged-row order
  bf16_t* gst;                // [rows][I] recomputed X W_gate^T
  bf16_t* ust;                // [rows][I] recomputed X W_up^T
  bf16_t* hst;                // [rows][I] recomputed SiLU(G) * U
  bf16_t* yst;                // [rows][H] recomputed expert outputs
  bf16_t* dyst;               // [rows][H] expert output gradients
  bf16_t* dgst;               // [rows][I]
  bf16_t* dust;               // [rows][I]
  bf16_t* dxst;               // [rows][H] expert input gradients
  float* dg;                  // [T*K] gate gradients
  float* dl;                  // [T*K] logit gradients of the chosen experts
  float* dlst;                // [T*K] the same per routed staged row
  float* wrt;                 // [E][H] W_r transposed
  float* dwrt;                // [E][H] dW_r transposed
  float* dw_gate;             // [E+S][I][H] float32 out
  float* dw_up;               // [E+S][I][H] float32 out
  float* dw_down;             // [E+S][H][I] float32 out
  int E, n_exp, T, TK, K, H, I;
};

int bwd_max_row_tiles(int T, int K, int E, int S);

// One stage of the backward (0 gather x, 1 SwiGLU, 2 combine backward,
// 3 router backward, 4 dH GEMM, 5 dX GEMM, 6 weight-gradient GEMMs,
// 7 dW_r, 8 dx); P / ks: router partials and their count.
hipError_t launch_backward_kernels(const BwdArgs& g, const float* P, int ks, const int32_t* idx,
                                   const int32_t* slot, const float* gate, const float* w_router,
                                   const bf16_t* dy, bf16_t* dx, float* dw_router, hipStream_t st,
                                   int stage);

}  // namespace moe
