// Internal launcher declarations of the gfx950 MoE library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;

// ---- routing (route_kernels.hip)
int router_ksplit(int H);
hipError_t launch_router(const void* x, bool x_bf16, const float* wr, float* P, int T, int H,
                         int E, hipStream_t st);
hipError_t launch_select(const float* P, int ksplit, const float* bias, int T, int E, int G,
                         int topk_groups, int topk, int group_topn, int32_t* idx, float* gate,
                         float* gap, hipStream_t st);
int perm_chunks(int T);
hipError_t launch_permute(const int32_t* idx, int T, int K, int E, int S, uint64_t* masks,
                          int32_t* hist, int32_t* base, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* slot, int bm_a, int32_t* mt_a, int bm_b,
                          int32_t* mt_b, hipStream_t st);
hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, long long TK,
                              float gamma, hipStream_t st);

// ---- expert GEMMs and combine (gemm_kernels.hip)
template <typename TE> struct GemmArgs {
  const TE* a;                // GATED: x [T][K]; else staged H [rows][K]
  const TE* w0;               // W_gate (GATED) or W_down: [E+S][N][K]
  const TE* w1;               // W_up (GATED) or unused
  TE* out;                    // staged rows [rows][N]
  const int32_t* perm;        // [TK] token of each routed row
  const int32_t* counts;      // [E]
  const int32_t* offsets;     // [E+1]
  const int32_t* mt_start;    // [E+S+1] m-tile prefix for this kernel's tile height
  int E, n_exp, T, TK, N, K;
};

int gemm_tile_m();
template <typename TE>
hipError_t launch_gemm(const GemmArgs<TE>& g, bool gated, int max_mtiles, hipStream_t st);
template <typename TE>
hipError_t launch_combine(const TE* Y, const int32_t* slot, const float* gate, const TE* residual,
                          TE* y, int T, int K, int H, int TK, int S, hipStream_t st);

}  // namespace moe
