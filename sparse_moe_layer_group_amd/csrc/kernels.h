// Internal launcher declarations of the gfx950 MoE library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;

// ---- routing (route_kernels.hip)
int router_ksplit(int H);                                // partials the workspace holds
int router_partials(int T, int H, int E, bool x_bf16);  // partials launch_router writes
size_t router_split_bytes(int H, int E);
hipError_t launch_router(const void* x, bool x_bf16, const float* wr, bf16_t* wt3, float* P,
                         int T, int H, int E, hipStream_t st);
hipError_t launch_select(const float* P, int ksplit, const float* bias, int T, int E, int G,
                         int topk_groups, int topk, int group_topn, int32_t* idx, float* gate,
                         float* gap, hipStream_t st);
int perm_chunks(int T);
hipError_t launch_permute(const int32_t* idx, int T, int K, int E, int S, uint64_t* masks,
                          int32_t* hist, int32_t* base, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* slot, int stream_max, int32_t* chunk_start,
                          int bm, int32_t* mt_start, hipStream_t st);
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

// weight-streaming GEMM (stream_gemm.hip), bf16 only
struct StreamArgs {
  const bf16_t* a;            // GATED: x [T][K]; else staged H [rows][K]
  const bf16_t* w0;           // W_gate or W_down [E+S][N][K]
  const bf16_t* w1;           // W_up (GATED)
  bf16_t* out;                // staged rows [rows][N]
  const int32_t* perm;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* chunk_start; // [E+S+1] prefix of kStreamChunk-row chunks of streamed experts
  int E, n_exp, T, TK, N, K;
  bf16_t* out_g;              // mode 2 (gated, for the backward): G and U too, [rows][N]
  bf16_t* out_u;
};
constexpr int kMaxStreamExperts = 1024;  // n_exp bound of the streaming GEMM's LDS tables
constexpr int kStreamChunk = 64;         // token rows per task of the streaming GEMM
// mode 0: out = A W0^T; 1: out = SiLU(x W0^T) * (x W1^T), x rows gathered
// through perm; 2: as 1, and the two products also to out_g and out_u
hipError_t launch_stream_gemm(const StreamArgs& g, int mode, int n_blocks, hipStream_t st);
int stream_waves_per_block(int mode);  // waves of one workgroup of launch_stream_gemm

// LDS-tiled GEMM for experts with many rows (tile_gemm.hip), bf16 only;
// kTileM-row tiles, gate/up column tiles of 128, down column tiles of 256
struct TileArgs {
  const bf16_t* a;
  const bf16_t* w0;
  const bf16_t* w1;
  bf16_t* out;
  const int32_t* perm;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* mt_start;    // [E+S+1] prefix of kTileM-row tiles of tiled experts
  int E, n_exp, T, TK, N, K;
  bf16_t* out_g;              // mode 2 (gated, for the backward): G and U too, [rows][N]
  bf16_t* out_u;
};
constexpr int kTileM = 320;  // token rows per tile of the tiled GEMM (2 waves of 5 x 32 rows)
hipError_t launch_tile_gemm(const TileArgs& g, int mode, int max_mtiles, hipStream_t st);  // modes as above

int gemm_tile_m();
template <typename TE>
hipError_t launch_gemm(const GemmArgs<TE>& g, bool gated, int max_mtiles, int max_blocks,
                       hipStream_t st);
template <typename TE>
hipError_t launch_combine(const TE* Y, const int32_t* slot, const float* gate, const TE* residual,
                          TE* y, int T, int K, int H, int TK, int S, hipStream_t st);

// ---- FP8 E4M3 path (fp8_kernels.hip)
// 1x128 activation quantisation: x bf16 [rows][C] -> codes [rows][C], scales [rows][C/128]
hipError_t launch_quant_1x128(const bf16_t* x, long long rows, int C, uint8_t* q, float* scales,
                              hipStream_t st);
// block-scaled tiled GEMM, kTileM8-row tiles.  GATED: A = quantised x (rows
// gathered through perm), out8/out_s = quantised SwiGLU output H and its 1x128
// scales.  Down: A = quantised H, out16 = bf16 staged rows.
struct TileArgs8 {
  const uint8_t* a;           // E4M3 codes [rows][K]
  const float* as;            // A scales [rows][K/128]
  const uint8_t* w0;          // W_gate or W_down codes [E+S][N][K]
  const uint8_t* w1;          // W_up (GATED)
  const float* ws0;           // weight block scales [E+S][N/128][K/128]
  const float* ws1;           // W_up block scales (GATED)
  uint8_t* out8;              // GATED: H codes [rows][N]
  bf16_t* out16;              // down: staged rows [rows][N]
  float* out_s;               // GATED: H scales [rows][N/128]
  const int32_t* perm;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* mt_start;    // [E+S+1] prefix of kTileM8-row tiles
  int E, n_exp, T, TK, N, K;
};
constexpr int kTileM8 = 192;  // token rows per tile of the fp8 GEMM
hipError_t launch_tile_gemm_fp8(const TileArgs8& g, bool gated, int max_mtiles, hipStream_t st);

// ---- sequence-wise balance loss (balance_kernels.hip)
int balance_chunks(int seq_len);  // token chunks per sequence in the reduction
hipError_t launch_balance(const float* P, int ksplit, int T, int E, int K, int seq_len,
                          float alpha, float* sn, int32_t* ids, double* psum, int32_t* pcnt,
                          float* loss, float* f, float* p, hipStream_t st);

}  // namespace moe
