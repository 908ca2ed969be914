// Grouped expert GEMMs and the gated combine for gfx950.
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §1.1 (SwiGLU
// experts, three matrices) and §1.3 Eq 12 (shared expert plus gate-weighted
// routed experts).
//
// Rows are the expert-ordered assignments: routed expert e owns staging rows
// offsets[e] .. offsets[e+1]-1 (tokens perm[row]); shared expert s owns rows
// TK + s*T .. TK + (s+1)*T - 1 (tokens in order).  A launch covers every
// (m-tile, n-tile) of every expert; m-tiles are numbered by the prefix table
// mt_start[0..E+S] built on the device, so no host synchronisation is needed.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

template <typename TE> struct Mfma;

// bf16: v_mfma_f32_16x16x32_bf16, each lane feeds 8 consecutive k of one row
template <> struct Mfma<bf16_t> {
  static constexpr int KI = 32;
  static constexpr int EPL = 8;
  MOE_DEV static f32x4 mma(const bf16_t* a, const bf16_t* b, f32x4 c) {
    bf16x8 av = *reinterpret_cast<const bf16x8*>(a);
    bf16x8 bv = *reinterpret_cast<const bf16x8*>(b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
  }
};

// f32: v_mfma_f32_16x16x4_f32, each lane feeds one k of one row
template <> struct Mfma<float> {
  static constexpr int KI = 4;
  static constexpr int EPL = 1;
  MOE_DEV static f32x4 mma(const float* a, const float* b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, c, 0, 0, 0);
  }
};

// Find the expert owning global m-tile `mt`: the largest e with mt_start[e] <= mt.
MOE_DEV int find_expert(const int32_t* __restrict__ mt_start, int n, int mt) {
  int lo = 0, hi = n - 1;  // invariant: mt_start[lo] <= mt < mt_start[hi + 1]
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (mt_start[mid] <= mt) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ============================================================================
// Tiled grouped GEMM, v1: block 256 threads = 2 x 2 waves, tile BM x BN, K in
// steps of BK through LDS with register prefetch of the next K step.
//   GATED:  A = gathered x rows, B = W_gate[e] and W_up[e] rows n0..n0+BN,
//           out = SiLU(A W_gate^T) * (A W_up^T)          (hidden -> inter)
//   !GATED: A = staged H rows, B = W_down[e] rows, out = A W_down^T (inter -> hidden)
// ============================================================================

// global -> registers: A rows through the row-source table, B rows of the expert
template <typename TE, bool GATED, int BN, int BK, int A_CHUNKS, int B_CHUNKS>
MOE_DEV void gemm_load(u32x4 (&ra)[A_CHUNKS], u32x4 (&rb)[B_CHUNKS], const TE* __restrict__ a,
                       const int* tok_s, const TE* Wb0, const TE* Wb1, int n0, int K, int k0,
                       int tid) {
  constexpr int CE = 16 / sizeof(TE);
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + i * 256;
    const int r = c / (BK / CE), kc = (c % (BK / CE)) * CE;
    const int src = tok_s[r];
    ra[i] = (src >= 0) ? *reinterpret_cast<const u32x4*>(a + (size_t)src * K + k0 + kc)
                       : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int c = tid + i * 256;
    const int r = c / (BK / CE), kc = (c % (BK / CE)) * CE;
    const TE* src = (GATED && r >= BN) ? (Wb1 + (size_t)(n0 + r - BN) * K)
                                       : (Wb0 + (size_t)(n0 + r) * K);
    rb[i] = *reinterpret_cast<const u32x4*>(src + k0 + kc);
  }
}

template <typename TE, bool GATED, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs<TE> g) {
  using M = Mfma<TE>;
  constexpr int CE = 16 / sizeof(TE);            // elements per 16-byte chunk
  constexpr int STRIDE = BK + CE;                // LDS row stride (elements), +16 bytes
  constexpr int NB = GATED ? 2 * BN : BN;        // B rows staged per K step
  constexpr int A_CHUNKS = BM * BK / CE / 256;
  constexpr int B_CHUNKS = NB * BK / CE / 256;
  constexpr int MT = BM / 2 / 16, NT = BN / 2 / 16;
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) TE A_s[BM * STRIDE];
  __shared__ __attribute__((aligned(16))) TE B_s[NB * STRIDE];
  __shared__ int tok_s[BM];

  const int n_nt = g.N / BN;
  const int n_tasks = g.mt_start[g.n_exp] * n_nt;
  const int K = g.K;
  for (int task = blockIdx.x; task < n_tasks; task += gridDim.x) {  // uniform per block
  const int mt = task / n_nt;
  const int e = find_expert(g.mt_start, g.n_exp, mt);
  const bool shared = e >= g.E;
  const int cnt = shared ? g.T : g.counts[e];
  const int row_base = shared ? g.TK + (e - g.E) * g.T : g.offsets[e];
  const int m0 = (mt - g.mt_start[e]) * BM;
  const int rows = min(BM, cnt - m0);
  const int n0 = (task - mt * n_nt) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // A row sources
  for (int r = tid; r < BM; r += 256) {
    int src = -1;
    if (r < rows) {
      int row = row_base + m0 + r;
      if (GATED) src = shared ? (m0 + r) : g.perm[row];
      else src = row;
    }
    tok_s[r] = src;
  }
  __syncthreads();

  const TE* Wb0 = g.w0 + (size_t)e * g.N * K;
  const TE* Wb1 = GATED ? g.w1 + (size_t)e * g.N * K : nullptr;

  u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
  f32x4 acc0[MT][NT], acc1[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc0[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int fr = lane & 15, fk = (lane >> 4) * M::EPL;
  gemm_load<TE, GATED, BN, BK, A_CHUNKS, B_CHUNKS>(ra, rb, g.a, tok_s, Wb0, Wb1, n0, K, 0, tid);
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + i * 256;
      const int r = c / (BK / CE), kc = (c % (BK / CE)) * CE;
      *reinterpret_cast<u32x4*>(&A_s[r * STRIDE + kc]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int c = tid + i * 256;
      const int r = c / (BK / CE), kc = (c % (BK / CE)) * CE;
      *reinterpret_cast<u32x4*>(&B_s[r * STRIDE + kc]) = rb[i];
    }
    __syncthreads();
    if (k0 + BK < K)
      gemm_load<TE, GATED, BN, BK, A_CHUNKS, B_CHUNKS>(ra, rb, g.a, tok_s, Wb0, Wb1, n0, K, k0 + BK,
                                                       tid);
#pragma unroll
    for (int kk = 0; kk < BK; kk += M::KI) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const TE* ap = &A_s[(wm * (BM / 2) + i * 16 + fr) * STRIDE + kk + fk];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int br = wn * (BN / 2) + j * 16 + fr;
          acc0[i][j] = M::mma(ap, &B_s[br * STRIDE + kk + fk], acc0[i][j]);
          if (GATED) acc1[i][j] = M::mma(ap, &B_s[(BN + br) * STRIDE + kk + fk], acc1[i][j]);
        }
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+q, column lane%16 of each 16x16 tile
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int r = wm * (BM / 2) + i * 16 + 4 * (lane >> 4) + q;
        int n = n0 + wn * (BN / 2) + j * 16 + (lane & 15);
        if (r < rows) {
          float v = GATED ? siluf(acc0[i][j][q]) * acc1[i][j][q] : acc0[i][j][q];
          g.out[(size_t)(row_base + m0 + r) * g.N + n] = from_f32<TE>(v);
        }
      }
  __syncthreads();  // tok_s is rewritten by the next task
  }
}

// ============================================================================
// Gated combine: y[t] = sum_s Y[TK + s*T + t] + sum_k gate[t][k] * Y[slot[t*K+k]]
// (+ residual), float32 accumulation, shared experts first then k ascending
// (the chosen ids ascend).  A 128-thread block covers 128 16-byte vectors of
// one token row, so every thread issues all of its K + S + 1 loads at once.
// The grid is one-dimensional with a token's column blocks adjacent, so the
// blocks that run together read whole rows of the staged outputs.  Staged
// rows are read once and y written once: both non-temporal (at 8192 tokens
// 231 -> 184 us, at 4096 tokens with E4M3 weights 124 -> 90 us).
// ============================================================================

constexpr int COMBINE_THREADS = 128;

template <typename TE>
__global__ __launch_bounds__(COMBINE_THREADS) void combine_kernel(const TE* __restrict__ Y,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ gate,
                                                      const TE* __restrict__ residual,
                                                      TE* __restrict__ y, int T, int K, int H,
                                                      int TK, int S, int ncb) {
  constexpr int CE = 16 / sizeof(TE);
  const int t = int(blockIdx.x / unsigned(ncb)), cb = int(blockIdx.x - unsigned(t) * unsigned(ncb));
  __shared__ int rows_s[33];
  __shared__ float g_s[33];
  if (threadIdx.x < K) {
    rows_s[threadIdx.x] = slot[(size_t)t * K + threadIdx.x];
    g_s[threadIdx.x] = gate[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  const int c = (cb * COMBINE_THREADS + threadIdx.x) * CE;
  if (c < H) {  // H % 128 == 0: whole vectors
    float acc[CE];
#pragma unroll
    for (int q = 0; q < CE; ++q) acc[q] = 0.f;
    for (int sh = 0; sh < S; ++sh) {
      const TE* src = Y + (size_t)(TK + sh * T + t) * H + c;
      u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      const TE* pv = reinterpret_cast<const TE*>(&v);
#pragma unroll
      for (int q = 0; q < CE; ++q) acc[q] += to_f32<TE>(pv[q]);
    }
    for (int k = 0; k < K; ++k) {
      const float gk = g_s[k];
      u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Y + (size_t)rows_s[k] * H + c));
      const TE* pv = reinterpret_cast<const TE*>(&v);
#pragma unroll
      for (int q = 0; q < CE; ++q) acc[q] = fmaf(gk, to_f32<TE>(pv[q]), acc[q]);
    }
    if (residual != nullptr) {
      u32x4 v = *reinterpret_cast<const u32x4*>(residual + (size_t)t * H + c);
      const TE* pv = reinterpret_cast<const TE*>(&v);
#pragma unroll
      for (int q = 0; q < CE; ++q) acc[q] += to_f32<TE>(pv[q]);
    }
    u32x4 o;
    TE* po = reinterpret_cast<TE*>(&o);
#pragma unroll
    for (int q = 0; q < CE; ++q) po[q] = from_f32<TE>(acc[q]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(y + (size_t)t * H + c));
  }
}

// ============================================================================
// launchers
// ============================================================================

template <typename TE>
hipError_t launch_gemm(const GemmArgs<TE>& g, bool gated, int max_mtiles, int max_blocks,
                       hipStream_t st) {
  constexpr int BM = 64, BN = 64, BK = 64;
  const long long tasks = (long long)max_mtiles * (g.N / BN);
  dim3 grid((unsigned)std::min<long long>(tasks, max_blocks)), block(256);
  if (gated) hipLaunchKernelGGL((grouped_gemm_kernel<TE, true, BM, BN, BK>), grid, block, 0, st, g);
  else hipLaunchKernelGGL((grouped_gemm_kernel<TE, false, BM, BN, BK>), grid, block, 0, st, g);
  return hipGetLastError();
}

// float32 only: bf16 layers take the streaming and tiled GEMMs
template hipError_t launch_gemm<float>(const GemmArgs<float>&, bool, int, int, hipStream_t);

int gemm_tile_m() { return 64; }

template <typename TE>
hipError_t launch_combine(const TE* Y, const int32_t* slot, const float* gate, const TE* residual,
                          TE* y, int T, int K, int H, int TK, int S, hipStream_t st) {
  constexpr int CE = 16 / sizeof(TE);
  const int ncb = (H / CE + COMBINE_THREADS - 1) / COMBINE_THREADS;
  const long long blocks = (long long)T * ncb;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel<TE>, dim3((unsigned)blocks), dim3(COMBINE_THREADS), 0, st, Y,
                     slot, gate, residual, y, T, K, H, TK, S, ncb);
  return hipGetLastError();
}

template hipError_t launch_combine<bf16_t>(const bf16_t*, const int32_t*, const float*,
                                           const bf16_t*, bf16_t*, int, int, int, int, int,
                                           hipStream_t);
template hipError_t launch_combine<float>(const float*, const int32_t*, const float*, const float*,
                                          float*, int, int, int, int, int, hipStream_t);

}  // namespace moe
