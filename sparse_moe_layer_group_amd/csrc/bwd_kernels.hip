// Backward of the MoE layer for one training step (bf16 path).
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §1.3 Eq 12-15
// (gated combine, normalised sigmoid gates), §1.4 (the bias takes no part in
// backpropagation) and §2.2 (the SwiGLU output is recomputed in the backward).
// For the upstream gradient dy of the layer output, the kernels below form the
// gradients of <dy, y> with respect to x, W_r and every expert's matrices; the
// selection of experts is the forward's and carries no gradient.
//
// Row layout ("staged rows", as in the forward): routed expert e's rows are
// rows offsets[e] .. offsets[e] + counts[e] - 1 in expert order (perm gives
// their token ids), then the shared expert's T rows (row T*K + t is token t).
//
// GEMMs.  LDS-tiled grouped GEMMs on 32x32x16 bf16 MFMAs, operands copied
// straight into LDS by buffer_load ... lds:
//   - dgrad:  out[row][n] = sum_k A[row][k] B[k][n] over an expert's rows,
//     A = staged rows (k contiguous), B = the expert's weight matrix read along
//     its slow dimension (dH = dY W_down; dX = dG W_gate + dU W_up).
//     dgrad_tile_kernel (32 or more rows per expert): 320 x 256 tiles, eight
//     waves, K steps of 64 in two stages; dgrad_gemm_kernel (decode-sized
//     batches): 128 x 256 tiles, four waves, K steps of 32 in three stages;
//   - wgrad:  out[m][n] = sum over the expert's rows r of A[r][m] B[r][n]
//     (dW_down = dY^T H, dW_gate = dG^T X, dW_up = dU^T X), float32 out;
//     128 x 256 tiles, K steps of 32 rows.  wgrad_ws_kernel (more than 64
//     rows per routed expert): one persistent workgroup per CU, four copy and
//     four MFMA waves, six stages; wgrad_gemm_kernel (decode-sized batches):
//     one workgroup of four waves per tile, three stages.
// Operands whose contraction index is their slow (row) dimension are staged in
// LDS as "k-rows" in memory order and read with ds_read_b64_tr_b16: in each
// group of 16 lanes, source lane s addresses 4 consecutive columns of k-row
// kb + s/4, and lane d receives k-rows kb .. kb+3 of column d.  Two such reads
// give an MFMA operand's 8 consecutive k.
#include <type_traits>

#include "bwd.h"
#include "common.h"
#include "lds_async.h"

namespace moe {

namespace {

constexpr int BG_M = 128, BG_N = 128, BG_K = 32, BG_NS = 3;
constexpr int BG_NWAVE = 4, BG_NT = 64 * BG_NWAVE;
static_assert(BG_M == 128 && BG_N == 128 && BG_K == 32, "copy layouts below assume this tile");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// rows of 32 k (64 bytes): 16-byte chunk c of row r at position c ^ ((r/2) % 4)
MOE_DEV int rswz(int r, int c) { return c ^ ((r >> 1) & 3); }
// k-rows of 128 elements (256 bytes): 16-byte chunk c of k-row r at c ^ (2 (r % 4)),
// so the four k-rows of one transposed read hit distinct banks
MOE_DEV int kswz(int r, int c) { return c ^ ((r & 3) << 1); }

MOE_DEV bf16x8 row_frag(const bf16_t* st, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(st + row * BG_K + (rswz(row, chunk) << 3));
}

// MFMA operand of column block i0 .. i0+31 over k kbase .. kbase+15 from a
// k-row stage of RL columns: lane l gets column i0 + l%32, k = kbase + 8 (l/32) .. +7
template <int RL = BG_N>
MOE_DEV bf16x8 tr_frag(const bf16_t* st, int kbase, int i0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = i0 + 16 * (g & 1) + 4 * (s & 3);
  v4i16 h[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int k = kbase + 8 * (g >> 1) + 4 * q + (s >> 2);
    const bf16_t* p = st + k * RL + (kswz(k, col >> 3) << 3) + (col & 7);
    h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)((__attribute__((address_space(3))) bf16_t*)p));
  }
  const v4i16 lo = h[0], hi = h[1];
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return __builtin_bit_cast(bf16x8, v);
}

constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xf00; }

MOE_DEV float sigm(float v) { return 1.0f / (1.0f + expf(-v)); }

// (row base, rows) of expert e in the staged layout
MOE_DEV void expert_rows(const BwdArgs& g, int e, int& base, int& cnt) {
  const bool shared = e >= g.E;
  cnt = shared ? g.T : g.counts[e];
  base = shared ? g.TK + (e - g.E) * g.T : g.offsets[e];
}

}  // namespace

// ---------------------------------------------------------------- dgrad GEMM
// (128-row tiles, for decode-sized batches; dgrad_tile_kernel below serves
// batches with 32 or more rows per expert.)
// MODE 0: dH = dY W_down (K = hidden, N = inter); epilogue: SwiGLU backward,
//         dG = dH * U * SiLU'(G), dU = dH * SiLU(G) from the staged G and U.
// MODE 1: dX = dG W_gate + dU W_up (K = 2 x inter in two passes, N = hidden).
// Tile 128 rows x 256 columns; wave tile 64 x 128 (2 x 4 MFMA blocks).  A is
// staged as rows of 32 k, B as k-rows of 256 columns read transposed.
namespace {
constexpr int DG_N = 256;                                // output columns per tile
constexpr int DG_STAGE = BG_M * BG_K + BG_K * DG_N;      // bf16 elements per stage (A then B)
constexpr int DG_ACP = BG_M * BG_K * 2 / 1024 / BG_NWAVE;  // 1 KB A copies per wave per step (2)
constexpr int DG_BCP = BG_K * DG_N * 2 / 1024 / BG_NWAVE;  // ... B copies (4)
}  // namespace

template <int MODE>
__global__ __launch_bounds__(BG_NT, 2) void dgrad_gemm_kernel(BwdArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[BG_NS * DG_STAGE];
  const int N = MODE == 0 ? g.I : g.H;           // output columns
  const int Kp = MODE == 0 ? g.H : g.I;          // K of one pass
  const int n_nt = N / DG_N;
  const int n_tasks = g.mt[g.n_exp] * n_nt;
  const int task = blockIdx.x;
  if (task >= n_tasks) return;  // uniform, before any barrier
  int lo = 0, hi = g.n_exp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.mt[mid] * n_nt <= task) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int n_mt = g.mt[e + 1] - g.mt[e];
  const int local = task - g.mt[e] * n_nt;
  const int nt = local / n_mt, mtile = local - nt * n_mt;
  int row_base, cnt;
  expert_rows(g, e, row_base, cnt);
  const int m0 = mtile * BG_M, n0 = nt * DG_N;
  const int rows = min(BG_M, cnt - m0);
  const int nk1 = Kp / BG_K;
  const int nk = MODE == 0 ? nk1 : 2 * nk1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // A: staged rows [rows_total][Kp]; B: the expert's weights read as [Kp][N]
  const uint32_t total_rows = uint32_t(g.TK + (g.n_exp - g.E) * g.T);
  const bf16_t* a0p = MODE == 0 ? g.dyst : g.dgst;
  const bf16_t* a1p = MODE == 0 ? g.dyst : g.dust;
  const __amdgpu_buffer_rsrc_t ar0 = buffer_rsrc(a0p, total_rows * uint32_t(Kp) * 2u);
  const __amdgpu_buffer_rsrc_t ar1 = buffer_rsrc(a1p, total_rows * uint32_t(Kp) * 2u);
  const size_t wsz = size_t(Kp) * N;
  const bf16_t* b0p = (MODE == 0 ? g.w_down : g.w_gate) + size_t(e) * wsz;
  const bf16_t* b1p = (MODE == 0 ? g.w_down : g.w_up) + size_t(e) * wsz;
  const __amdgpu_buffer_rsrc_t br0 = buffer_rsrc(b0p, uint32_t(wsz * 2));
  const __amdgpu_buffer_rsrc_t br1 = buffer_rsrc(b1p, uint32_t(wsz * 2));

  // copy sources: A copy i of wave w covers tile rows 16 (2w+i) .. +15 (lane
  // l: row + l/4, position l%4); B copy i covers k-rows 2 (4w+i) .. +1 (lane
  // l: k-row + l/32, position l%32)
  uint32_t aoff[DG_ACP], boff[DG_BCP];
#pragma unroll
  for (int i = 0; i < DG_ACP; ++i) {
    const int r = 16 * (DG_ACP * wave + i) + (lane >> 2);
    const int m = row_base + m0 + min(r, rows - 1);  // rows past the count re-read a valid row
    aoff[i] = (uint32_t(m) * uint32_t(Kp) + uint32_t(rswz(r, lane & 3) * 8)) * 2u;
  }
#pragma unroll
  for (int i = 0; i < DG_BCP; ++i) {
    const int kr = 2 * (DG_BCP * wave + i) + (lane >> 5);
    boff[i] = (uint32_t(kr) * uint32_t(N) + uint32_t(n0 + kswz(kr, lane & 31) * 8)) * 2u;
  }
  auto copy_step = [&](int kt) {
    const int k = min(kt, nk - 1);
    const bool second = MODE == 1 && k >= nk1;
    const int kk = second ? k - nk1 : k;
    bf16_t* st = smem + (kt % BG_NS) * DG_STAGE;
    const __amdgpu_buffer_rsrc_t ar = second ? ar1 : ar0;
    const __amdgpu_buffer_rsrc_t br = second ? br1 : br0;
#pragma unroll
    for (int i = 0; i < DG_ACP; ++i)
      copy_to_lds_async16(ar, aoff[i] + uint32_t(kk * BG_K * 2), st + 16 * (DG_ACP * wave + i) * BG_K);
#pragma unroll
    for (int i = 0; i < DG_BCP; ++i)
      copy_to_lds_async16(br, boff[i] + uint32_t(kk * BG_K) * uint32_t(N) * 2u,
                    st + BG_M * BG_K + 2 * (DG_BCP * wave + i) * DG_N);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  copy_step(0);
  copy_step(1);
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(DG_ACP + DG_BCP));  // this wave's copies of kt landed
    __builtin_amdgcn_s_barrier();
    copy_step(kt + 2);
    const bf16_t* st = smem + (kt % BG_NS) * DG_STAGE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = row_frag(st, wm * 64 + 32 * i + (lane & 31), 2 * s + (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = tr_frag<DG_N>(st + BG_M * BG_K, 16 * s, wn * 128 + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  // epilogue.  32x32 accumulator v of lane l: row 8 (v/4) + 4 (l/32) + v%4, column l%32
  float part[2][16];  // MODE 0 with g.dgp: this lane's sum of dH * H per row
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) part[i][v] = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= rows) continue;
        const size_t o = size_t(row_base + m0 + r) * N + col;
        const float d = acc[i][j][v];
        if (MODE == 0) {
          const float G = bf16_to_f32(g.gst[o]), U = bf16_to_f32(g.ust[o]);
          const float sg = sigm(G);
          g.dgst[o] = f32_to_bf16(d * U * sg * (1.0f + G * (1.0f - sg)));
          const float du = d * G * sg;  // dH SiLU(G)
          g.dust[o] = f32_to_bf16(du);
          part[i][v] = fmaf(du, U, part[i][v]);  // dH H, H = SiLU(G) U
        } else {
          g.dxst[o] = f32_to_bf16(d);
        }
      }
    }
  if (MODE == 0 && g.dgp != nullptr) {
    // row sums over the tile's 256 columns: 32 lanes of a half-wave (fixed
    // butterfly), then the 2 waves along N through LDS in wave order
    float* red = reinterpret_cast<float*>(smem);  // [2][BG_M]
    __syncthreads();  // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float t = part[i][v];
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) t += __shfl_xor(t, off, 32);
        if ((lane & 31) == 0)
          red[wn * BG_M + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)] = t;
      }
    __syncthreads();
    if (tid < rows)
      g.dgp[size_t(nt) * (g.TK + (g.n_exp - g.E) * g.T) + row_base + m0 + tid] =
          red[tid] + red[BG_M + tid];
  }
}

// ---------------------------------------------------------------- dgrad GEMM, large tiles
// The same products as dgrad_gemm_kernel on the forward tile GEMM's design:
// tile 320 rows x 256 output columns, eight waves in 2 x 4 of 160 x 64 (5 x 2
// MFMA blocks, 32-row blocks past the expert's count skipped per wave), K in
// steps of 64 with two LDS stages.  Waves 0-3 copy only weight k-rows (2
// k-rows of 256 columns per 1 KB copy), waves 4-7 only staged rows (8 rows of
// 128 bytes per copy), and each waits only for its own copies.  A step's four
// k16 slices: each slice's fragments are read among the previous slice's
// MFMAs; after slice 2's MFMAs a wave waits for its copies of the next step
// and its LDS reads, the workgroup barriers, the copies two steps ahead go
// into the stage just finished, and slice 0 of the next step is read among
// slice 3's MFMAs.  Weight fragments come through ds_read_b64_tr_b16.
namespace {
constexpr int DT_M = 320, DT_N = 256, DT_K = 64;
constexpr int DT_MBW = DT_M / 64;                   // 32-row MFMA blocks per wave (5)
constexpr int DT_WN = 4, DT_NWAVE = 8, DT_NT = 64 * DT_NWAVE;
constexpr int DT_NJ = DT_N / DT_WN / 32;            // 32-column MFMA blocks per wave (2)
constexpr int DT_ASTAGE = DT_M * DT_K, DT_BSTAGE = DT_K * DT_N;  // bf16 elements per stage
constexpr int DT_ACP = DT_M / 8 / 4;                // 1 KB copies per row wave per step (10)
constexpr int DT_BCP = DT_K / 2 / 4;                // ... per weight wave (8)
static_assert(DT_ACP * 2 < 64 && DT_BCP * 2 < 64, "vmcnt field is 6 bits");

MOE_DEV bf16x8 dt_afrag(const bf16_t* base, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(base + row * DT_K + ((chunk ^ (row & 7)) << 3));
}
}  // namespace

int dgrad_tile_rows() { return DT_M; }
size_t dgrad_tile_lds_bytes() { return size_t(2 * (DT_ASTAGE + DT_BSTAGE)) * sizeof(bf16_t); }

template <int MODE>
__global__ __launch_bounds__(DT_NT, 1) void dgrad_tile_kernel(BwdArgs g) {
  extern __shared__ __attribute__((aligned(16))) bf16_t dsm[];
  bf16_t* As = dsm;                    // [2][DT_M][DT_K]
  bf16_t* Bs = dsm + 2 * DT_ASTAGE;    // [2][DT_K][DT_N]
  const int N = MODE == 0 ? g.I : g.H;           // output columns
  const int Kp = MODE == 0 ? g.H : g.I;          // K of one pass
  const int n_nt = N / DT_N;
  const int n_tasks = g.mtd[g.n_exp] * n_nt;
  const int task = blockIdx.x;
  if (task >= n_tasks) return;  // uniform, before any barrier
  int lo = 0, hi = g.n_exp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.mtd[mid] * n_nt <= task) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int n_mt = g.mtd[e + 1] - g.mtd[e];
  const int local = task - g.mtd[e] * n_nt;
  const int nt = local / n_mt, mtile = local - nt * n_mt;
  int row_base, cnt;
  expert_rows(g, e, row_base, cnt);
  const int m0 = mtile * DT_M, n0 = nt * DT_N;
  const int rows = min(DT_M, cnt - m0);
  const int nk1 = Kp / DT_K;
  const int nk = MODE == 0 ? nk1 : 2 * nk1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / DT_WN, wn = wave % DT_WN;
  const bool copies_b = wave < 4;
  const int cw = wave & 3;

  const uint32_t total_rows = uint32_t(g.TK + (g.n_exp - g.E) * g.T);
  __amdgpu_buffer_rsrc_t r0, r1;
  uint32_t off[DT_ACP > DT_BCP ? DT_ACP : DT_BCP];
  if (copies_b) {
    const size_t wsz = size_t(Kp) * N;
    r0 = buffer_rsrc((MODE == 0 ? g.w_down : g.w_gate) + size_t(e) * wsz, uint32_t(wsz * 2));
    r1 = buffer_rsrc((MODE == 0 ? g.w_down : g.w_up) + size_t(e) * wsz, uint32_t(wsz * 2));
#pragma unroll
    for (int i = 0; i < DT_BCP; ++i) {  // k-rows 2 (DT_BCP cw + i) + lane/32, chunk lane%32
      const int kr = 2 * (DT_BCP * cw + i) + (lane >> 5);
      off[i] = (uint32_t(kr) * uint32_t(N) + uint32_t(n0 + kswz(kr, lane & 31) * 8)) * 2u;
    }
  } else {
    r0 = buffer_rsrc(MODE == 0 ? g.dyst : g.dgst, total_rows * uint32_t(Kp) * 2u);
    r1 = buffer_rsrc(MODE == 0 ? g.dyst : g.dust, total_rows * uint32_t(Kp) * 2u);
#pragma unroll
    for (int i = 0; i < DT_ACP; ++i) {  // rows 8 (DT_ACP cw + i) + lane/8, position lane%8
      const int r = 8 * (DT_ACP * cw + i) + (lane >> 3);
      const int m = row_base + m0 + min(r, rows - 1);  // rows past the count re-read a valid row
      off[i] = (uint32_t(m) * uint32_t(Kp) + uint32_t(((lane & 7) ^ (r & 7)) * 8)) * 2u;
    }
  }
  auto copy_step = [&](int kt) {
    const int k = min(kt, nk - 1);
    const bool second = MODE == 1 && k >= nk1;
    const uint32_t kk = uint32_t(second ? k - nk1 : k);
    const __amdgpu_buffer_rsrc_t rs = second ? r1 : r0;
    if (copies_b) {
      bf16_t* d = Bs + (kt & 1) * DT_BSTAGE + 2 * DT_BCP * cw * DT_N;
      const uint32_t ko = kk * uint32_t(DT_K) * uint32_t(N) * 2u;
#pragma unroll
      for (int i = 0; i < DT_BCP; ++i) copy_to_lds_async16(rs, off[i] + ko, d + 2 * i * DT_N);
    } else {
      bf16_t* d = As + (kt & 1) * DT_ASTAGE + 8 * DT_ACP * cw * DT_K;
      const uint32_t ko = kk * uint32_t(DT_K) * 2u;
#pragma unroll
      for (int i = 0; i < DT_ACP; ++i) copy_to_lds_async16(rs, off[i] + ko, d + 8 * i * DT_K);
    }
  };

  const int mrows = rows - wm * 32 * DT_MBW;
  const int mact = __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : min(DT_MBW, (mrows + 31) >> 5));
  f32x16 acc[DT_MBW][DT_NJ];
#pragma unroll
  for (int i = 0; i < DT_MBW; ++i)
#pragma unroll
    for (int j = 0; j < DT_NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int arow0 = wm * 32 * DT_MBW + (lane & 31);

  auto mainloop = [&](auto mact_c) {
    constexpr int MACT = decltype(mact_c)::value;
    struct Frags { bf16x8 a[DT_MBW], b[DT_NJ]; };
    auto rd = [&](Frags& f, int kt, int sl) {
      const bf16_t* a = As + (kt & 1) * DT_ASTAGE;
      const bf16_t* b = Bs + (kt & 1) * DT_BSTAGE;
#pragma unroll
      for (int j = 0; j < DT_NJ; ++j) f.b[j] = tr_frag<DT_N>(b, 16 * sl, wn * 64 + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < MACT; ++i) f.a[i] = dt_afrag(a, arow0 + 32 * i, 2 * sl + (lane >> 5));
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
      for (int i = 0; i < MACT; ++i)
#pragma unroll
        for (int j = 0; j < DT_NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };
    // reads per slice: MACT row fragments and 2 DT_NJ transposed reads
    auto interleave = [&]() {
      static_assert(DT_NJ == 2, "two transposed weight fragments per slice");
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int k = 0; k < MACT; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (MACT * DT_NJ > MACT + DT_NJ)
        __builtin_amdgcn_sched_group_barrier(0x008, MACT * DT_NJ - MACT - DT_NJ, 0);
    };
    copy_step(0);
    copy_step(1);
    if (copies_b) __builtin_amdgcn_s_waitcnt(vm_wait_imm(DT_BCP));
    else __builtin_amdgcn_s_waitcnt(vm_wait_imm(DT_ACP));
    __builtin_amdgcn_s_barrier();
    Frags f0, f1;
    rd(f0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      rd(f1, kt, 1);
      mma(f0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      rd(f0, kt, 2);
      mma(f1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      rd(f1, kt, 3);
      mma(f0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      copy_step(kt + 2);
      __builtin_amdgcn_sched_barrier(0);
      rd(f0, kt + 1, 0);
      mma(f1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no copy left in flight
  };
  switch (mact) {
    case 5: mainloop(std::integral_constant<int, 5>{}); break;
    case 4: mainloop(std::integral_constant<int, 4>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    default: mainloop(std::integral_constant<int, 0>{}); break;
  }

  // epilogue.  32x32 accumulator v of lane l: row 8 (v/4) + 4 (l/32) + v%4,
  // column l%32.  Each wave stages one 32-row block of its 64 columns at a
  // time (float32) in a slot of its own; a lane then takes 8 consecutive
  // columns of a row, so G and U are read and dG, dU (dX) written 16 bytes a
  // lane instead of 2 bytes per accumulator element.
  constexpr int EP_PITCH = 64 * 4 + 16;  // staged row bytes (rows r, r + 4 in other banks)
  static_assert(DT_NWAVE * 32 * EP_PITCH + DT_WN * DT_M * 4 <= 2 * (DT_ASTAGE + DT_BSTAGE) * 2,
                "the staging slots and row sums fit the stages");
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  typedef __attribute__((address_space(3))) float lds_f32;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  __syncthreads();  // every wave is done with the stages
  lds_u8* slot = (lds_u8*)dsm + wave * 32 * EP_PITCH;
  lds_f32* red = (lds_f32*)((lds_u8*)dsm + DT_NWAVE * 32 * EP_PITCH);  // [DT_WN][DT_M] row sums
  const int er = lane >> 3, ec = 8 * (lane & 7);  // row within an 8-row pass, first column
#pragma unroll
  for (int i = 0; i < DT_MBW; ++i) {
    if (i >= mact) continue;  // uniform
#pragma unroll
    for (int j = 0; j < DT_NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        *(lds_f32*)(slot + (8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * EP_PITCH + 4 * (32 * j + (lane & 31))) =
            acc[i][j][v];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 8 * q + er;                     // row within the block
      const int r = wm * 32 * DT_MBW + 32 * i + rr;  // row within the tile
      const f32x4 d0 = *(const lds_f32x4*)(slot + rr * EP_PITCH + 4 * ec);
      const f32x4 d1 = *(const lds_f32x4*)(slot + rr * EP_PITCH + 4 * ec + 16);
      const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      float psum = 0.f;  // MODE 0: sum of dH * H over these 8 columns, in column order
      if (r < rows) {
        const size_t o = size_t(row_base + m0 + r) * N + n0 + wn * 64 + ec;
        u32x4 w0;
        if (MODE == 0) {
          const u32x4 gr = *reinterpret_cast<const u32x4*>(g.gst + o);
          const u32x4 ur = *reinterpret_cast<const u32x4*>(g.ust + o);
          u32x4 w1;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t pg = 0, pu = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float G = bf16_to_f32(bf16_t(gr[k] >> (16 * h))), U = bf16_to_f32(bf16_t(ur[k] >> (16 * h)));
              const float dh = d[2 * k + h];
              const float sg = sigm(G);
              const float du = dh * G * sg;  // dH SiLU(G)
              pg |= uint32_t(f32_to_bf16(dh * U * sg * (1.0f + G * (1.0f - sg)))) << (16 * h);
              pu |= uint32_t(f32_to_bf16(du)) << (16 * h);
              psum = fmaf(du, U, psum);      // dH H, H = SiLU(G) U
            }
            w0[k] = pg;
            w1[k] = pu;
          }
          *reinterpret_cast<u32x4*>(g.dgst + o) = w0;
          *reinterpret_cast<u32x4*>(g.dust + o) = w1;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            w0[k] = uint32_t(f32_to_bf16(d[2 * k])) | (uint32_t(f32_to_bf16(d[2 * k + 1])) << 16);
          *reinterpret_cast<u32x4*>(g.dxst + o) = w0;
        }
      }
      if (MODE == 0 && g.dgp != nullptr) {
        // the row's sum over this wave's 64 columns: its 8 lanes, fixed butterfly
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) psum += __shfl_xor(psum, off, 8);
        if ((lane & 7) == 0) red[wn * DT_M + r] = psum;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if (MODE == 0 && g.dgp != nullptr) {
    // row sums over the tile's 256 columns: the 4 waves along N in wave order
    __syncthreads();
    if (tid < rows) {
      const int wmr = tid / (32 * DT_MBW), mb = (tid - wmr * 32 * DT_MBW) >> 5;
      // rows of 32-row blocks past a wave's active count were never written
      const int mrows_r = rows - wmr * 32 * DT_MBW;
      if (mb < min(DT_MBW, (mrows_r + 31) >> 5)) {
        const float t = ((red[tid] + red[DT_M + tid]) + red[2 * DT_M + tid]) + red[3 * DT_M + tid];
        g.dgp[size_t(nt) * (g.TK + (g.n_exp - g.E) * g.T) + row_base + m0 + tid] = t;
      }
    }
  }
}

// ---------------------------------------------------------------- wgrad GEMM
// (one workgroup per tile, for decode-sized batches of up to 64 rows per
// routed expert, where the tiles are nearly pure stores; wgrad_ws_kernel below
// serves larger batches.)
// out[e][m][n] = sum over expert e's rows r of A[r][m] B[r][n], float32.
// MODE 0: dW_down (A = dY [.][hidden], B = H [.][inter]);
// MODE 1: dW_gate (A = dG [.][inter], B = X [.][hidden]); MODE 2: dW_up (A = dU).
// Tile 128 (m) x 256 (n); wave tile 64 x 128 (2 x 4 MFMA blocks).  Both
// operands are staged as k-rows (one per token row, 32 per step): A rows of
// 128, B rows of 256 elements.  Rows past the expert's count read beyond the
// buffer, which returns zeros, so they add nothing.
namespace {
constexpr int WG_N = 256;                               // n columns per tile


constexpr int WG_STAGE = BG_K * BG_M + BG_K * WG_N;     // bf16 elements per stage (A then B)
constexpr int WG_ACP = BG_K * BG_M * 2 / 1024 / BG_NWAVE;  // 1 KB A copies per wave per step (2)
constexpr int WG_BCP = BG_K * WG_N * 2 / 1024 / BG_NWAVE;  // ... B copies (4)
}  // namespace

template <int MODE>
__global__ __launch_bounds__(BG_NT, 2) void wgrad_gemm_kernel(BwdArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[BG_NS * WG_STAGE];
  const int M = MODE == 0 ? g.H : g.I;
  const int N = MODE == 0 ? g.I : g.H;
  const int tm = M / BG_M, tn = N / WG_N;
  // experts in reverse order: the shared experts' tiles, which contract over
  // all T rows, start first instead of forming the launch's tail.  Workgroup
  // b runs on XCD b % 8; the shared experts' tiles are dealt round-robin and
  // the routed experts' tiles to the XCDs in contiguous eighths, so each XCD
  // writes a contiguous eighth of the gradients (7.9 -> 7.3 ms for the three
  // launches at 256 tokens).  The shared tiles' count is a multiple of 8, and
  // the launch holds 8 ceil(routed tiles / 8) slots past them.
  const int per_e = tm * tn;
  const int sh_tiles = (g.n_exp - g.E) * per_e;
  int task = blockIdx.x;
  if (task >= sh_tiles) {
    const int b = task - sh_tiles, rt = g.E * per_e, per = (rt + 7) >> 3;
    const int j = b >> 3;
    task = sh_tiles + (b & 7) * per + j;
    if (j >= per || task >= sh_tiles + rt) return;  // uniform
  }
  const int eb = task / per_e;
  if (eb >= g.n_exp) return;  // uniform
  const int e = g.n_exp - 1 - eb;
  const int t = task - eb * per_e;
  const int mt = t / tn, ntile = t - mt * tn;
  const int m0 = mt * BG_M, n0 = ntile * WG_N;
  int row_base, cnt;
  expert_rows(g, e, row_base, cnt);
  const int nk = (cnt + BG_K - 1) / BG_K;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const uint32_t total_rows = uint32_t(g.TK + (g.n_exp - g.E) * g.T);
  const bf16_t* ap = MODE == 0 ? g.dyst : (MODE == 1 ? g.dgst : g.dust);
  const bf16_t* bp = MODE == 0 ? g.hst : g.xst;
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(ap, total_rows * uint32_t(M) * 2u);
  const __amdgpu_buffer_rsrc_t br = buffer_rsrc(bp, total_rows * uint32_t(N) * 2u);
  // A copy i of wave w: k-rows 4 (2w+i) .. +3 (lane l: + l/16, position l%16);
  // B copy i: k-rows 2 (4w+i) .. +1 (lane l: + l/32, position l%32)
  uint32_t acol[WG_ACP], bcol[WG_BCP];
  int akr[WG_ACP], bkr[WG_BCP];
#pragma unroll
  for (int i = 0; i < WG_ACP; ++i) {
    akr[i] = 4 * (WG_ACP * wave + i) + (lane >> 4);
    acol[i] = uint32_t(m0 + kswz(akr[i], lane & 15) * 8);
  }
#pragma unroll
  for (int i = 0; i < WG_BCP; ++i) {
    bkr[i] = 2 * (WG_BCP * wave + i) + (lane >> 5);
    bcol[i] = uint32_t(n0 + kswz(bkr[i], lane & 31) * 8);
  }
  auto copy_step = [&](int kt) {
    const int k = min(kt, max(nk - 1, 0));
    bf16_t* st = smem + (kt % BG_NS) * WG_STAGE;
#pragma unroll
    for (int i = 0; i < WG_ACP; ++i) {
      const int r = k * BG_K + akr[i];
      const uint32_t o = r < cnt ? (uint32_t(row_base + r) * uint32_t(M) + acol[i]) * 2u : 0xfffffff0u;
      copy_to_lds_async16(ar, o, st + 4 * (WG_ACP * wave + i) * BG_M);
    }
#pragma unroll
    for (int i = 0; i < WG_BCP; ++i) {
      const int r = k * BG_K + bkr[i];
      const uint32_t o = r < cnt ? (uint32_t(row_base + r) * uint32_t(N) + bcol[i]) * 2u : 0xfffffff0u;
      copy_to_lds_async16(br, o, st + BG_K * BG_M + 2 * (WG_BCP * wave + i) * WG_N);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (nk > 0) {  // uniform
    copy_step(0);
    copy_step(1);
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(WG_ACP + WG_BCP));  // this wave's copies of kt landed
      __builtin_amdgcn_s_barrier();
      copy_step(kt + 2);
      const bf16_t* st = smem + (kt % BG_NS) * WG_STAGE;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 af[2], bf[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = tr_frag<BG_M>(st, 16 * s, wm * 64 + 32 * i, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bf[j] = tr_frag<WG_N>(st + BG_K * BG_M, 16 * s, wn * 128 + 32 * j, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
  }

  float* out = (MODE == 0 ? g.dw_down : (MODE == 1 ? g.dw_gate : g.dw_up)) + size_t(e) * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        // written once: non-temporal (16.6 -> 14.8 ms for the three launches at 8192 tokens)
        __builtin_nontemporal_store(acc[i][j][v], out + size_t(r) * N + col);
      }
    }
  // (staging the tile through LDS for 1 KB row stores measured no better here:
  // +0.9% at 8192 tokens, -3% at 256)
}

// ---------------------------------------------------------------- wgrad, persistent
// The products of wgrad_gemm_kernel with its waves split by role, so that the
// gradient stores overlap the copies and MFMAs of the tiles after them.  One
// workgroup per CU walks a fixed list of 128 x 256 tiles: the shared experts'
// tiles dealt round-robin over all workgroups, then routed expert e's tiles
// dealt round-robin over the workgroups with b % 8 == e % 8 (workgroup b runs
// on XCD b % 8, so each expert's operands are fetched into one L2).
// MODE 0: dW_down; MODE 1: dW_gate and dW_up, each tile's two in a row.
//   - waves 4-7 only copy: k-steps of 32 rows into a ring of WS_NS LDS stages,
//     WS_NS - 1 steps ahead; before barrier p they wait until steps p and p + 1
//     have landed, after it they refill the stage step p - 1 used;
//   - waves 0-3 only compute (64 x 128 each, as wgrad_gemm_kernel's waves) and
//     store.  Such a wave never waits for a load issued after its stores, so
//     the stores drain while the next tiles run.  Each step's first k16 slice
//     is read in the step before (barrier p certifies step p + 1).
// Stores keep the MFMA's layout: 4-byte stores, 32 lanes on 128 contiguous
// bytes of one gradient row.  (16-byte stores measured slower: after 4 x 4
// transposes within lane quads, 8 rows x 128 bytes per instruction, +13% at
// 8192 tokens; with the operands swapped, 32 rows x 32 bytes, 2-4x.)
namespace {
// Measured at 8192 tokens against this shape (12.65 ms for the stage): barrier
// p certifying step p only, 12.86 ms; two workgroups per CU of four MFMA and
// two copy waves with three stages each, 14.59 ms.
constexpr int WS_NS = 6;                                // LDS stages
constexpr int WS_CW = 4;                                // copy waves
constexpr int WS_PF = 1;                                // barrier p certifies steps p and p + 1
constexpr int WS_BPC = 1;                               // workgroups per CU
constexpr int WS_NT = 64 * (4 + WS_CW);                 // 4 compute waves + the copy waves
constexpr int WS_ACP = BG_K * BG_M * 2 / 1024 / WS_CW;  // 1 KB A copies per copy wave and step
constexpr int WS_BCP = BG_K * WG_N * 2 / 1024 / WS_CW;  // ... B copies
constexpr int WS_CPW = WS_ACP + WS_BCP;                 // copies per copy wave and step
static_assert(WS_CPW * (WS_NS - 2) < 64, "vmcnt holds 6 bits");
static_assert(WS_NS >= 3 + WS_PF, "a stage is refilled only after its step was read");

struct WsTile {
  int e, m0, n0, base, cnt, mode;
};

// Tile i of workgroup b's list (G workgroups), or false past its end; the
// experts' (first row, rows) from the LDS copies rb, rc.  With nmode = 2
// (dW_gate and dW_up in one launch) each tile comes twice in a row, mode 0
// then 1: the two share their X slab, which is then fetched once.
MOE_DEV bool ws_tile(const BwdArgs& g, const int* rb, const int* rc, int tm, int tn, int nmode, int b, int G,
                     int i, WsTile& t) {
  const int per_e = tm * tn * nmode;
  const int sh = (g.n_exp - g.E) * per_e;
  const int n_sh = b < sh ? (sh - 1 - b) / G + 1 : 0;
  int e, q;
  if (i < n_sh) {
    const int task = b + i * G;
    e = g.E + task / per_e;
    q = task - (e - g.E) * per_e;
  } else {
    const int x = b & 7, nx = (G - 1 - x) / 8 + 1;  // workgroups on XCD x
    const int task = (b >> 3) + (i - n_sh) * nx;
    const int eo = task / per_e;
    e = x + 8 * eo;
    if (e >= g.E) return false;
    q = task - eo * per_e;
  }
  // row-major over the expert's tiles: the XCD's workgroups write whole rows
  // of the gradient at a time (column-major, which fetches 2.5x fewer operand
  // bytes for dW_gate and dW_up, measured 27% slower at 8192 tokens)
  t.mode = nmode == 2 ? (q & 1) : 0;
  if (nmode == 2) q >>= 1;
  const int mt = q / tn, nt = q - mt * tn;
  t.e = e;
  t.m0 = mt * BG_M;
  t.n0 = nt * WG_N;
  t.base = rb[e];
  t.cnt = rc[e];
  return true;
}
}  // namespace

template <int MODE>
// (the second bound is waves per SIMD: WS_BPC workgroups of 4 + WS_CW waves per CU)
__global__ __launch_bounds__(WS_NT, WS_BPC * (4 + WS_CW) / 4) void wgrad_ws_kernel(BwdArgs g) {
  // WS_NS stages of WG_STAGE, then every expert's first row and rows: read
  // from LDS, the tile walk issues no global load (a wave that has stores in
  // flight would wait for them before one)
  extern __shared__ __attribute__((aligned(16))) bf16_t wsm[];
  int* rb = reinterpret_cast<int*>(wsm + WS_NS * WG_STAGE);
  int* rc = rb + g.n_exp;
  constexpr int NMODE = MODE == 0 ? 1 : 2;
  const int M = MODE == 0 ? g.H : g.I;
  const int N = MODE == 0 ? g.I : g.H;
  const int tm = M / BG_M, tn = N / WG_N;
  const int b = blockIdx.x, G = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int e = tid; e < g.n_exp; e += WS_NT) expert_rows(g, e, rb[e], rc[e]);
  __syncthreads();
  WsTile t;

  if (wave >= 4) {
    // ---- copy waves.  Copy wave c: A copies 2c, 2c + 1 (k-rows 4 (2c + i) .. +3,
    // lane l: + l/16, position l%16), B copies 4c .. 4c + 3 (k-rows 2 (4c + i) .. +1)
    const int c = wave - 4;
    const uint32_t total_rows = uint32_t(g.TK + (g.n_exp - g.E) * g.T);
    const __amdgpu_buffer_rsrc_t ar0 = buffer_rsrc(MODE == 0 ? g.dyst : g.dgst, total_rows * uint32_t(M) * 2u);
    const __amdgpu_buffer_rsrc_t ar1 = buffer_rsrc(MODE == 0 ? g.dyst : g.dust, total_rows * uint32_t(M) * 2u);
    const __amdgpu_buffer_rsrc_t br = buffer_rsrc(MODE == 0 ? g.hst : g.xst, total_rows * uint32_t(N) * 2u);
    int akr[WS_ACP], ach[WS_ACP], bkr[WS_BCP], bch[WS_BCP];
#pragma unroll
    for (int i = 0; i < WS_ACP; ++i) {
      akr[i] = 4 * (WS_ACP * c + i) + (lane >> 4);
      ach[i] = kswz(akr[i], lane & 15) * 8;
    }
#pragma unroll
    for (int i = 0; i < WS_BCP; ++i) {
      bkr[i] = 2 * (WS_BCP * c + i) + (lane >> 5);
      bch[i] = kswz(bkr[i], lane & 31) * 8;
    }
    // look-ahead cursor: step lk of tile li (tiles without rows have no steps)
    int li = 0, lk = 0, issued = 0;
    WsTile lt;
    bool more = ws_tile(g, rb, rc, tm, tn, NMODE, b, G, 0, lt);
    while (more && lt.cnt == 0) more = ws_tile(g, rb, rc, tm, tn, NMODE, b, G, ++li, lt);
    auto issue = [&]() {
      bf16_t* st = wsm + (issued % WS_NS) * WG_STAGE;
      const int r0 = lk * BG_K;
      const __amdgpu_buffer_rsrc_t ar = lt.mode ? ar1 : ar0;
#pragma unroll
      for (int i = 0; i < WS_ACP; ++i) {
        const int r = r0 + akr[i];
        const uint32_t o =
            r < lt.cnt ? (uint32_t(lt.base + r) * uint32_t(M) + uint32_t(lt.m0 + ach[i])) * 2u : 0xfffffff0u;
        copy_to_lds_async16(ar, o, st + 4 * (WS_ACP * c + i) * BG_M);
      }
#pragma unroll
      for (int i = 0; i < WS_BCP; ++i) {
        const int r = r0 + bkr[i];
        const uint32_t o =
            r < lt.cnt ? (uint32_t(lt.base + r) * uint32_t(N) + uint32_t(lt.n0 + bch[i])) * 2u : 0xfffffff0u;
        copy_to_lds_async16(br, o, st + BG_K * BG_M + 2 * (WS_BCP * c + i) * WG_N);
      }
      ++issued;
      if (++lk * BG_K >= lt.cnt) {
        lk = 0;
        do more = ws_tile(g, rb, rc, tm, tn, NMODE, b, G, ++li, lt);
        while (more && lt.cnt == 0);
      }
    };
    for (int s = 0; s < WS_NS - 1 && more; ++s) issue();
    if (WS_PF) {
      if (issued == WS_NS - 1) __builtin_amdgcn_s_waitcnt(vm_wait_imm(WS_CPW * (WS_NS - 2)));
      else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
      __builtin_amdgcn_s_barrier();  // step 0 landed
    }
    int p = 0;
    for (int i = 0; ws_tile(g, rb, rc, tm, tn, NMODE, b, G, i, t); ++i) {
      const int nk = (t.cnt + BG_K - 1) / BG_K;
      for (int kt = 0; kt < nk; ++kt, ++p) {
        // steps p (and with WS_PF p + 1) landed: the copies of p + 1 + WS_PF ..
        // issued - 1 may still fly
        if (issued - p - 1 - WS_PF == WS_NS - 2 - WS_PF)
          __builtin_amdgcn_s_waitcnt(vm_wait_imm(WS_CPW * (WS_NS - 2 - WS_PF)));
        else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (more) issue();  // step p + WS_NS - 1 into the stage of step p - 1
      }
    }
    return;
  }

  // ---- compute waves
  const int wm = wave >> 1, wn = wave & 1;
  auto frags = [&](const bf16_t* st, int s, bf16x8* af, bf16x8* bf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) af[i] = tr_frag<BG_M>(st, 16 * s, wm * 64 + 32 * i, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = tr_frag<WG_N>(st + BG_K * BG_M, 16 * s, wn * 128 + 32 * j, lane);
  };
  bf16x8 a0[2], b0[4];  // the first k16 slice of the coming step
  if (WS_PF) {
    __builtin_amdgcn_s_barrier();  // step 0 landed
    asm volatile("" ::: "memory");
    frags(wsm, 0, a0, b0);
  }
  int p = 0;
  for (int i = 0; ws_tile(g, rb, rc, tm, tn, NMODE, b, G, i, t); ++i) {
    f32x16 acc[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[u][j][v] = 0.f;
    const int nk = (t.cnt + BG_K - 1) / BG_K;
    for (int kt = 0; kt < nk; ++kt, ++p) {
      __builtin_amdgcn_s_barrier();  // steps p and p + 1 landed; step p - 1's stage is being refilled
      asm volatile("" ::: "memory");
      const bf16_t* st = wsm + (p % WS_NS) * WG_STAGE;
      bf16x8 a1[2], b1[4];
      if (!WS_PF) frags(st, 0, a0, b0);
      frags(st, 1, a1, b1);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[u][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[u], b0[j], acc[u][j], 0, 0, 0);
      if (WS_PF) frags(wsm + ((p + 1) % WS_NS) * WG_STAGE, 0, a0, b0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[u][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[u], b1[j], acc[u][j], 0, 0, 0);
    }
    // lane l holds column n0 + wn 128 + 32 j + l%32 of rows m0 + wm 64 + 32 u + 8 (v/4) + 4 (l/32) + v%4
    float* outb = MODE == 0 ? g.dw_down : (t.mode ? g.dw_up : g.dw_gate);
    float* out = outb + size_t(t.e) * M * N + size_t(t.m0 + wm * 64 + 4 * (lane >> 5)) * N + t.n0 + wn * 128 +
                 (lane & 31);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)  // written once, never read here: non-temporal
          __builtin_nontemporal_store(acc[u][j][v], out + size_t(32 * u + 8 * (v >> 2) + (v & 3)) * N + 32 * j);
  }
}

// ---------------------------------------------------------------- row kernels

// Xst[r] = x[perm[r]] (routed rows), Xst[T K + t] = x[t] (shared rows)
__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm, int T,
                                                          int TK, int S, int H,
                                                          bf16_t* __restrict__ xst) {
  const int r = blockIdx.x;
  const int src = r < TK ? perm[r] : (r - TK) % T;
  const u32x4* s = reinterpret_cast<const u32x4*>(x + size_t(src) * H);
  u32x4* d = reinterpret_cast<u32x4*>(xst + size_t(r) * H);
  for (int c = threadIdx.x; c < H / 8; c += 256) d[c] = s[c];
}

// Per token t: for each chosen expert k, the gate gradient dg = <dy_t, Y_k[t]>
// (fixed-order block reduction) and the expert's output gradient g_k dy_t; the
// shared expert's output gradient is dy_t itself.  dyst == nullptr: gate
// gradients only; yst == nullptr: output gradients only.
__global__ __launch_bounds__(256) void combine_bwd_kernel(const bf16_t* __restrict__ dy,
                                                          const bf16_t* __restrict__ yst,
                                                          const int32_t* __restrict__ slot,
                                                          const float* __restrict__ gate, int T,
                                                          int K, int H, int TK, int S,
                                                          bf16_t* __restrict__ dyst,
                                                          float* __restrict__ dg) {
  __shared__ float red[32][4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = H / 8;
  const u32x4* d8 = reinterpret_cast<const u32x4*>(dy + size_t(t) * H);
  if (S > 0 && dyst != nullptr) {
    u32x4* o = reinterpret_cast<u32x4*>(dyst + size_t(TK + t) * H);
    for (int c = tid; c < nch; c += 256) o[c] = d8[c];
  }
  if (yst == nullptr) {  // output gradients only (the gate gradients come from dH)
    for (int k = 0; k < K; ++k) {
      const int sl = slot[t * K + k];
      const float gk = gate[t * K + k];
      u32x4* o = reinterpret_cast<u32x4*>(dyst + size_t(sl) * H);
      for (int c = tid; c < nch; c += 256) {
        const u32x4 dv = d8[c];
        u32x4 ov;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ov[q] = uint32_t(f32_to_bf16(gk * __uint_as_float(dv[q] << 16))) |
                  (uint32_t(f32_to_bf16(gk * __uint_as_float(dv[q] & 0xffff0000u))) << 16);
        o[c] = ov;
      }
    }
    return;
  }
  for (int k0 = 0; k0 < K; k0 += 32) {
    const int kn = min(32, K - k0);
    float part[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) part[k] = 0.f;
    for (int c = tid; c < nch; c += 256) {
      const u32x4 dv = d8[c];
      float dyf[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dyf[2 * q] = __uint_as_float(dv[q] << 16);
        dyf[2 * q + 1] = __uint_as_float(dv[q] & 0xffff0000u);
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (k >= kn) continue;  // uniform
        const int sl = slot[t * K + k0 + k];
        const float gk = gate[t * K + k0 + k];
        const u32x4 yv = reinterpret_cast<const u32x4*>(yst + size_t(sl) * H)[c];
        u32x4 ov;
        float p = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float y0 = __uint_as_float(yv[q] << 16), y1 = __uint_as_float(yv[q] & 0xffff0000u);
          p = fmaf(dyf[2 * q], y0, p);
          p = fmaf(dyf[2 * q + 1], y1, p);
          ov[q] = uint32_t(f32_to_bf16(gk * dyf[2 * q])) |
                  (uint32_t(f32_to_bf16(gk * dyf[2 * q + 1])) << 16);
        }
        part[k] += p;
        if (dyst != nullptr) reinterpret_cast<u32x4*>(dyst + size_t(sl) * H)[c] = ov;
      }
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k >= kn) continue;  // uniform
      const float w = wave_sum(part[k]);
      if (lane == 0) red[k][wave] = w;
    }
    __syncthreads();
    if (tid < kn) dg[t * K + k0 + tid] = ((red[tid][0] + red[tid][1]) + red[tid][2]) + red[tid][3];
    __syncthreads();
  }
}

// Per token: affinities of the chosen experts from the router partials (added
// in partial order, as the selection does), gate normalisation and sigmoid
// backward: ds_k = (dg_k - sum_j dg_j g_j) / S, dL_k = ds_k s_k (1 - s_k).
// Writes dL per assignment [T][K] and per staged row.  With dgp the gate
// gradients are first formed from the data-gradient GEMM's row sums.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ P, int ks,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ slot,
                                                         float* __restrict__ dg, int T,
                                                         int E, int K, float* __restrict__ dl,
                                                         float* __restrict__ dlst,
                                                         const float* __restrict__ dgp, int n_part,
                                                         long long rows_total,
                                                         const float* __restrict__ gate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  if (dgp != nullptr) {
    // dg_k = <dy, Y_k> = <dy W_down, H_k> = <dH_k, H_k> / g_k, dH_k = g_k dy W_down
    // (the data-gradient GEMM's per-tile row sums, added in tile order).  A gate
    // of exactly 0 (its sigmoid underflowed) gets dg_k = 0: below, dg_k enters
    // only through g_k dg_k and through ds_k, which is scaled by s_k (1 - s_k) = 0,
    // so every logit gradient is the same as with the true <dy, Y_k>.
    for (int k = 0; k < K; ++k) {
      const long long r = slot[t * K + k];
      float a = 0.f;
      for (int p = 0; p < n_part; ++p) a += dgp[p * rows_total + r];
      const float gk = gate[t * K + k];
      dg[t * K + k] = gk > 0.f ? a / gk : 0.f;
    }
  }
  float s[32];
  float S = 0.f;
  for (int k = 0; k < K; ++k) {
    const int e = idx[t * K + k];
    float L = 0.f;
    for (int c = 0; c < ks; ++c) L += P[(size_t(c) * T + t) * E + e];
    s[k] = sigm(L);
    S += s[k];
  }
  float dsum = 0.f;
  for (int k = 0; k < K; ++k) dsum += dg[t * K + k] * (s[k] / S);
  for (int k = 0; k < K; ++k) {
    const float v = (dg[t * K + k] - dsum) / S * s[k] * (1.0f - s[k]);
    dl[t * K + k] = v;
    dlst[slot[t * K + k]] = v;
  }
}

// dW_r^T[e][h] = sum over expert e's routed rows r of dL_r X_r[h], rows in order.
// X_r is token perm[r]'s row of x, read through the permutation (x is small
// enough to stay in the caches, its staged copy is not); eight rows' loads are
// issued together and added in row order.
__global__ __launch_bounds__(256) void dwr_kernel(const float* __restrict__ dlst,
                                                  const bf16_t* __restrict__ x,
                                                  const int32_t* __restrict__ perm,
                                                  const int32_t* __restrict__ counts,
                                                  const int32_t* __restrict__ offsets, int H,
                                                  float* __restrict__ dwrt) {
  constexpr int U = 8;
  const int e = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  const int base = offsets[e], cnt = counts[e];
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  auto add = [&](float w, uint2 v) {
    a0 = fmaf(w, __uint_as_float(v.x << 16), a0);
    a1 = fmaf(w, __uint_as_float(v.x & 0xffff0000u), a1);
    a2 = fmaf(w, __uint_as_float(v.y << 16), a2);
    a3 = fmaf(w, __uint_as_float(v.y & 0xffff0000u), a3);
  };
  int r = 0;
  for (; r + U <= cnt; r += U) {
    float w[U];
    uint2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w[u] = dlst[base + r + u];
      v[u] = *reinterpret_cast<const uint2*>(x + size_t(perm[base + r + u]) * H + h);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) add(w[u], v[u]);
  }
  for (; r < cnt; ++r)
    add(dlst[base + r], *reinterpret_cast<const uint2*>(x + size_t(perm[base + r]) * H + h));
  *reinterpret_cast<f32x4*>(dwrt + size_t(e) * H + h) = f32x4{a0, a1, a2, a3};
}

// out[c][r] = in[r][c], float32, through a 32 x 33 LDS tile
__global__ __launch_bounds__(256) void transpose_f32_kernel(const float* __restrict__ in, int R,
                                                            int C, float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 8 rows per pass
  for (int i = ty; i < 32; i += 8)
    if (r0 + i < R && c0 + tx < C) tile[i][tx] = in[size_t(r0 + i) * C + c0 + tx];
  __syncthreads();
  for (int i = ty; i < 32; i += 8)
    if (c0 + i < C && r0 + tx < R) out[size_t(c0 + i) * R + r0 + tx] = tile[tx][i];
}

// dx_t = dX_shared[t] + sum_k dX[slot(t, k)] + sum_k dL_tk W_r[:, e_k], float32
// in that order, bf16 out.  The token's slots, expert ids and logit gradients
// sit in LDS, and the rows of each group of up to eight terms are loaded
// together before they are added in order.
__global__ __launch_bounds__(256) void dx_kernel(const bf16_t* __restrict__ dxst,
                                                 const int32_t* __restrict__ slot,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ dl,
                                                 const float* __restrict__ wrt, int T, int K,
                                                 int H, int TK, int S, bf16_t* __restrict__ dx) {
  constexpr int U = 8;
  __shared__ int sl_s[32], ix_s[32];
  __shared__ float dl_s[32];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    sl_s[threadIdx.x] = slot[t * K + threadIdx.x];
    ix_s[threadIdx.x] = idx[t * K + threadIdx.x];
    dl_s[threadIdx.x] = dl[t * K + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    float a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = 0.f;
    auto add_row = [&](const u32x4& v) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[2 * q] += __uint_as_float(v[q] << 16);
        a[2 * q + 1] += __uint_as_float(v[q] & 0xffff0000u);
      }
    };
    if (S > 0) add_row(reinterpret_cast<const u32x4*>(dxst + size_t(TK + t) * H)[c]);
    for (int k0 = 0; k0 < K; k0 += U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (k0 + u < K) v[u] = reinterpret_cast<const u32x4*>(dxst + size_t(sl_s[k0 + u]) * H)[c];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (k0 + u < K) add_row(v[u]);
    }
    for (int k0 = 0; k0 < K; k0 += U) {
      f32x4 r0[U], r1[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (k0 + u < K) {
          const f32x4* r = reinterpret_cast<const f32x4*>(wrt + size_t(ix_s[k0 + u]) * H + 8 * c);
          r0[u] = r[0];
          r1[u] = r[1];
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (k0 + u < K) {
          const float w = dl_s[k0 + u];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a[q] = fmaf(w, r0[u][q], a[q]);
            a[4 + q] = fmaf(w, r1[u][q], a[4 + q]);
          }
        }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = uint32_t(f32_to_bf16(a[2 * q])) | (uint32_t(f32_to_bf16(a[2 * q + 1])) << 16);
    reinterpret_cast<u32x4*>(dx + size_t(t) * H)[c] = o;
  }
}

// row-tile prefix of the dgrad GEMM: mt[e] = sum over experts before e of
// ceil(rows / 128) (routed counts, then the shared experts' T rows)
__global__ __launch_bounds__(64) void bwd_tile_prefix_kernel(const int32_t* __restrict__ counts,
                                                             int E, int S, int T, int tile,
                                                             int32_t* __restrict__ mt) {
  if (threadIdx.x != 0) return;
  int acc = 0;
  for (int e = 0; e < E + S; ++e) {
    mt[e] = acc;
    const int c = e < E ? counts[e] : T;
    acc += (c + tile - 1) / tile;
  }
  mt[E + S] = acc;
}

// ---------------------------------------------------------------- launches

int bwd_max_row_tiles(int T, int K, int E, int S) {
  return (T * K + BG_M - 1) / BG_M + E + S * ((T + BG_M - 1) / BG_M);
}

namespace {
int dgrad_max_tiles(int T, int K, int E, int S) {
  return (T * K + DT_M - 1) / DT_M + E + S * ((T + DT_M - 1) / DT_M);
}

template <int MODE>
hipError_t launch_dgrad_tile(const BwdArgs& g, unsigned blocks, hipStream_t st) {
  static bool attr_set = false;
  const size_t lds = dgrad_tile_lds_bytes();
  if (!attr_set) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&dgrad_tile_kernel<MODE>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL(dgrad_tile_kernel<MODE>, dim3(blocks), dim3(DT_NT), lds, st, g);
  return hipGetLastError();
}

// One persistent workgroup per CU (at least 8, one per XCD)
template <int MODE>
hipError_t launch_wgrad_ws(const BwdArgs& g, hipStream_t st) {
  constexpr int kLdsMax = 160 * 1024;  // LDS per CU
  static bool attr_set = false;
  const size_t lds = size_t(WS_NS) * WG_STAGE * sizeof(bf16_t) + 2 * sizeof(int) * size_t(g.n_exp);
  if (lds * WS_BPC > size_t(kLdsMax)) return hipErrorInvalidValue;  // too many experts
  if (!attr_set) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&wgrad_ws_kernel<MODE>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(wgrad_ws_kernel<MODE>, dim3(unsigned(WS_BPC * (cus < 8 ? 8 : cus))), dim3(WS_NT), lds, st, g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_backward_kernels(const BwdArgs& g, const float* P, int ks, const int32_t* idx,
                                   const int32_t* slot, const float* gate, const float* w_router,
                                   const bf16_t* dy, bf16_t* dx, float* dw_router, hipStream_t st,
                                   int stage) {
  const int T = g.T, K = g.K, E = g.E, S = g.n_exp - g.E, H = g.H, I = g.I;
  const int rows = g.TK + S * T;
  switch (stage) {
    case 0:  // expert-ordered copy of x
      hipLaunchKernelGGL(gather_rows_kernel, dim3(rows), dim3(256), 0, st, g.x, g.perm, T, g.TK, S,
                         H, g.xst);
      break;
    case 2:  // combine backward (without dgp; with dgp only the output gradients), tile prefixes
      hipLaunchKernelGGL(combine_bwd_kernel, dim3(T), dim3(256), 0, st, dy,
                         g.dgp != nullptr ? nullptr : g.yst, slot, gate, T, K, H, g.TK, S, g.dyst,
                         g.dg);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(bwd_tile_prefix_kernel, dim3(1), dim3(64), 0, st, g.counts, E, S, T, BG_M,
                         const_cast<int32_t*>(g.mt));
      if (g.mtd != nullptr) {
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL(bwd_tile_prefix_kernel, dim3(1), dim3(64), 0, st, g.counts, E, S, T,
                           DT_M, g.mtd);
      }
      break;
    case 3:  // router backward (with dgp: after the dH GEMM)
      hipLaunchKernelGGL(router_bwd_kernel, dim3((T + 255) / 256), dim3(256), 0, st, P, ks, idx,
                         slot, g.dg, T, E, K, g.dl, g.dlst, g.dgp, I / DG_N,
                         (long long)(g.TK + S * T), gate);
      break;
    case 4:  // dH = dY W_down with the SwiGLU backward
      if (g.mtd != nullptr) return launch_dgrad_tile<0>(g, unsigned(dgrad_max_tiles(T, K, E, S) * (I / DT_N)), st);
      hipLaunchKernelGGL(dgrad_gemm_kernel<0>, dim3(unsigned(bwd_max_row_tiles(T, K, E, S) * (I / DG_N))),
                         dim3(BG_NT), 0, st, g);
      break;
    case 5:  // dX = dG W_gate + dU W_up
      if (g.mtd != nullptr) return launch_dgrad_tile<1>(g, unsigned(dgrad_max_tiles(T, K, E, S) * (H / DT_N)), st);
      hipLaunchKernelGGL(dgrad_gemm_kernel<1>, dim3(unsigned(bwd_max_row_tiles(T, K, E, S) * (H / DG_N))),
                         dim3(BG_NT), 0, st, g);
      break;
    case 6: {  // weight gradients
      if (!g.wg_xcd) {  // more than 64 rows per routed expert on average: persistent
        hipError_t err = launch_wgrad_ws<0>(g, st);
        if (err == hipSuccess) err = launch_wgrad_ws<1>(g, st);  // dW_gate and dW_up
        return err;
      }
      const unsigned per_e = unsigned((H / BG_M) * (I / WG_N));
      const unsigned tiles = per_e * S + 8 * ((per_e * E + 7) / 8);  // slots past the tiles exit
      hipLaunchKernelGGL(wgrad_gemm_kernel<0>, dim3(tiles), dim3(BG_NT), 0, st, g);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(wgrad_gemm_kernel<1>, dim3(tiles), dim3(BG_NT), 0, st, g);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(wgrad_gemm_kernel<2>, dim3(tiles), dim3(BG_NT), 0, st, g);
      break;
    }
    case 7:  // router weight gradient: dW_r^T per expert, then transposed
      hipLaunchKernelGGL(dwr_kernel, dim3(E, (H / 4 + 255) / 256), dim3(256), 0, st, g.dlst, g.x,
                         g.perm, g.counts, g.offsets, H, g.dwrt);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(transpose_f32_kernel, dim3((H + 31) / 32, (E + 31) / 32), dim3(256), 0, st,
                         g.dwrt, E, H, dw_router);
      break;
    case 8:  // dx: W_r^T, then the fixed-order gather
      hipLaunchKernelGGL(transpose_f32_kernel, dim3((E + 31) / 32, (H + 31) / 32), dim3(256), 0, st,
                         w_router, H, E, g.wrt);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      hipLaunchKernelGGL(dx_kernel, dim3(T), dim3(256), 0, st, g.dxst, slot, idx, g.dl, g.wrt, T, K,
                         H, g.TK, S, dx);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
