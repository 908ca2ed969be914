// Backward of the MoE layer on E4M3 weights.
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §2.2 (FP8
// training framework).  Every GEMM of the expert backward takes E4M3
// operands: activations and activation gradients in 1x128 tiles (one scale
// per token row and 128 channels) where the product contracts over channels,
// weights in 128x128 blocks, and the products that contract over tokens (the
// weight gradients) in 128x1 tiles (one scale per channel and 128 consecutive
// rows of one expert).  The SwiGLU input is cached in E4M3 and its output is
// recomputed from that cache.  Products are summed exactly within a 128-wide
// K block by one MFMA and promoted to the float32 accumulator with the two
// scales, as in the forward.
//
// Steps (rows are staged rows: routed experts in expert order, then the
// shared expert's T rows):
//   G = Q(x) W_gate^T, U = Q(x) W_up^T (float32), cached as Q(G), Q(U);
//   H = SiLU(Q(G)) Q(U), quantised 1x128 for the down GEMM that recomputes Y
//   (with the same grouped GEMM);
//   dY = g dy, quantised 1x128;   dH = Q(dY) W_down;
//   dG = dH Q(U) SiLU'(Q(G)), dU = dH SiLU(Q(G)) (float32), quantised 1x128;
//   dX = Q(dG) W_gate + Q(dU) W_up;
//   dW_down = Q'(dY)^T Q'(H), dW_gate = Q'(dG)^T Q'(x), dW_up = Q'(dU)^T Q'(x)
//   with Q' the 128x1 tiles over each expert's rows.
//
// The data-gradient GEMMs contract over the weights' slow dimension: their
// weight operand is staged in LDS as it is stored ([K][N] k-rows) and read
// with the transposing ds_read_b64_tr_b8.  The 128x1 operands of the weight
// gradients are written transposed: per expert e, [C][Kp_e] codes with Kp_e =
// its rows rounded up to 128 (zero codes past its last row) and [C][Kp_e/128]
// scales.
#include <type_traits>

#include "bwd.h"
#include "common.h"
#include "lds_async.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- GEMM
// C[m][n] = sum over K blocks kb of sa[m][kb] sb[n][kb] sum_{k in kb} A[m][k] B[n][k]
// Tile 128 x 128, four waves of 64 x 64 (4 x 4 blocks of
// v_mfma_scale_f32_16x16x128_f8f6f4, one per 128-wide K block), two LDS
// stages filled one step ahead by buffer_load ... lds copies.  Operand bytes
// of lane l: row l % 16 of a 16-row block, 16-byte chunks l / 16 and
// l / 16 + 4 of the 128-byte K block (the same K map on both sides).
//
// GROUP 0 (row-grouped): expert e's staged rows against its [N][K] weight
//   matrix with 128x128 block scales ([N/128][K/128]), tiles over mt[]
//   (128-row tiles); optionally A rows gathered through perm from a [T][K]
//   matrix.  BN: the weight matrix is [K][N] with [K/128][N/128] scales.
// GROUP 1 (K-grouped): expert e's [M][Kp_e] A against its [N][Kp_e] B, both
//   with per-row scales; C is expert e's [M][N] float32 slice.
// NSRC == 2: C = A0 B0 + A1 B1 (same shapes), one accumulator.

constexpr int F8_T = 128;                       // tile rows and columns
constexpr int F8_NS = 2;                        // LDS stages
constexpr int F8_NT = 256;                      // four waves
constexpr int F8_OP = F8_T * 128;               // code bytes of one operand's stage
constexpr int F8_STAGE = 2 * F8_OP + 2 * F8_T * 4;  // A, B codes; A, B scales
constexpr int F8_CPW = F8_OP / 1024 / 4;        // 1 KB copies per operand and wave (4)

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

MOE_DEV void copy16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint8_t* dst) { copy_to_lds_async16(rs, voff, dst); }
MOE_DEV void copy4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint8_t* dst) { copy_to_lds_async4(rs, voff, dst); }

template <int GROUP, int NSRC, typename TO, bool BN>
__global__ __launch_bounds__(F8_NT, 2) void f8_gemm_kernel(F8GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[F8_NS * F8_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int c16 = lane & 15, g4 = lane >> 4;

  int e, m0, n0, rows, row_base = 0, KB, kp0 = 0;
  uint32_t a_bytes, as_bytes, b_bytes, bs_bytes, a_rowb, a_rows_s;
  if (GROUP == 0) {
    const int nN = g.N / F8_T;
    const int n_tasks = g.mt[g.n_exp] * nN;
    const int task = blockIdx.x;
    if (task >= n_tasks) return;  // uniform per workgroup, before any barrier
    int lo = 0, hi = g.n_exp - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.mt[mid] * nN <= task) lo = mid;
      else hi = mid - 1;
    }
    e = lo;
    const int n_mt = g.mt[e + 1] - g.mt[e];
    const int local = task - g.mt[e] * nN;
    const int nt = local / n_mt, mtile = local - nt * n_mt;
    const bool shared = e >= g.E;
    const int cnt = shared ? g.T : g.counts[e];
    row_base = shared ? g.TK + (e - g.E) * g.T : g.offsets[e];
    m0 = mtile * F8_T;
    n0 = nt * F8_T;
    rows = min(F8_T, cnt - m0);
    KB = g.K / 128;
    const uint32_t a_rows = g.perm ? uint32_t(g.T) : uint32_t(g.TK + (g.n_exp - g.E) * g.T);
    a_rowb = uint32_t(g.K);
    a_rows_s = uint32_t(KB);
    a_bytes = a_rows * a_rowb;
    as_bytes = a_rows * a_rows_s * 4u;
    b_bytes = uint32_t(g.N) * uint32_t(g.K);
    bs_bytes = uint32_t(g.N / 128) * uint32_t(KB) * 4u;
  } else {
    const int nM = g.M / F8_T, nN = g.N / F8_T;
    // experts in reverse order: the shared experts' tiles, which contract
    // over all T rows, start first instead of forming the launch's tail.
    // With g.xcd (decode-sized batches) the routed experts' tiles go to the
    // XCDs (workgroup b runs on XCD b % 8) in contiguous eighths, so each XCD
    // writes a contiguous eighth of the gradients; the shared tiles' count is
    // a multiple of 8 and the launch holds 8 ceil(routed tiles / 8) slots.
    const int per_e = nM * nN, sh_tiles = (g.n_exp - g.E) * per_e;
    int task = blockIdx.x;
    if (g.xcd && task >= sh_tiles) {
      const int b = task - sh_tiles, rt = g.E * per_e, per = (rt + 7) >> 3;
      const int j = b >> 3;
      task = sh_tiles + (b & 7) * per + j;
      if (j >= per || task >= sh_tiles + rt) return;  // uniform
    }
    const int eb = task / per_e;
    if (eb >= g.n_exp) return;
    e = g.n_exp - 1 - eb;
    const int rem = task - eb * per_e;
    m0 = (rem / nN) * F8_T;
    n0 = (rem % nN) * F8_T;
    rows = F8_T;
    kp0 = g.kp[e];
    const int kpe = g.kp[e + 1] - kp0;
    KB = kpe / 128;
    a_rowb = uint32_t(kpe);
    a_rows_s = uint32_t(KB);
    a_bytes = uint32_t(g.M) * a_rowb;
    as_bytes = uint32_t(g.M) * a_rows_s * 4u;
    b_bytes = uint32_t(g.N) * uint32_t(kpe);
    bs_bytes = uint32_t(g.N) * a_rows_s * 4u;
  }
  const int steps = NSRC * KB;

  // ---- operand buffers of source s
  auto a_base = [&](int s) -> const uint8_t* {
    const uint8_t* a = s ? g.a1 : g.a0;
    return GROUP == 0 ? a : a + (size_t)kp0 * g.M;
  };
  auto as_base = [&](int s) -> const float* {
    const float* a = s ? g.as1 : g.as0;
    return GROUP == 0 ? a : a + (size_t)(kp0 / 128) * g.M;
  };
  auto b_base = [&](int s) -> const uint8_t* {
    const uint8_t* b = s ? g.b1 : g.b0;
    return GROUP == 0 ? b + (size_t)e * g.N * g.K : b + (size_t)kp0 * g.N;
  };
  auto bs_base = [&](int s) -> const float* {
    const float* b = s ? g.bs1 : g.bs0;
    return GROUP == 0 ? b + (size_t)e * (g.N / 128) * KB : b + (size_t)(kp0 / 128) * g.N;
  };
  const __amdgpu_buffer_rsrc_t ar0 = buffer_rsrc(a_base(0), a_bytes);
  const __amdgpu_buffer_rsrc_t ar1 = NSRC == 2 ? buffer_rsrc(a_base(1), a_bytes) : ar0;
  const __amdgpu_buffer_rsrc_t sr0 = buffer_rsrc(as_base(0), as_bytes);
  const __amdgpu_buffer_rsrc_t sr1 = NSRC == 2 ? buffer_rsrc(as_base(1), as_bytes) : sr0;
  const __amdgpu_buffer_rsrc_t br0 = buffer_rsrc(b_base(0), b_bytes);
  const __amdgpu_buffer_rsrc_t br1 = NSRC == 2 ? buffer_rsrc(b_base(1), b_bytes) : br0;
  const __amdgpu_buffer_rsrc_t bsr = buffer_rsrc(bs_base(0), bs_bytes);  // GROUP 1 only

  // A row (in the A buffer) of tile row r; rows past the count read past the
  // buffer's end (zeros)
  auto a_row_ok = [&](int r) { return r < rows; };
  auto a_row = [&](int r) -> uint32_t {
    if (GROUP == 1) return uint32_t(m0 + r);
    const int sr = row_base + m0 + r;
    if (!g.perm) return uint32_t(sr);
    return uint32_t(sr < g.TK ? g.perm[sr] : m0 + r);  // shared rows: token m0 + r
  };
  // copy i of this wave covers tile rows 8 (4 wave + i) .. +7; lane l writes
  // LDS bytes 16 l of that 1 KB: row r0 + l/8, position l%8 = chunk (l%8)^(row%8)
  uint32_t aoff[F8_CPW], boff[F8_CPW];
#pragma unroll
  for (int i = 0; i < F8_CPW; ++i) {
    const int r = 8 * (F8_CPW * wave + i) + (lane >> 3);
    const uint32_t sw = uint32_t(((lane & 7) ^ (r & 7)) * 16);
    aoff[i] = a_row_ok(r) ? a_row(r) * a_rowb + sw : a_bytes;
    // BN: tile row r is k-row r of the [K][N] matrix, bytes n0 .. n0 + 127
    boff[i] = BN ? uint32_t(r) * uint32_t(g.N) + uint32_t(n0) + sw
                 : uint32_t(n0 + r) * (GROUP == 0 ? uint32_t(g.K) : a_rowb) + sw;
  }
  // one 4-byte scale copy per wave: waves 0, 1: A scales of tile rows
  // 64 w + l; waves 2, 3: B scales of tile rows 64 (w - 2) + l (GROUP 1), or
  // the A scales again (GROUP 0: the same bytes to the same slots)
  const int srow = 64 * (wave & 1) + lane;
  const bool bscale = GROUP == 1 && wave >= 2;
  const uint32_t soff = bscale ? uint32_t(n0 + srow) * a_rows_s * 4u
                               : (a_row_ok(srow) ? a_row(srow) * a_rows_s * 4u : as_bytes);
  const int sdst = (bscale ? F8_T * 4 : 0) + 4 * 64 * (wave & 1);

  // GROUP 0: the weight-block scales of this tile's 128 columns, lane l
  // holding K blocks l and 64 + l of each source (read with v_readlane)
  float sbv[NSRC][2];
  if (GROUP == 0) {
#pragma unroll
    for (int s = 0; s < NSRC; ++s) {
      // block (n0 / 128, kb) of [N/128][K/128] scales, or (kb, n0 / 128) of [K/128][N/128] (BN)
      const float* p = bs_base(s) + (BN ? (size_t)(n0 / 128) : (size_t)(n0 / 128) * KB);
      const int stride = BN ? g.N / 128 : 1;
#pragma unroll
      for (int c = 0; c < 2; ++c) sbv[s][c] = p[(size_t)min(64 * c + lane, KB - 1) * stride];
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  auto issue = [&](int step) {
    const bool s1 = NSRC == 2 && step >= KB;
    const uint32_t kb = uint32_t(s1 ? step - KB : step);
    uint8_t* st = smem + (step % F8_NS) * F8_STAGE;
#pragma unroll
    for (int i = 0; i < F8_CPW; ++i)
      copy16(s1 ? ar1 : ar0, aoff[i] + kb * 128u, st + 8 * (F8_CPW * wave + i) * 128);
#pragma unroll
    for (int i = 0; i < F8_CPW; ++i)
      copy16(s1 ? br1 : br0, boff[i] + kb * (BN ? 128u * uint32_t(g.N) : 128u),
             st + F8_OP + 8 * (F8_CPW * wave + i) * 128);
    copy4(bscale ? bsr : (s1 ? sr1 : sr0), soff + kb * 4u, st + 2 * F8_OP + sdst);
  };

  // active 16-row blocks of this wave (uniform)
  const int rb_act = __builtin_amdgcn_readfirstlane(max(0, min(4, (rows - 64 * wm + 15) >> 4)));

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const uint8_t* base, int r) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + r * 128 + ((g4 ^ (r & 7)) << 4));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + r * 128 + (((g4 + 4) ^ (r & 7)) << 4));
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  // The same operand of columns c0 .. c0 + 15 from a stage of k-rows (128 k x
  // 128 columns, chunk c of k-row r at position c ^ (r % 8)), by four
  // ds_read_b64_tr_b8: in each 16-lane group, source lane s addresses 8 bytes
  // of k-row kq + s/2 (columns c0 + 8 (s%2) ..), and lane d receives byte d%8
  // of source lane 2 j + d/8 as its byte j, i.e. k-rows kq .. kq + 7 of
  // column c0 + d.  Lane l's k-rows: 16 (l/16) .. + 15 and 64 + 16 (l/16) .. + 15.
  auto frag_kn = [&](const uint8_t* base, int c0) {
    const int s = lane & 15;
    v2i32 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = 16 * g4 + 64 * (i >> 1) + 8 * (i & 1) + (s >> 1);
      const uint8_t* p = base + kr * 128 + ((((c0 >> 4) ^ (kr & 7))) << 4) + 8 * (s & 1);
      q[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i32*)((__attribute__((address_space(3))) uint8_t*)p));
    }
    return i32x8{q[0].x, q[0].y, q[1].x, q[1].y, q[2].x, q[2].y, q[3].x, q[3].y};
  };

  // One K step of NRB active row blocks.  The weight-side fragment is the
  // MFMA's first operand, so a lane's four results of a block are four
  // adjacent columns of one row: GROUP 0 promotes them with one scale
  // product per row block.  The MFMA of pair p + 1 is issued before the
  // promotion of pair p, so the vector ALU works while the matrix core does;
  // all of the step's fragments are read up front.
  auto step_body = [&](int step, auto nrb_c) {
    constexpr int NRB = decltype(nrb_c)::value;
    if constexpr (NRB > 0) {
      const uint8_t* st = smem + (step % F8_NS) * F8_STAGE;
      const float* scA = reinterpret_cast<const float*>(st + 2 * F8_OP);
      const float* scB = scA + F8_T;
      float sbb = 1.f;
      if (GROUP == 0) {
        const bool s1 = NSRC == 2 && step >= KB;
        const int kb = s1 ? step - KB : step;
        const float v = kb < 64 ? sbv[s1 ? NSRC - 1 : 0][0] : sbv[s1 ? NSRC - 1 : 0][1];
        sbb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kb & 63));
      }
      i32x8 bf[4];
      f32x4 sbq[4];  // GROUP 1: the scales of the lane's four columns of block j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf[j] = BN ? frag_kn(st + F8_OP, 64 * wn + 16 * j) : frag(st + F8_OP, 64 * wn + 16 * j + c16);
        if (GROUP == 1) sbq[j] = *reinterpret_cast<const f32x4*>(scB + 64 * wn + 16 * j + 4 * g4);
      }
      i32x8 af[NRB];
      float sa[NRB];
#pragma unroll
      for (int i = 0; i < NRB; ++i) {
        af[i] = frag(st, 64 * wm + 16 * i + c16);
        sa[i] = scA[64 * wm + 16 * i + c16];
      }
      constexpr int P = 4 * NRB;
      f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[0], af[0], zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int i = p >> 2, j = p & 3;
        f32x4 u = zero;
        if (p + 1 < P)
          u = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[(p + 1) & 3], af[(p + 1) >> 2], zero, 0, 0,
                                                               0, 127, 0, 127);
        if (GROUP == 0) {
          const float sc = sa[i] * sbb;
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(t[v], sc, acc[i][j][v]);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(t[v], sa[i] * sbq[j][v], acc[i][j][v]);
        }
        if (p + 1 < P) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // the next MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, GROUP == 0 ? 4 : 8, 0);  // this promotion
        }
        t = u;
      }
    }
  };
  auto mainloop = [&](auto nrb_c) {
    if (steps > 0) issue(0);
    for (int step = 0; step < steps; ++step) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's copies of step landed
      __syncthreads();                     // everyone's; everyone is done with step - 1
      if (step + 1 < steps) issue(step + 1);
      step_body(step, nrb_c);
    }
  };
  switch (rb_act) {
    case 4: mainloop(std::integral_constant<int, 4>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    default: mainloop(std::integral_constant<int, 0>{}); break;
  }

  // ---- epilogue.  16x16 accumulator v of lane l: row l%16, column 4 (l/16) + v
  if (GROUP == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= rb_act) continue;
      const int r = 64 * wm + 16 * i + c16;
      if (r >= rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        TO* o = static_cast<TO*>(g.out) + (size_t)(row_base + m0 + r) * g.N + n0 + 64 * wn + 16 * j + 4 * g4;
        if constexpr (std::is_same<TO, float>::value) {
          *reinterpret_cast<f32x4*>(o) = acc[i][j];
        } else {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          const uint32_t p0 = uint32_t(from_f32<TO>(acc[i][j][0])) | (uint32_t(from_f32<TO>(acc[i][j][1])) << 16);
          const uint32_t p1 = uint32_t(from_f32<TO>(acc[i][j][2])) | (uint32_t(from_f32<TO>(acc[i][j][3])) << 16);
          *reinterpret_cast<u32x2*>(o) = u32x2{p0, p1};
        }
      }
    }
  } else {
    // the float32 tile goes through LDS (the two stages hold exactly 128 rows
    // of 132 floats) so that every store is 16 bytes per lane, 1 KB per wave:
    // two whole 512-byte rows of the output.  Measured against storing the
    // 16x16 blocks from registers (64-byte row pieces): 10.5 -> 9.6 ms for
    // the three weight-gradient launches at 4096 tokens.
    constexpr int LD = F8_T + 4;
    static_assert(F8_T * LD * 4 <= F8_NS * F8_STAGE, "the output tile must fit the stages");
    float* tile = reinterpret_cast<float*>(smem);
    __syncthreads();  // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(tile + (64 * wm + 16 * i + c16) * LD + 64 * wn + 16 * j + 4 * g4) = acc[i][j];
    __syncthreads();
    float* out = static_cast<float*>(g.out) + ((size_t)e * g.M + m0) * g.N + n0;
#pragma unroll
    for (int p = 0; p < F8_T / 8; ++p) {
      const int r = 8 * p + (tid >> 5), c = 4 * (tid & 31);
      const f32x4 v = *reinterpret_cast<const f32x4*>(tile + r * LD + c);
      // written once: non-temporal
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + (size_t)r * g.N + c));
    }
  }
}

// ---------------------------------------------------------------- small kernels

// mt[e]: prefix of 128-row tiles; kp[e]: prefix of rows rounded up to 128
// (routed counts, then the shared experts' T rows)
__global__ __launch_bounds__(64) void f8_prefix_kernel(const int32_t* __restrict__ counts, int E,
                                                       int S, int T, int32_t* __restrict__ mt,
                                                       int32_t* __restrict__ kp) {
  if (threadIdx.x != 0) return;
  int a = 0, b = 0;
  for (int e = 0; e < E + S; ++e) {
    mt[e] = a;
    kp[e] = b;
    const int c = e < E ? counts[e] : T;
    a += (c + 127) / 128;
    b += (c + 127) / 128 * 128;
  }
  mt[E + S] = a;
  kp[E + S] = b;
}

// 1x128 quantisation of 8 values per lane, 16 lanes per slice: scale =
// amax / 448 (1 where that is zero), codes RNE(v / scale); returns the
// codes packed in two words
MOE_DEV uint2 quant_slice8(const float (&v)[8], float& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  scale = e4m3_scale(amax);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_encode(v[i] / scale) << (8 * i);
    hi |= e4m3_encode(v[4 + i] / scale) << (8 * i);
  }
  return uint2{lo, hi};
}

MOE_DEV void decode8(uint2 c, float s, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = e4m3_decode((c.x >> (8 * i)) & 0xffu) * s;
    v[4 + i] = e4m3_decode((c.y >> (8 * i)) & 0xffu) * s;
  }
}

MOE_DEV float sigm8(float v) { return 1.0f / (1.0f + expf(-v)); }

// H = SiLU(G) U of one element of the cached (dequantised) SwiGLU input
MOE_DEV float swiglu_h(float gv, float uv) { return gv * sigm8(gv) * uv; }

// float32 rows [rows][C] -> 1x128 codes and scales
__global__ __launch_bounds__(256) void quant_f32_kernel(const float* __restrict__ x,
                                                        long long n_slices, int C,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ scales) {
  const long long slice = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool ok = slice < n_slices;
  const long long sl = ok ? slice : n_slices - 1;
  const int spr = C / 128;
  const long long row = sl / spr;
  const size_t at = (size_t)row * C + size_t(sl - row * spr) * 128 + 8 * j;
  const f32x4 a = *reinterpret_cast<const f32x4*>(x + at);
  const f32x4 b = *reinterpret_cast<const f32x4*>(x + at + 4);
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  float scale;
  const uint2 c = quant_slice8(v, scale);
  if (ok) {
    *reinterpret_cast<uint2*>(q + at) = c;
    if (j == 0) scales[sl] = scale;
  }
}

// H from the cached G, U codes, quantised 1x128 (the down GEMM's input)
__global__ __launch_bounds__(256) void swiglu_fp8_kernel(const uint8_t* __restrict__ gq,
                                                         const float* __restrict__ gs,
                                                         const uint8_t* __restrict__ uq,
                                                         const float* __restrict__ us,
                                                         long long n_slices, uint8_t* __restrict__ hq,
                                                         float* __restrict__ hs) {
  const long long slice = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool ok = slice < n_slices;
  const long long sl = ok ? slice : n_slices - 1;
  const size_t at = (size_t)sl * 128 + 8 * j;  // rows of I columns: slice sl starts at 128 sl
  float gv[8], uv[8], h[8];
  decode8(*reinterpret_cast<const uint2*>(gq + at), gs[sl], gv);
  decode8(*reinterpret_cast<const uint2*>(uq + at), us[sl], uv);
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = swiglu_h(gv[i], uv[i]);
  float scale;
  const uint2 c = quant_slice8(h, scale);
  if (ok) {
    *reinterpret_cast<uint2*>(hq + at) = c;
    if (j == 0) hs[sl] = scale;
  }
}

// dY of every staged row (routed: g_k dy_t at row slot(t, k); shared: dy_t),
// quantised 1x128; also the gate of each routed staged row
__global__ __launch_bounds__(256) void quant_dy_kernel(const bf16_t* __restrict__ dy,
                                                       const int32_t* __restrict__ slot,
                                                       const float* __restrict__ gate, int T,
                                                       int K, int S, int H, int TK,
                                                       long long n_slices, uint8_t* __restrict__ q,
                                                       float* __restrict__ scales,
                                                       float* __restrict__ rowgate) {
  const long long slice = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool ok = slice < n_slices;
  const long long sl = ok ? slice : n_slices - 1;
  const int spr = H / 128;
  const long long tj = sl / spr;
  const int cs = int(sl - tj * spr);
  const int t = int(tj / (K + S)), k = int(tj - (long long)t * (K + S));
  const int row = k < K ? slot[t * K + k] : TK + (k - K) * T + t;
  const float gk = k < K ? gate[t * K + k] : 1.0f;
  const u32x4 raw = *reinterpret_cast<const u32x4*>(dy + (size_t)t * H + cs * 128 + 8 * j);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = gk * __uint_as_float(raw[i] << 16);
    v[2 * i + 1] = gk * __uint_as_float(raw[i] & 0xffff0000u);
  }
  float scale;
  const uint2 c = quant_slice8(v, scale);
  if (ok) {
    *reinterpret_cast<uint2*>(q + (size_t)row * H + cs * 128 + 8 * j) = c;
    if (j == 0) {
      scales[(size_t)row * spr + cs] = scale;
      if (k < K && cs == 0) rowgate[row] = gk;
    }
  }
}

// SwiGLU backward from dH (float32) and the cached G, U:
// dU = dH SiLU(G), dG = dH U SiLU'(G); float32 copies and 1x128 codes
__global__ __launch_bounds__(256) void swiglu_bwd_fp8_kernel(
    const float* __restrict__ dh, const uint8_t* __restrict__ gq, const float* __restrict__ gs,
    const uint8_t* __restrict__ uq, const float* __restrict__ us, long long n_slices,
    float* __restrict__ dg32, float* __restrict__ du32, uint8_t* __restrict__ dgq,
    float* __restrict__ dgs, uint8_t* __restrict__ duq, float* __restrict__ dus) {
  const long long slice = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool ok = slice < n_slices;
  const long long sl = ok ? slice : n_slices - 1;
  const size_t at = (size_t)sl * 128 + 8 * j;
  float gv[8], uv[8], dG[8], dU[8];
  decode8(*reinterpret_cast<const uint2*>(gq + at), gs[sl], gv);
  decode8(*reinterpret_cast<const uint2*>(uq + at), us[sl], uv);
  const f32x4 a = *reinterpret_cast<const f32x4*>(dh + at);
  const f32x4 b = *reinterpret_cast<const f32x4*>(dh + at + 4);
  const float d[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sg = sigm8(gv[i]);
    dU[i] = d[i] * (gv[i] * sg);
    dG[i] = d[i] * uv[i] * (sg * (1.0f + gv[i] * (1.0f - sg)));
  }
  float sgs, sus;
  const uint2 cg = quant_slice8(dG, sgs);
  const uint2 cu = quant_slice8(dU, sus);
  if (ok) {
    *reinterpret_cast<f32x4*>(dg32 + at) = f32x4{dG[0], dG[1], dG[2], dG[3]};
    *reinterpret_cast<f32x4*>(dg32 + at + 4) = f32x4{dG[4], dG[5], dG[6], dG[7]};
    *reinterpret_cast<f32x4*>(du32 + at) = f32x4{dU[0], dU[1], dU[2], dU[3]};
    *reinterpret_cast<f32x4*>(du32 + at + 4) = f32x4{dU[4], dU[5], dU[6], dU[7]};
    *reinterpret_cast<uint2*>(dgq + at) = cg;
    *reinterpret_cast<uint2*>(duq + at) = cu;
    if (j == 0) {
      dgs[sl] = sgs;
      dus[sl] = sus;
    }
  }
}

// ---------------------------------------------------------------- 128x1 re-tiling
// Block (64-column chunk, 128-row block of one expert): the block's values
// (float32) go through LDS; each column's max-abs over the 128 rows gives its
// scale; the codes are written transposed, 128 rows of one column contiguous.
enum RetileSrc { RT_DY = 0, RT_X = 1, RT_H = 2, RT_F32 = 3 };

struct RetileArgs {
  const bf16_t* dy;        // RT_DY: [T][C]
  const float* rowgate;    // RT_DY: gate of each routed staged row
  const bf16_t* x;         // RT_X: [T][C]
  const uint8_t* gq;       // RT_H: cached G, U codes [rows][C] and scales
  const float* gs;
  const uint8_t* uq;
  const float* us;
  const float* f32;        // RT_F32: [rows][C]
  const int32_t* perm;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* kp;
  uint8_t* out;            // per expert e at kp[e] C: [C][Kp_e]
  float* outs;             // per expert e at kp[e]/128 C: [C][Kp_e/128]
  int E, n_exp, T, TK, C;
};

template <int SRC>
__global__ __launch_bounds__(256) void retile_kernel(RetileArgs g) {
  __shared__ float tile[128][65];
  const int nblk = g.kp[g.n_exp] / 128;
  const int gb = blockIdx.y;
  if (gb >= nblk) return;  // uniform
  int lo = 0, hi = g.n_exp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.kp[mid] / 128 <= gb) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int rb = gb - g.kp[e] / 128;
  const int kpe = g.kp[e + 1] - g.kp[e];
  const bool shared = e >= g.E;
  const int cnt = shared ? g.T : g.counts[e];
  const int row_base = shared ? g.TK + (e - g.E) * g.T : g.offsets[e];
  const int c0 = blockIdx.x * 64;
  const int C = g.C;

  {  // load: thread (row r, 32 columns from 32 h)
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const int lr = rb * 128 + r;
    const int cb = c0 + 32 * h;
    float v[32];
    if (lr < cnt) {
      const int sr = row_base + lr;
      const int t = shared ? lr : (SRC == RT_DY || SRC == RT_X ? g.perm[sr] : 0);
      if (SRC == RT_DY || SRC == RT_X) {
        const bf16_t* p = (SRC == RT_DY ? g.dy : g.x) + (size_t)t * C + cb;
        const float gk = SRC == RT_DY && !shared ? g.rowgate[sr] : 1.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 raw = reinterpret_cast<const u32x4*>(p)[q];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = __uint_as_float(raw[i] << 16), b = __uint_as_float(raw[i] & 0xffff0000u);
            v[8 * q + 2 * i] = SRC == RT_DY ? gk * a : a;
            v[8 * q + 2 * i + 1] = SRC == RT_DY ? gk * b : b;
          }
        }
      } else if (SRC == RT_H) {
        const size_t at = (size_t)sr * C + cb;
        const float sgv = g.gs[(size_t)sr * (C / 128) + cb / 128];
        const float suv = g.us[(size_t)sr * (C / 128) + cb / 128];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float gv[8], uv[8];
          decode8(*reinterpret_cast<const uint2*>(g.gq + at + 8 * q), sgv, gv);
          decode8(*reinterpret_cast<const uint2*>(g.uq + at + 8 * q), suv, uv);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[8 * q + i] = swiglu_h(gv[i], uv[i]);
        }
      } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(g.f32 + (size_t)sr * C + cb);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const f32x4 a = p[q];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * q + i] = a[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) tile[r][32 * h + i] = v[i];
  }
  __syncthreads();
  // thread (column c, rows 32 q .. 32 q + 31)
  const int c = threadIdx.x >> 2, q = threadIdx.x & 3;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(tile[32 * q + i][c]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
  const float scale = e4m3_scale(amax);
  u32x4 w0, w1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a |= e4m3_encode(tile[32 * q + 4 * i + k][c] / scale) << (8 * k);
      b |= e4m3_encode(tile[32 * q + 16 + 4 * i + k][c] / scale) << (8 * k);
    }
    w0[i] = a;
    w1[i] = b;
  }
  uint8_t* o = g.out + (size_t)g.kp[e] * C + (size_t)(c0 + c) * kpe + rb * 128 + 32 * q;
  reinterpret_cast<u32x4*>(o)[0] = w0;
  reinterpret_cast<u32x4*>(o)[1] = w1;
  if (q == 0) g.outs[(size_t)(g.kp[e] / 128) * C + (size_t)(c0 + c) * (kpe / 128) + rb] = scale;
}

template <int GROUP, int NSRC, typename TO, bool BN = false>
hipError_t launch_gemm(const F8GemmArgs& a, unsigned blocks, hipStream_t st) {
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((f8_gemm_kernel<GROUP, NSRC, TO, BN>), dim3(blocks), dim3(F8_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int f8_max_row_tiles(int T, int K, int E, int S) {
  return (T * K + F8_T - 1) / F8_T + E + S * ((T + F8_T - 1) / F8_T);
}


hipError_t launch_backward_fp8(const BwdArgs8& g, hipStream_t st, int stage) {
  const int T = g.T, K = g.K, E = g.E, S = g.n_exp - g.E, H = g.H, I = g.I, n = g.n_exp;
  const int rows = g.TK + S * T;
  const unsigned mtiles = unsigned(f8_max_row_tiles(T, K, E, S));
  auto slices_grid = [](long long n_slices) { return dim3(unsigned((n_slices + 15) / 16)); };
  hipError_t err;
#define F8_TRY(x)                               \
  do {                                          \
    if ((err = (x)) != hipSuccess) return err;  \
  } while (0)
  auto last = [] { return hipGetLastError(); };
  switch (stage) {
    case 1:  // tile and padded-row prefixes
      hipLaunchKernelGGL(f8_prefix_kernel, dim3(1), dim3(64), 0, st, g.counts, E, S, T, g.mt,
                         g.kp);
      break;
    case 2: {  // G, U (float32) -> cached Q(G), Q(U); H -> Q(H); Y
      F8GemmArgs a{};
      a.a0 = g.xq;
      a.as0 = g.xs;
      a.perm = g.perm;
      a.counts = g.counts;
      a.offsets = g.offsets;
      a.mt = g.mt;
      a.E = E;
      a.n_exp = n;
      a.T = T;
      a.TK = g.TK;
      a.N = I;
      a.K = H;
      a.b0 = g.w_gate;
      a.bs0 = g.s_gate;
      a.out = g.f32a;
      F8_TRY((launch_gemm<0, 1, float>(a, mtiles * (I / F8_T), st)));
      a.b0 = g.w_up;
      a.bs0 = g.s_up;
      a.out = g.f32b;
      F8_TRY((launch_gemm<0, 1, float>(a, mtiles * (I / F8_T), st)));
      const long long ns = (long long)rows * (I / 128);
      hipLaunchKernelGGL(quant_f32_kernel, slices_grid(ns), dim3(256), 0, st, g.f32a, ns, I, g.gq,
                         g.gs);
      F8_TRY(last());
      hipLaunchKernelGGL(quant_f32_kernel, slices_grid(ns), dim3(256), 0, st, g.f32b, ns, I, g.uq,
                         g.us);
      F8_TRY(last());
      hipLaunchKernelGGL(swiglu_fp8_kernel, slices_grid(ns), dim3(256), 0, st, g.gq, g.gs, g.uq,
                         g.us, ns, g.hq, g.hs);
      F8_TRY(last());
      // Y = Q(H) W_down^T, bf16 staged rows (for the gate gradients)
      a.a0 = g.hq;
      a.as0 = g.hs;
      a.perm = nullptr;
      a.b0 = g.w_down;
      a.bs0 = g.s_down;
      a.out = g.yst;
      a.N = H;
      a.K = I;
      F8_TRY((launch_gemm<0, 1, bf16_t>(a, mtiles * (H / F8_T), st)));
      break;
    }
    case 3: {  // Q(dY) and the gate of each routed staged row
      const long long ns = (long long)T * (K + S) * (H / 128);
      hipLaunchKernelGGL(quant_dy_kernel, slices_grid(ns), dim3(256), 0, st, g.dy, g.slot, g.gate,
                         T, K, S, H, g.TK, ns, g.dyq, g.dys, g.rowgate);
      break;
    }
    case 4: {  // dH = Q(dY) W_down, then the SwiGLU backward
      F8GemmArgs a{};
      a.a0 = g.dyq;
      a.as0 = g.dys;
      a.b0 = g.w_down;  // [H][I]: k-rows of the contraction over H
      a.bs0 = g.s_down;
      a.out = g.f32a;
      a.counts = g.counts;
      a.offsets = g.offsets;
      a.mt = g.mt;
      a.E = E;
      a.n_exp = n;
      a.T = T;
      a.TK = g.TK;
      a.N = I;
      a.K = H;
      F8_TRY((launch_gemm<0, 1, float, true>(a, mtiles * (I / F8_T), st)));
      const long long ns = (long long)rows * (I / 128);
      hipLaunchKernelGGL(swiglu_bwd_fp8_kernel, slices_grid(ns), dim3(256), 0, st, g.f32a, g.gq,
                         g.gs, g.uq, g.us, ns, g.dg32, g.du32, g.dgq, g.dgs, g.duq, g.dus);
      break;
    }
    case 5: {  // dX = Q(dG) W_gate + Q(dU) W_up, bf16 staged rows
      F8GemmArgs a{};
      a.a0 = g.dgq;
      a.as0 = g.dgs;
      a.b0 = g.w_gate;  // [I][H]: k-rows of the contraction over I
      a.bs0 = g.s_gate;
      a.a1 = g.duq;
      a.as1 = g.dus;
      a.b1 = g.w_up;
      a.bs1 = g.s_up;
      a.out = g.dxst;
      a.counts = g.counts;
      a.offsets = g.offsets;
      a.mt = g.mt;
      a.E = E;
      a.n_exp = n;
      a.T = T;
      a.TK = g.TK;
      a.N = H;
      a.K = I;
      F8_TRY((launch_gemm<0, 2, bf16_t, true>(a, mtiles * (H / F8_T), st)));
      break;
    }
    case 6: {  // 128x1 operands of the weight gradients
      RetileArgs r{};
      r.dy = g.dy;
      r.rowgate = g.rowgate;
      r.x = g.x;
      r.gq = g.gq;
      r.gs = g.gs;
      r.uq = g.uq;
      r.us = g.us;
      r.perm = g.perm;
      r.counts = g.counts;
      r.offsets = g.offsets;
      r.kp = g.kp;
      r.E = E;
      r.n_exp = n;
      r.T = T;
      r.TK = g.TK;
      const unsigned kb = mtiles;  // 128-row blocks: the same count as the row tiles
      r.C = H;
      r.out = g.dyT;
      r.outs = g.dysT;
      hipLaunchKernelGGL(retile_kernel<RT_DY>, dim3(H / 64, kb), dim3(256), 0, st, r);
      F8_TRY(last());
      r.out = g.xT;
      r.outs = g.xsT;
      hipLaunchKernelGGL(retile_kernel<RT_X>, dim3(H / 64, kb), dim3(256), 0, st, r);
      F8_TRY(last());
      r.C = I;
      r.out = g.hT;
      r.outs = g.hsT;
      hipLaunchKernelGGL(retile_kernel<RT_H>, dim3(I / 64, kb), dim3(256), 0, st, r);
      F8_TRY(last());
      r.f32 = g.dg32;
      r.out = g.dgT;
      r.outs = g.dgsT;
      hipLaunchKernelGGL(retile_kernel<RT_F32>, dim3(I / 64, kb), dim3(256), 0, st, r);
      F8_TRY(last());
      r.f32 = g.du32;
      r.out = g.duT;
      r.outs = g.dusT;
      hipLaunchKernelGGL(retile_kernel<RT_F32>, dim3(I / 64, kb), dim3(256), 0, st, r);
      break;
    }
    case 7: {  // weight gradients from the 128x1 operands
      F8GemmArgs a{};
      a.kp = g.kp;
      a.E = E;
      a.n_exp = n;
      a.T = T;
      a.TK = g.TK;
      a.xcd = int64_t(T) * K <= int64_t(64) * E;  // decode-sized: at most 64 rows per expert
      const unsigned per_e = unsigned((H / F8_T) * (I / F8_T));
      const unsigned wtiles = per_e * unsigned(S) + 8 * ((per_e * unsigned(E) + 7) / 8);
      // dW_down [H][I] = Q'(dY)^T Q'(H)
      a.a0 = g.dyT;
      a.as0 = g.dysT;
      a.b0 = g.hT;
      a.bs0 = g.hsT;
      a.out = g.dw_down;
      a.M = H;
      a.N = I;
      F8_TRY((launch_gemm<1, 1, float>(a, wtiles, st)));
      // dW_gate, dW_up [I][H] = Q'(dG)^T Q'(x), Q'(dU)^T Q'(x)
      a.M = I;
      a.N = H;
      a.b0 = g.xT;
      a.bs0 = g.xsT;
      a.a0 = g.dgT;
      a.as0 = g.dgsT;
      a.out = g.dw_gate;
      F8_TRY((launch_gemm<1, 1, float>(a, wtiles, st)));
      a.a0 = g.duT;
      a.as0 = g.dusT;
      a.out = g.dw_up;
      F8_TRY((launch_gemm<1, 1, float>(a, wtiles, st)));
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
#undef F8_TRY
  return hipGetLastError();
}

}  // namespace moe
