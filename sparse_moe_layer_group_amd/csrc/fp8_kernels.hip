// FP8 (OCP E4M3FN) path: online 1x128 activation quantisation and the
// block-scaled grouped expert GEMM.
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §2.2 (FP8
// training framework): weights carry one float32 scale per 128x128 block,
// activations one per 1x128 slice of a token row, taken from the slice's
// current max-abs value; the products of each 128-wide K block are summed at
// full precision and multiplied by the two scales before they join the
// float32 accumulator.
//
// Quantiser: scale = amax / 448 in float32 (1 where that is zero), code =
// round-to-nearest-even of the float32 quotient v / scale (IEEE division),
// saturated to +-448.  The encoder is integer arithmetic on the float32 bits,
// so the codes do not depend on a hardware conversion mode.
//
// GEMM: see the comment above tile_gemm_fp8_kernel.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------- quantiser
// One 16-lane group per 1x128 slice: lane j holds elements 8j..8j+7.
__global__ __launch_bounds__(256) void quant_1x128_kernel(const bf16_t* __restrict__ x,
                                                          long long n_slices, int C,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ scales) {
  const long long slice = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool ok = slice < n_slices;
  const long long sl = ok ? slice : n_slices - 1;
  const int spr = C / 128;  // slices per row
  const long long row = sl / spr;
  const int col = int(sl - row * spr) * 128 + 8 * j;
  const u32x4 raw = *reinterpret_cast<const u32x4*>(x + row * C + col);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(raw[i] << 16);
    v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const float scale = e4m3_scale(amax);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_encode(v[i] / scale) << (8 * i);
    hi |= e4m3_encode(v[4 + i] / scale) << (8 * i);
  }
  if (ok) {
    *reinterpret_cast<uint2*>(q + row * C + col) = uint2{lo, hi};
    if (j == 0) scales[sl] = scale;
  }
}

hipError_t launch_quant_1x128(const bf16_t* x, long long rows, int C, uint8_t* q, float* scales,
                              hipStream_t st) {
  const long long n = rows * (C / 128);
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 15) / 16;
  hipLaunchKernelGGL(quant_1x128_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, C, q,
                     scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp8 GEMM
// Tile: kTileM8 (192) token rows x 256 weight rows.  Eight waves, two per
// SIMD; wave w owns 32 weight rows (gate/up: 16 columns of W_gate and the
// same 16 of W_up; down: 32 columns of W_down) against all 192 token rows, as
// 2 x 12 blocks of v_mfma_scale_f32_16x16x128_f8f6f4.  One such MFMA covers a
// whole 128-wide K block, so its result is the block's full-precision
// partial product: it is scaled by (row scale * weight-block scale) and added
// to the float32 accumulator at once (hardware block scales left at 1).
//
// The weight fragment is the MFMA's first operand, so a lane's four results
// of a block are four adjacent output columns of one token row: they share
// one row scale and one weight-block scale, and the promotion takes one
// multiply per lane and block pair (two for gate/up) besides the four
// multiply-adds per block.  (With the token rows as the first operand each
// result had a row of its own: one multiply per result, 8 rather than 5
// vector instructions per MFMA for gate/up, and four times the LDS bytes for
// the row scales.)  The MFMAs of row block i + 1 are issued before the
// promotion of block i, so the vector ALU works while the matrix core does.
//
// Operand bytes: lane l holds, for its row (token or weight) l % 16, the two
// 16-byte chunks g and g + 4 of the 128-byte block, g = l / 16.  Both
// operands use the same lane -> K map, so the dot product is unchanged.
//
// Copies (buffer_load ... lds, 1 KB = 8 rows x 128 bytes per wave
// instruction; chunk c of row r stored at position c ^ (r % 8)):
//   - weight rows: each wave copies its own 32 rows into a private LDS ring
//     of FS_NSB blocks; a block's stage is refilled as soon as the wave has
//     read its fragments into registers, so FS_NSB blocks (64 KB per CU)
//     are in flight while one is multiplied;
//   - token rows and their scales: shared by all waves, a ring of FS_NSA
//     blocks, FS_NSA - 1 ahead.
// The waits are explicit vmcnt counts.  Per block kb: wait until this wave's
// copies of kb have landed (a wave's copies complete in issue order),
// workgroup barrier (everyone's token rows of kb are in LDS and everyone is
// done with kb-1), read the weight fragments of kb, issue the token copies of
// kb+2 into the stage of kb-1 and the weight copies of kb+2 into the stage
// just read, multiply block kb.  Blocks past the end re-read the last block
// so that every iteration issues the same copies.
//
// Gate/up tiles hold 128 columns of W_gate and the same 128 of W_up, exactly
// one 1x128 slice of the SwiGLU output H: the epilogue forms SiLU(gate) * up,
// reduces each row's max-abs across the eight waves through LDS, and writes H
// as E4M3 codes (four adjacent columns per 4-byte store) plus one scale per
// row.
//
// Measured at 4096 tokens, gate/up on one box: 2300 us as first built (token
// rows as the first operand, MFMAs and promotion of a block back to back),
// 2160 us with the promotion of block i after the MFMAs of block i + 1, 1910
// us with the weights as the first operand.  Token rows two blocks ahead
// instead of one (with two weight blocks in flight instead of three) changed
// gate/up by under 1% and down by -2%.  A per-workgroup rotation of the K
// order measured no faster.
namespace {

constexpr int FS_TBM = kTileM8;                  // token rows per tile
constexpr int FS_RB = FS_TBM / 16;               // 16-row MFMA blocks
constexpr int FS_TBN = 256;                      // weight rows per tile
constexpr int FS_NWAVE = 8, FS_NTHREAD = 64 * FS_NWAVE;
constexpr int FS_NSA = 3;                        // shared LDS stages of token rows
constexpr int FS_NSB = 2;                        // private LDS stages of weight rows per wave
constexpr int FS_ACOPY = FS_TBM / 8 / FS_NWAVE;  // 1 KB token-row copies per wave per block
constexpr int FS_BCOPY = FS_TBN / 8 / FS_NWAVE;  // 1 KB weight-row copies per wave per block
constexpr int FS_ASTAGE = FS_TBM * 128;          // code bytes per token stage
constexpr int FS_STAGE = FS_ASTAGE + FS_TBM * 4; // + one float32 scale per row
constexpr int FS_BWAVE = FS_BCOPY * 1024;        // bytes of one wave's weight block
constexpr int FS_BBASE = FS_NSA * FS_STAGE;      // start of the weight rings
constexpr int FS_ACOPIES = FS_ACOPY + 1;         // token-row copies + scale copy
static_assert(FS_TBM == 192, "scale copies: three waves of 64 rows");
static_assert(FS_TBM % 32 == 0 && (FS_TBM / 8) % FS_NWAVE == 0 && FS_BCOPY == 4, "tile configuration");
static_assert(FS_BBASE + FS_NWAVE * FS_NSB * FS_BWAVE <= 160 * 1024, "LDS per workgroup");
static_assert(FS_NSA == 3 && FS_NSB == 2, "the prologue and wait count below assume this ring");

}  // namespace

template <bool GATED>
__global__ __launch_bounds__(FS_NTHREAD, 1) void tile_gemm_fp8_kernel(TileArgs8 g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];

  // column tiles (N % 128 == 0; a down tile may be half past N)
  const int n_nt = GATED ? g.N / (FS_TBN / 2) : (g.N + FS_TBN - 1) / FS_TBN;
  const int n_tasks = g.mt_start[g.n_exp] * n_nt;
  const int task = blockIdx.x;
  if (task >= n_tasks) return;  // uniform per workgroup, before any barrier
  int lo = 0, hi = g.n_exp - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (g.mt_start[mid] * n_nt <= task) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int n_mt = g.mt_start[e + 1] - g.mt_start[e];
  const int local = task - g.mt_start[e] * n_nt;
  const int nt = local / n_mt;
  const int mtile = local - nt * n_mt;
  const bool shared = e >= g.E;
  const int cnt = shared ? g.T : g.counts[e];
  const int row_base = shared ? g.TK + (e - g.E) * g.T : g.offsets[e];
  const int m0 = mtile * FS_TBM;
  const int rows = min(FS_TBM, cnt - m0);
  const int K = g.K;
  const int KB = K / 128;                        // scale blocks along K
  const int NB = g.N / 128;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;

  // ---- token rows: buffer resources over the activation codes [T][K]
  // (gate/up) or this expert's own staged rows (down, at most T), and their
  // scales [rows][K/128]; the entry points bound T * K below 4 GiB
  const int a_rows = GATED ? g.T : cnt;
  const __amdgpu_buffer_rsrc_t ars =
      buffer_rsrc(GATED ? g.a : g.a + (size_t)row_base * K, uint32_t(a_rows) * uint32_t(K));
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(GATED ? g.as : g.as + (size_t)row_base * KB,
                                                 uint32_t(a_rows) * uint32_t(KB) * 4u);
  auto a_row = [&](int r) {  // activation row of tile row r (rows past the count re-read one)
    const int m = m0 + min(r, rows - 1);
    return GATED ? (shared ? m : g.perm[row_base + m]) : m;
  };
  // copy i of wave w fills tile rows 8 (FS_ACOPY w + i) .. +7; lane l writes
  // LDS bytes 16 l of that 1 KB: row r0 + l/8 at position l%8, which holds
  // logical chunk (l%8) ^ (row%8)
  uint32_t aoff[FS_ACOPY];
#pragma unroll
  for (int i = 0; i < FS_ACOPY; ++i) {
    const int r = 8 * (FS_ACOPY * wave + i) + (lane >> 3);
    aoff[i] = uint32_t(a_row(r)) * uint32_t(K) + uint32_t(((lane & 7) ^ (r & 7)) * 16);
  }
  // row scales: waves 0, 1, 2 copy rows 64 w + l; the other waves repeat
  // wave 2's copy (the same bytes to the same LDS slots)
  const int srow0 = 64 * min(wave, 2);
  const uint32_t soff = uint32_t(a_row(srow0 + lane)) * uint32_t(KB) * 4u;

  // ---- weight rows of this wave (32: local row q = 16 j + c16 is MFMA
  // column block j's row c16).  Gate/up: 16 columns of W_gate (rows 0-15)
  // and the same 16 of W_up (rows 16-31); down: 32 columns (rows past N
  // re-read row N-1 and are never stored).  Copy i covers local rows
  // 8 i .. 8 i + 7.
  const uint32_t wbytes = uint32_t(g.N) * uint32_t(K);
  const __amdgpu_buffer_rsrc_t wr0 = buffer_rsrc(g.w0 + (size_t)e * g.N * K, wbytes);
  const __amdgpu_buffer_rsrc_t wr1 = GATED ? buffer_rsrc(g.w1 + (size_t)e * g.N * K, wbytes) : wr0;
  uint32_t boff[FS_BCOPY];
#pragma unroll
  for (int i = 0; i < FS_BCOPY; ++i) {
    const int q = 8 * i + (lane >> 3);
    const int wrow = GATED ? nt * 128 + 16 * wave + (q & 15)
                           : min(nt * FS_TBN + 32 * wave + q, g.N - 1);
    boff[i] = uint32_t(wrow) * uint32_t(K) + uint32_t(((lane & 7) ^ (q & 7)) * 16);
  }

  // weight-block scales of this wave's columns: gate/up use block nt of
  // s_gate and s_up; down block (nt*256 + 32 w) / 128 of s_down.  Held in
  // registers (lane l: blocks l and 64 + l) and read with v_readlane.
  const float* __restrict__ sw0 =
      g.ws0 + (size_t)e * NB * KB +
      (size_t)(GATED ? nt : min((nt * FS_TBN + 32 * wave) / 128, NB - 1)) * KB;
  const float* __restrict__ sw1 = GATED ? g.ws1 + (size_t)e * NB * KB + (size_t)nt * KB : sw0;
  float swv0[2], swv1[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int kb = min(64 * c + lane, KB - 1);
    swv0[c] = sw0[kb];
    swv1[c] = sw1[kb];
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the counts below start from zero

  // loop indices past the end repeat the last block
  auto kblock = [&](int i) { return min(i, KB - 1); };

  uint8_t* bring = smem8 + FS_BBASE + wave * FS_NSB * FS_BWAVE;  // this wave's weight ring
  // token-row copies of block kb into shared stage kb % FS_NSA
  auto copy_a = [&](int kb) {
    const uint32_t kc = uint32_t(kblock(kb));
    uint8_t* st = smem8 + (kb % FS_NSA) * FS_STAGE;
#pragma unroll
    for (int i = 0; i < FS_ACOPY; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ars, (lds_void*)(st + 8 * (FS_ACOPY * wave + i) * 128), 16, aoff[i] + kc * 128u, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void*)(st + FS_ASTAGE + srow0 * 4), 4,
                                             soff + kc * 4u, 0, 0, 0);
  };
  // weight-row copies of block kb into private stage kb % FS_NSB.  An expert
  // with one row tile reads its weights once: those copies are non-temporal
  // (streamed past the caches; 2350 -> 2280 us for gate/up at 4096 tokens).
  // An expert with more row tiles keeps them cacheable for its other tiles.
  const bool once = n_mt == 1;
  auto copy_b = [&](int kb) {
    const uint32_t ko = uint32_t(kblock(kb)) * 128u;
    uint8_t* st = bring + (kb % FS_NSB) * FS_BWAVE;
    if (once) {
#pragma unroll
      for (int i = 0; i < FS_BCOPY; ++i) {
        const __amdgpu_buffer_rsrc_t rs = (GATED && i >= FS_BCOPY / 2) ? wr1 : wr0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + 1024 * i), 16, boff[i] + ko, 0, 0,
                                                 2 /* nt */);
      }
    } else {
#pragma unroll
      for (int i = 0; i < FS_BCOPY; ++i) {
        const __amdgpu_buffer_rsrc_t rs = (GATED && i >= FS_BCOPY / 2) ? wr1 : wr0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + 1024 * i), 16, boff[i] + ko, 0, 0, 0);
      }
    }
  };

  const int mact = __builtin_amdgcn_readfirstlane((rows + 31) >> 5);  // active 32-row pairs
  f32x4 acc[FS_RB][2];
#pragma unroll
  for (int i = 0; i < FS_RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // 32 bytes of operand row r of a staged block: chunks g4 and g4 + 4
  auto frag = [&](const uint8_t* base, int r) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + r * 128 + ((g4 ^ (r & 7)) << 4));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + r * 128 + (((g4 + 4) ^ (r & 7)) << 4));
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  auto compute = [&](int kb, const i32x8& b0, const i32x8& b1, auto mact_c) {
    constexpr int NRB = 2 * decltype(mact_c)::value;
    const uint8_t* st = smem8 + (kb % FS_NSA) * FS_STAGE;
    const float* sc = reinterpret_cast<const float*>(st + FS_ASTAGE);
    const int kr = kblock(kb);
    const float sb0 = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(kr < 64 ? swv0[0] : swv0[1]), kr & 63));
    const float sb1 = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(kr < 64 ? swv1[0] : swv1[1]), kr & 63));
    // token fragments and row scales are read three row blocks ahead of
    // their promotion, two ahead of their MFMAs; the MFMAs of row block i + 1
    // are issued before the promotion of block i, so the vector ALU works
    // while the matrix core does
    i32x8 af[NRB];
    float sa[NRB];
    auto rd = [&](int i) {
      af[i] = frag(st, 16 * i + c16);
      sa[i] = sc[16 * i + c16];
    };
    rd(0);
    if (NRB > 1) rd(1);
    if (NRB > 2) rd(2);
    const float sbb = GATED ? sb1 : sb0;
    f32x4 t0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b0, af[0], zero, 0, 0, 0, 127, 0, 127);
    f32x4 t1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1, af[0], zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      if (i + 3 < NRB) rd(i + 3);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 u0 = zero, u1 = zero;
      if (i + 1 < NRB) {
        u0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b0, af[i + 1], zero, 0, 0, 0, 127, 0, 127);
        u1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1, af[i + 1], zero, 0, 0, 0, 127, 0, 127);
      }
      const float s0 = sa[i] * sb0, s1 = GATED ? sa[i] * sbb : s0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[i][0][v] = fmaf(t0[v], s0, acc[i][0][v]);
        acc[i][1][v] = fmaf(t1[v], s1, acc[i][1][v]);
      }
      if (i + 1 < NRB) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, GATED ? 5 : 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      t0 = u0;
      t1 = u1;
    }
  };

  // Issue order (W = weight rows, A = token rows and scales):
  //   prologue W0 W1 A0 A1; block kb: A(kb+2) W(kb+2)
  // At the top of block kb >= 1 the copies issued after W(kb) are exactly
  // A(kb+1) and W(kb+1), and A(kb) was issued before W(kb): waiting until at
  // most FS_ACOPIES + FS_BCOPY copies are in flight completes both (before
  // block 0, at most FS_ACOPIES: only A1 follows A0).  The wave then reads
  // its weight fragments of kb into registers, which frees its weight stage
  // of kb for W(kb+2).
  // s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt/lgkmcnt at maxima.
  constexpr int VMW = FS_BCOPY + FS_ACOPIES;
  constexpr int WAITIMM = (VMW & 15) | ((VMW >> 4) << 14) | 0x70 | 0xf00;
  constexpr int VMW0 = FS_ACOPIES;
  constexpr int WAITIMM0 = (VMW0 & 15) | ((VMW0 >> 4) << 14) | 0x70 | 0xf00;
  auto mainloop = [&](auto mact_c) {
    copy_b(0);
    copy_b(1);
    copy_a(0);
    copy_a(1);
    __builtin_amdgcn_s_waitcnt(WAITIMM0);  // W0, W1, A0 landed
    for (int kb = 0; kb < KB; ++kb) {
      __builtin_amdgcn_s_waitcnt(WAITIMM);  // this wave's token and weight rows of kb landed
      __builtin_amdgcn_s_barrier();         // everyone's; everyone is done with kb-1
      const uint8_t* bst = bring + (kb % FS_NSB) * FS_BWAVE;
      const i32x8 b0 = frag(bst, c16), b1 = frag(bst, 16 + c16);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the weight stage of kb is free
      copy_a(kb + 2);                       // into the token stage of kb-1
      copy_b(kb + FS_NSB);                  // into this wave's weight stage of kb
      compute(kb, b0, b1, mact_c);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  };
  switch (mact) {
    case 6: mainloop(std::integral_constant<int, 6>{}); break;
    case 5: mainloop(std::integral_constant<int, 5>{}); break;
    case 4: mainloop(std::integral_constant<int, 4>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    default: mainloop(std::integral_constant<int, 1>{}); break;
  }

  // ---- epilogue.  16x16 accumulator v of lane l (weights as the MFMA's
  // first operand): column 4*(l/16) + v of the block, token row l%16
  if (GATED) {
    // H = SiLU(gate) * up for the tile's 128 columns (one 1x128 slice per row)
    float* red = reinterpret_cast<float*>(smem8);  // [NWAVE][TBM] row max-abs per wave
    __syncthreads();  // every wave is done with the staged operands
    f32x4 h[FS_RB];
#pragma unroll
    for (int i = 0; i < FS_RB; ++i) {
      if (2 * mact <= i) continue;  // uniform
      float m = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        h[i][v] = siluf(acc[i][0][v]) * acc[i][1][v];
        m = fmaxf(m, fabsf(h[i][v]));
      }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (g4 == 0) red[wave * FS_TBM + 16 * i + c16] = m;
    }
    __syncthreads();
    const int col = nt * 128 + 16 * wave + 4 * g4;
#pragma unroll
    for (int i = 0; i < FS_RB; ++i) {
      if (2 * mact <= i) continue;
      const int r = 16 * i + c16;
      float amax = 0.f;
#pragma unroll
      for (int w = 0; w < FS_NWAVE; ++w) amax = fmaxf(amax, red[w * FS_TBM + r]);
      const float scale = e4m3_scale(amax);
      uint32_t codes = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) codes |= e4m3_encode(h[i][v] / scale) << (8 * v);
      if (r < rows) {
        const size_t orow = (size_t)(row_base + m0 + r);
        *reinterpret_cast<uint32_t*>(g.out8 + orow * g.N + col) = codes;
        if (wave == 0 && g4 == 0) g.out_s[orow * NB + nt] = scale;
      }
    }
  } else {
    // through a slot of each wave's own in LDS, 16 rows at a time: one 16-byte
    // store per lane writes 16 rows x the wave's 64 bytes (2-byte stores from
    // the accumulators write 32-byte pieces)
    constexpr int PITCH = 64 + 16;  // staging row bytes
    typedef __attribute__((address_space(3))) uint8_t lds8;
    __syncthreads();  // every wave is done with the staged operands
    lds8* stg = (lds8*)smem8 + wave * 16 * PITCH;
    const int col0 = nt * FS_TBN + 32 * wave;
    const bool cols_ok = col0 < g.N;  // a down tile may be half past N
#pragma unroll
    for (int i = 0; i < FS_RB; ++i) {
      if (2 * mact <= i) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t p0 = uint32_t(f32_to_bf16(acc[i][j][0])) | (uint32_t(f32_to_bf16(acc[i][j][1])) << 16);
        const uint32_t p1 = uint32_t(f32_to_bf16(acc[i][j][2])) | (uint32_t(f32_to_bf16(acc[i][j][3])) << 16);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *(__attribute__((address_space(3))) u32x2*)(stg + c16 * PITCH + 2 * (16 * j + 4 * g4)) = u32x2{p0, p1};
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int rr = lane >> 2, cb = 16 * (lane & 3);
      const u32x4 val = *(__attribute__((address_space(3))) const u32x4*)(stg + rr * PITCH + cb);
      const int r = 16 * i + rr;
      if (cols_ok && r < rows)
        *reinterpret_cast<u32x4*>(g.out16 + (size_t)(row_base + m0 + r) * g.N + col0 + cb / 2) = val;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

size_t tile_gemm_fp8_lds_bytes() { return size_t(FS_BBASE) + size_t(FS_NWAVE) * FS_NSB * FS_BWAVE; }

template <bool GATED>
static hipError_t launch_fp8_one(const TileArgs8& g, int max_mtiles, hipStream_t st) {
  const int n_nt = GATED ? g.N / (FS_TBN / 2) : (g.N + FS_TBN - 1) / FS_TBN;
  const long long blocks = (long long)max_mtiles * n_nt;
  if (blocks <= 0) return hipSuccess;
  const size_t lds = tile_gemm_fp8_lds_bytes();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&tile_gemm_fp8_kernel<GATED>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL((tile_gemm_fp8_kernel<GATED>), dim3((unsigned)blocks), dim3(FS_NTHREAD), lds,
                     st, g);
  return hipGetLastError();
}

hipError_t launch_tile_gemm_fp8(const TileArgs8& g, bool gated, int max_mtiles, hipStream_t st) {
  return gated ? launch_fp8_one<true>(g, max_mtiles, st) : launch_fp8_one<false>(g, max_mtiles, st);
}

}  // namespace moe
