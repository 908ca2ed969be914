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
// Quantiser: scale = amax / 448 in float32 (1 for an all-zero slice), code =
// round-to-nearest-even of the float32 quotient v / scale (IEEE division),
// saturated to +-448.  The encoder is integer arithmetic on the float32 bits,
// so the codes do not depend on a hardware conversion mode.
//
// GEMM tile: F8_TBM (192) token rows x 256 weight rows, one 128-wide K block
// per LDS stage (128 bytes per row, eight 16-byte chunks stored at
// chunk ^ (row % 8)), two stages (116 KB) filled by direct global->LDS copies
// one block ahead.  192 rows hold nearly every expert of a 4096-token batch
// in one row tile, so its weights stream once (128-row tiles with three
// stages measured 25% slower: second row tiles re-read the weights).  Eight
// waves in 2 (rows) x 4 (columns).  Per K block and 32x32 output block: two
// v_mfma_scale_f32_32x32x64_f8f6f4 (hardware block scales left at 1) into a
// temporary, then acc += tmp * (row scale * weight-block scale).  The row
// scales of the block ride along with the A copies into LDS; a wave's
// weight-block scales (one per K block) are loaded into registers before the
// pipeline starts.
// Gate/up tiles hold 128 columns of W_gate and the same 128 of W_up, which is
// exactly one 1x128 slice of the SwiGLU output H: the epilogue forms
// SiLU(gate) * up, reduces each row's max-abs across the four column waves
// through LDS, and writes H as E4M3 codes plus one scale per row.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int F8_MBW = MOE_F8_MBW;          // 32-row MFMA blocks per wave
constexpr int F8_TBM = 64 * F8_MBW;         // token rows per tile (2 waves along M)
constexpr int F8_TBN = 256;                 // weight rows per tile
constexpr int F8_TBK = 128;                 // K per stage (bytes per row) = one scale block
#ifndef MOE_F8_NSTAGE
#define MOE_F8_NSTAGE 2
#endif
constexpr int F8_NSTAGE = MOE_F8_NSTAGE;
constexpr int F8_WN = 4;                    // waves along N
constexpr int F8_NWAVE = 2 * F8_WN, F8_NTHREAD = 64 * F8_NWAVE;
constexpr int F8_RPW = F8_TBM / F8_NWAVE;   // rows whose A scale one wave copies
constexpr int F8_ASTAGE = F8_TBM * F8_TBK;  // bytes
constexpr int F8_BSTAGE = F8_TBN * F8_TBK;
constexpr int F8_SSTAGE = F8_NWAVE * 64 * 4;  // one 4-byte copy per lane per wave
constexpr int F8_STAGE = F8_ASTAGE + F8_BSTAGE + F8_SSTAGE;
static_assert(F8_TBM == kTileM8, "row tile shared with the tile prefix scan");
static_assert(F8_RPW % 4 == 0 && F8_RPW <= 64, "scale copy layout");
static_assert(F8_NSTAGE * F8_STAGE <= 160 * 1024, "LDS per workgroup");

typedef __attribute__((address_space(3))) void lds_void;

MOE_DEV int swz8(int row, int chunk) { return chunk ^ (row & 7); }

// LDS float slot of row r's A scale within a stage's scale area
MOE_DEV int scale_slot(int r) { return (r / F8_RPW) * 64 + (r % F8_RPW); }

// 32 bytes (logical chunks c, c+1) of a staged row
MOE_DEV i32x8 ld_frag8(const uint8_t* base, int row, int c) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + row * F8_TBK + (swz8(row, c) << 4));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + row * F8_TBK + (swz8(row, c + 1) << 4));
  return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// OCP E4M3FN code of a float32 value, round to nearest even, |v| clamped to 448
MOE_DEV uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  if (a < 0.015625f) {  // below the smallest normal 2^-6: steps of 2^-9
    return sign | uint32_t(rintf(a * 512.0f));  // 8 lands on the smallest normal's code
  }
  uint32_t u = __float_as_uint(a);
  u += 0x7ffffu + ((u >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
  return sign | ((u >> 20) - (120u << 3));  // rebias the exponent 127 -> 7
}

MOE_DEV float max4(float a, float b, float c, float d) { return fmaxf(fmaxf(a, b), fmaxf(c, d)); }

}  // namespace

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
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
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

// ---------------------------------------------------------------- fp8 tiled GEMM
template <bool GATED>
__global__ __launch_bounds__(F8_NTHREAD, 1) void tile_gemm_fp8_kernel(TileArgs8 g) {
  constexpr int AGRP = F8_TBM / 8;               // 1 KB copies (8 rows) of A per stage
  constexpr int ACPW = AGRP / F8_NWAVE;
  constexpr int BCPW = F8_TBN / 8 / F8_NWAVE;
  constexpr int NJ = F8_TBN / F8_WN / 32;        // 32-column MFMA blocks per wave
  static_assert(AGRP % F8_NWAVE == 0 && BCPW >= 1 && NJ == 2, "tile configuration");
  constexpr int CPS = ACPW + BCPW + 1;           // copies per wave per stage (+1: scales)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];

  // column tiles (N % 128 == 0; a down tile may be half past N)
  const int n_nt = GATED ? g.N / (F8_TBN / 2) : (g.N + F8_TBN - 1) / F8_TBN;
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
  const int m0 = mtile * F8_TBM;
  const int rows = min(F8_TBM, cnt - m0);
  const int K = g.K;
  const int KB = K / 128;                        // scale blocks along K = stages
  const int NB = g.N / 128;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / F8_WN, wn = wave % F8_WN;

  // ---- copy sources (byte offsets from uniform bases; A offsets < T * K)
  const uint8_t* __restrict__ abase = GATED ? g.a : g.a + (size_t)row_base * K;
  const float* __restrict__ sabase = GATED ? g.as : g.as + (size_t)row_base * KB;
  const uint8_t* __restrict__ wb0 = g.w0 + (size_t)e * g.N * K;
  const uint8_t* __restrict__ wb1 = GATED ? g.w1 + (size_t)e * g.N * K : wb0;
  auto a_row = [&](int r) {  // activation row of tile row r (rows past the count re-read one)
    const int m = m0 + min(r, rows - 1);
    return GATED ? (shared ? m : g.perm[row_base + m]) : m;
  };
  uint32_t aoff[ACPW], boff[BCPW];
#pragma unroll
  for (int i = 0; i < ACPW; ++i) {
    const int r = 8 * (wave + F8_NWAVE * i) + (lane >> 3);
    aoff[i] = uint32_t(a_row(r)) * uint32_t(K) + uint32_t(swz8(r, lane & 7) * 16);
  }
#pragma unroll
  for (int i = 0; i < BCPW; ++i) {
    const int r = 8 * (wave * BCPW + i) + (lane >> 3);
    // weight rows past N (a partial down tile) re-read row N-1; never stored
    const int col =
        GATED ? nt * (F8_TBN / 2) + (r & (F8_TBN / 2 - 1)) : min(nt * F8_TBN + r, g.N - 1);
    boff[i] = uint32_t(col) * uint32_t(K) + uint32_t(swz8(r, lane & 7) * 16);
  }
  const uint8_t* __restrict__ wsrc = (GATED && wave >= F8_NWAVE / 2) ? wb1 : wb0;
  // lane l copies the scale of row wave*RPW + l % RPW (lanes past RPW repeat)
  const uint32_t soff = uint32_t(a_row(wave * F8_RPW + lane % F8_RPW)) * uint32_t(KB) * 4u;

  // weight-block scales of this wave's columns: gate/up tiles use block nt of
  // s_gate and s_up; down tiles block (nt*256 + wn*64) / 128 of s_down
  const float* __restrict__ sw0 = g.ws0 + (size_t)e * NB * KB +
                                  (size_t)(GATED ? nt : min((nt * F8_TBN + wn * 64) / 128, NB - 1)) * KB;
  const float* __restrict__ sw1 = GATED ? g.ws1 + (size_t)e * NB * KB + (size_t)nt * KB : sw0;

  // Held in registers before the pipeline starts (lane l: blocks l and 64 + l)
  // and read with v_readlane: no vector load may be outstanding inside the
  // pipeline, whose waits count only the LDS copies.
  float swv0[2], swv1[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int kb = min(64 * c + lane, KB - 1);
    swv0[c] = sw0[kb];
    swv1[c] = sw1[kb];
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  const int mrows = rows - wm * 32 * F8_MBW;
  const int mact =
      __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : min(F8_MBW, (mrows + 31) >> 5));

  f32x16 acc[F8_MBW][NJ];
#pragma unroll
  for (int i = 0; i < F8_MBW; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  int brow0[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    brow0[j] = GATED ? ((j < NJ / 2) ? (wn * (F8_TBN / 2 / F8_WN) + 32 * j)
                                     : (F8_TBN / 2 + wn * (F8_TBN / 2 / F8_WN) + 32 * (j - NJ / 2)))
                     : (wn * (F8_TBN / F8_WN) + 32 * j);
  const int arow0 = wm * 32 * F8_MBW + (lane & 31);

  auto copy_step = [&](int kt) {
    const int kc = min(kt, KB - 1);
    const uint32_t koff = uint32_t(kc * F8_TBK);
    uint8_t* st = smem8 + (kt % F8_NSTAGE) * F8_STAGE;
    uint8_t* a = st + (8 * wave) * F8_TBK;
    uint8_t* b = st + F8_ASTAGE + (8 * BCPW * wave) * F8_TBK;
    uint8_t* s = st + F8_ASTAGE + F8_BSTAGE + wave * 256;
#pragma unroll
    for (int i = 0; i < ACPW; ++i)
      __builtin_amdgcn_global_load_lds(abase + (aoff[i] + koff),
                                       (lds_void*)(a + 8 * F8_NWAVE * i * F8_TBK), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < BCPW; ++i)
      __builtin_amdgcn_global_load_lds(wsrc + (boff[i] + koff), (lds_void*)(b + 8 * i * F8_TBK), 16,
                                       0, 0);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(sabase) + (soff + kc * 4u),
                                     (lds_void*)s, 4, 0, 0);
  };

  const f32x16 zero = {};
  auto compute = [&](int kt, auto mact_c) {
    constexpr int MACT = decltype(mact_c)::value;
    const uint8_t* st = smem8 + (kt % F8_NSTAGE) * F8_STAGE;
    const uint8_t* a = st;
    const uint8_t* b = st + F8_ASTAGE;
    const float* sc = reinterpret_cast<const float*>(st + F8_ASTAGE + F8_BSTAGE);
    const float sb0 = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(kt < 64 ? swv0[0] : swv0[1]), kt & 63));
    const float sb1 = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(kt < 64 ? swv1[0] : swv1[1]), kt & 63));
    i32x8 bf[2][NJ];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[h][j] = ld_frag8(b, brow0[j] + (lane & 31), 4 * h + 2 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < MACT; ++i) {
      const i32x8 a0 = ld_frag8(a, arow0 + 32 * i, 2 * (lane >> 5));
      const i32x8 a1 = ld_frag8(a, arow0 + 32 * i, 4 + 2 * (lane >> 5));
      f32x4 sa[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sa[q] = *reinterpret_cast<const f32x4*>(
            sc + scale_slot(wm * 32 * F8_MBW + 32 * i + 8 * q + 4 * (lane >> 5)));
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        f32x16 t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bf[0][j], zero, 0, 0, 0,
                                                                   127, 0, 127);
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bf[1][j], t, 0, 0, 0, 127, 0, 127);
        const float sbj = (GATED && j >= NJ / 2) ? sb1 : sb0;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(t[v], sa[v >> 2][v & 3] * sbj, acc[i][j][v]);
      }
    }
  };

  // pipeline as in the bf16 tiled GEMM: copies run NSTAGE-1 blocks ahead;
  // s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt/lgkmcnt at maxima
  constexpr int VMWAIT = (F8_NSTAGE - 2) * CPS;
  static_assert(VMWAIT < 64, "vmcnt field is 6 bits");
  constexpr int WAITIMM = (VMWAIT & 15) | ((VMWAIT >> 4) << 14) | 0x70 | 0xf00;
  auto mainloop = [&](auto mact_c) {
#pragma unroll
    for (int p = 0; p < F8_NSTAGE - 1; ++p) copy_step(p);
    for (int kt = 0; kt < KB; ++kt) {
      __builtin_amdgcn_s_waitcnt(WAITIMM);
      __builtin_amdgcn_s_barrier();
      copy_step(kt + F8_NSTAGE - 1);
      compute(kt, mact_c);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  };
  static_assert(F8_MBW <= 4, "dispatch below covers up to 4 blocks");
  switch (mact) {
    case 4: mainloop(std::integral_constant<int, (F8_MBW >= 4 ? 4 : 0)>{}); break;
    case 3: mainloop(std::integral_constant<int, (F8_MBW >= 3 ? 3 : 0)>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    default: mainloop(std::integral_constant<int, 0>{}); break;
  }

  // ---- epilogue.  32x32 accumulator v of lane l: row 8*(v/4) + 4*(l/32) + v%4,
  // column l%32
  if (GATED) {
    // H = SiLU(gate) * up for the tile's 128 columns (one 1x128 slice per row)
    float* red = reinterpret_cast<float*>(smem8);  // [WN][TBM] row max-abs per column wave
    __syncthreads();  // every wave is done with the staged operands
    float h[F8_MBW][16];
#pragma unroll
    for (int i = 0; i < F8_MBW; ++i) {
      if (i >= mact) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        h[i][v] = siluf(acc[i][0][v]) * acc[i][1][v];
        float m = fabsf(h[i][v]);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        const int r = wm * 32 * F8_MBW + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if ((lane & 31) == 0) red[wn * F8_TBM + r] = m;
      }
    }
    __syncthreads();
    const int col = nt * 128 + wn * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < F8_MBW; ++i) {
      if (i >= mact) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 32 * F8_MBW + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const float amax = max4(red[r], red[F8_TBM + r], red[2 * F8_TBM + r], red[3 * F8_TBM + r]);
        const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
        if (r < rows) {
          const size_t orow = (size_t)(row_base + m0 + r);
          g.out8[orow * g.N + col] = uint8_t(e4m3_encode(h[i][v] / scale));
          if (wn == 0 && (lane & 31) == 0) g.out_s[orow * NB + nt] = scale;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < F8_MBW; ++i) {
      if (i >= mact) break;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = nt * F8_TBN + wn * (F8_TBN / F8_WN) + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 32 * F8_MBW + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (r < rows && col < g.N)
            g.out16[(size_t)(row_base + m0 + r) * g.N + col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
}

size_t tile_gemm_fp8_lds_bytes() { return size_t(F8_NSTAGE) * F8_STAGE; }

template <bool GATED>
static hipError_t launch_fp8_one(const TileArgs8& g, int max_mtiles, hipStream_t st) {
  const int n_nt = GATED ? g.N / (F8_TBN / 2) : (g.N + F8_TBN - 1) / F8_TBN;
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
  hipLaunchKernelGGL((tile_gemm_fp8_kernel<GATED>), dim3((unsigned)blocks), dim3(F8_NTHREAD), lds,
                     st, g);
  return hipGetLastError();
}

hipError_t launch_tile_gemm_fp8(const TileArgs8& g, bool gated, int max_mtiles, hipStream_t st) {
  return gated ? launch_fp8_one<true>(g, max_mtiles, st) : launch_fp8_one<false>(g, max_mtiles, st);
}

}  // namespace moe
