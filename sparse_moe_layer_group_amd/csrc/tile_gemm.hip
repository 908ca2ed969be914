// LDS-tiled grouped expert GEMM for experts with many rows (prefill-sized batches).
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §1.1 (SwiGLU
// experts) and §1.3 Eq 12.
//
// Workgroup tile: 256 rows x 256 weight rows, K in steps of 64.  Gate/up
// tiles hold 128 columns: weight rows 0..127 come from W_gate and 128..255
// from W_up for the same columns, so SiLU(gate) * up is formed in registers.
// Down tiles hold 256 columns of W_down.  Eight waves in 2 (rows) x 4
// (columns), each owning a 128 x 64 sub-tile as 4 x 2 v_mfma_f32_32x32x16_bf16
// blocks (128 fp32 accumulators per lane), two waves per SIMD so one
// multiplies while the other waits.  32-row blocks past the expert's row count
// are skipped per wave.
//
// LDS: four stages of A[256][32] and B[256][32] bf16 (32 KB each).  A row is
// four 16-byte chunks; chunk c of row r is stored at position c ^ ((r/2) & 3),
// so the eight rows read together by a fragment load hit distinct banks.
// Global memory is copied straight into LDS (global_load_lds, 1 KB per wave
// instruction, no registers), three K steps ahead of the step being
// multiplied.  Each step waits for its own copies with an explicit vmcnt
// (the copies of the next two steps stay in flight), meets the workgroup at
// one barrier, refills the stage freed by the previous step and multiplies.
// Copies past the last step re-read the last step so that every step issues
// the same number of copies.
//
// Task order: for each expert and column tile, its row tiles are consecutive
// workgroups, so the workgroups sharing a weight tile run together and read it
// from HBM once (L2 / MALL serve the others).  Dealing each XCD a contiguous
// eighth of the tasks (MOE_TILE_XCD=1) keeps an expert's token rows in one L2
// and cuts L2 misses, but measured 6% slower at 8192 tokens.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Tile configuration: TBN weight rows per workgroup tile (128: two workgroups
// per CU; 256: one), NSTAGE LDS stages (copies run NSTAGE-1 steps ahead).
#ifndef MOE_TILE_TBN
#define MOE_TILE_TBN 256
#endif
#ifndef MOE_TILE_NSTAGE
#define MOE_TILE_NSTAGE 4
#endif
#ifndef MOE_TILE_WN
#define MOE_TILE_WN 4
#endif
#ifndef MOE_TILE_XCD
#define MOE_TILE_XCD 0
#endif
constexpr int MBW = MOE_TILE_MBW;           // 32-row MFMA blocks per wave (2 waves along M)
constexpr int TBM = 64 * MBW, TBK = 32;
constexpr int TBN = MOE_TILE_TBN, NSTAGE = MOE_TILE_NSTAGE;
constexpr int WN = MOE_TILE_WN;            // waves along N (2 along M)
constexpr int NWAVE = 2 * WN, NTHREAD = 64 * NWAVE;
constexpr int WGS_PER_CU = (TBN == 128 && WN == 2) ? 2 : 1;
constexpr int ASTAGE = TBM * TBK;  // bf16 elements of A per stage
static_assert(TBM == kTileM, "row tile shared with the tile prefix scan");

typedef __attribute__((address_space(3))) void lds_void;

MOE_DEV int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

MOE_DEV bf16x8 ld_frag(const bf16_t* base, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(base + row * TBK + (swz(row, chunk) << 3));
}

}  // namespace

// Wave tile 128 x TBN/WN.  (The tile configuration is a set of namespace
// constants rather than template parameters: with more than one template
// parameter this compiler does not emit the host-side launch stubs.)
template <bool GATED>
__global__ __launch_bounds__(NTHREAD, WGS_PER_CU) void tile_gemm_kernel(TileArgs g) {
  constexpr int BSTAGE = TBN * TBK;              // bf16 elements of B per stage
  constexpr int AGRP = TBM / 16;                 // 16-row groups of A per stage
  constexpr int ACPW = (AGRP + NWAVE - 1) / NWAVE;  // 1 KB copies of A per wave (at most)
  constexpr int ACPW_MIN = AGRP / NWAVE;         // ... at least
  constexpr int BCPW = TBN / 16 / NWAVE;         // 1 KB copies of B per wave per step
  constexpr int NJ = TBN / WN / 32;              // 32-column MFMA blocks per wave
  static_assert(ACPW_MIN >= 1 && BCPW >= 1 && NJ >= 2 && NJ % 2 == 0, "tile configuration");
  constexpr int CPS = ACPW_MIN + BCPW;           // copies per wave per step (smallest)
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* As = smem;                             // [NSTAGE][TBM][32]
  bf16_t* Bs = smem + NSTAGE * ASTAGE;           // [NSTAGE][TBN][32]

  // column tiles (N % 128 == 0; a down tile may be half past N)
  const int n_nt = GATED ? g.N / (TBN / 2) : (g.N + TBN - 1) / TBN;
  const int n_tasks = g.mt_start[g.n_exp] * n_nt;
#if MOE_TILE_XCD
  // Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
  // b % 8).  XCD x takes the x-th contiguous eighth of the actual task list,
  // so the column tiles of one expert run on one XCD and its token rows are
  // fetched into one L2.
  const int per = (n_tasks + 7) >> 3;
  const int j = blockIdx.x >> 3;
  const int task = (blockIdx.x & 7) * per + j;
  if (j >= per || task >= n_tasks) return;  // uniform per workgroup, before any barrier
#else
  const int task = blockIdx.x;
  if (task >= n_tasks) return;  // uniform per workgroup, before any barrier
#endif
  // task -> expert, then (column tile, row tile) with row tiles fastest
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
  const int m0 = mtile * TBM;
  const int rows = min(TBM, cnt - m0);
  const int K = g.K;
  const int nk = K / TBK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- copy sources.  Copy i of wave w fills 16 rows of a stage (A row group
  // w + NWAVE i, B rows 16(w*BCPW + i)..); lane l writes LDS bytes 16 l of that
  // 1 KB, i.e. row r0 + l/4 at swizzled position l%4, which holds logical chunk
  // swz(row, l%4).  32-bit byte offsets from uniform base pointers.
  // (A offsets stay below T * K * 2 bytes: x rows are token ids < T; staged
  // rows are addressed from the expert's first row)
  uint32_t aoff[ACPW], boff[BCPW];
  const char* __restrict__ abase =
      reinterpret_cast<const char*>(GATED ? g.a : g.a + (size_t)row_base * K);
  const char* __restrict__ wb0 = reinterpret_cast<const char*>(g.w0 + (size_t)e * g.N * K);
  const char* __restrict__ wb1 =
      GATED ? reinterpret_cast<const char*>(g.w1 + (size_t)e * g.N * K) : wb0;
#pragma unroll
  for (int i = 0; i < ACPW; ++i) {
    const int r = 16 * min(wave + NWAVE * i, AGRP - 1) + (lane >> 2);
    const int chunk = swz(r, lane & 3);
    const int m = m0 + min(r, rows - 1);  // rows past the count re-read a valid row
    int arow;
    if (GATED) arow = shared ? m : g.perm[row_base + m];
    else arow = m;
    aoff[i] = (uint32_t(arow) * uint32_t(K) + uint32_t(chunk * 8)) * 2u;
  }
#pragma unroll
  for (int i = 0; i < BCPW; ++i) {
    const int r = 16 * (wave * BCPW + i) + (lane >> 2);
    const int chunk = swz(r, lane & 3);
    // weight rows past N (a partial down tile) re-read row N-1; never stored
    const int col = GATED ? nt * (TBN / 2) + (r & (TBN / 2 - 1)) : min(nt * TBN + r, g.N - 1);
    boff[i] = (uint32_t(col) * uint32_t(K) + uint32_t(chunk * 8)) * 2u;
  }
  // gate rows (0..TBN/2-1) are copied by the first half of the waves, up rows
  // by the second half
  const char* __restrict__ wsrc = (GATED && wave >= NWAVE / 2) ? wb1 : wb0;

  // ---- wave sub-tile: active 32-row blocks (uniform per wave)
  const int mrows = rows - wm * 32 * MBW;
  const int mact = __builtin_amdgcn_readfirstlane(mrows <= 0 ? 0 : min(MBW, (mrows + 31) >> 5));

  f32x16 acc[MBW][NJ];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // B sub-tile rows of this wave in the staged tile: gated waves take the same
  // columns of gate (first half of their blocks) and up (second half)
  int brow0[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    brow0[j] = GATED ? ((j < NJ / 2) ? (wn * (TBN / 2 / WN) + 32 * j)
                                     : (TBN / 2 + wn * (TBN / 2 / WN) + 32 * (j - NJ / 2)))
                     : (wn * (TBN / WN) + 32 * j);
  const int arow0 = wm * 32 * MBW + (lane & 31);

  // copies of K step kt into LDS stage kt % NSTAGE (steps past the end re-read
  // the last step)
  auto copy_step = [&](int kt) {
    const uint32_t koff = uint32_t(min(kt, nk - 1) * TBK * 2);
    const int stage = kt % NSTAGE;
    bf16_t* a = As + stage * ASTAGE + (16 * wave) * TBK;
    bf16_t* b = Bs + stage * BSTAGE + (16 * BCPW * wave) * TBK;
#pragma unroll
    for (int i = 0; i < ACPW; ++i)
      if (i < ACPW_MIN || wave + NWAVE * i < AGRP)  // uniform per wave
        __builtin_amdgcn_global_load_lds(abase + (aoff[i] + koff),
                                         (lds_void*)(a + 16 * NWAVE * i * TBK), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < BCPW; ++i)
      __builtin_amdgcn_global_load_lds(wsrc + (boff[i] + koff), (lds_void*)(b + 16 * i * TBK), 16,
                                       0, 0);
  };
  // MACT active 32-row blocks: fragments of k16 slice s+1 are read while the
  // MFMAs of slice s run; straight-line code for each MACT
  auto compute = [&](int stage, auto mact_c) {
    constexpr int MACT = decltype(mact_c)::value;
    const bf16_t* a = As + stage * ASTAGE;
    const bf16_t* b = Bs + stage * BSTAGE;
    bf16x8 af[2][MBW], bf[2][NJ];
    auto rd = [&](int s, bf16x8 (&afr)[MBW], bf16x8 (&bfr)[NJ]) {
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[j] = ld_frag(b, brow0[j] + (lane & 31), ch);
#pragma unroll
      for (int i = 0; i < MACT; ++i) afr[i] = ld_frag(a, arow0 + 32 * i, ch);
    };
    rd(0, af[0], bf[0]);
#pragma unroll
    for (int s = 0; s < TBK / 16; ++s) {
      if (s + 1 < TBK / 16) rd(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < MACT; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bf[s & 1][j],
                                                             acc[i][j], 0, 0, 0);
    }
  };

  // ---- pipeline: copies run NSTAGE-1 steps ahead.  At step kt a wave waits
  // until its copies of step kt have landed (2 * CPW copies per step; the
  // copies of steps kt+1 .. kt+NSTAGE-2 stay in flight), the workgroup meets
  // (every wave's copies of step kt are in LDS, and every wave has finished
  // multiplying step kt-1), the stage of step kt-1 is refilled with step
  // kt+NSTAGE-1, and step kt is multiplied.
  // s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
  // 6:4 and lgkmcnt 11:8 left at their maxima (no wait)
  constexpr int VMWAIT = (NSTAGE - 2) * CPS;
  static_assert(VMWAIT < 64, "vmcnt field is 6 bits");
  constexpr int WAITIMM = (VMWAIT & 15) | ((VMWAIT >> 4) << 14) | 0x70 | 0xf00;
  auto mainloop = [&](auto mact_c) {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p) copy_step(p);
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(WAITIMM);  // this wave's copies of step kt are done
      __builtin_amdgcn_s_barrier();
      copy_step(kt + NSTAGE - 1);
      compute(kt % NSTAGE, mact_c);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): no copy left in flight
  };
  static_assert(MBW <= 5, "dispatch below covers up to 5 blocks");
  switch (mact) {
    case 5: mainloop(std::integral_constant<int, (MBW >= 5 ? 5 : 0)>{}); break;
    case 4: mainloop(std::integral_constant<int, 4>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    default: mainloop(std::integral_constant<int, 0>{}); break;
  }

  // ---- epilogue.  32x32 accumulator v of lane l: row 8*(v/4) + 4*(l/32) + v%4,
  // column l%32
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    if (i >= mact) break;
#pragma unroll
    for (int j = 0; j < (GATED ? NJ / 2 : NJ); ++j) {
      const int col = GATED ? (nt * (TBN / 2) + wn * (TBN / 2 / WN) + 32 * j + (lane & 31))
                            : (nt * TBN + wn * (TBN / WN) + 32 * j + (lane & 31));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 32 * MBW + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r < rows && col < g.N) {
          const float val = GATED ? siluf(acc[i][j][v]) * acc[i][j + NJ / 2][v] : acc[i][j][v];
          g.out[(size_t)(row_base + m0 + r) * g.N + col] = f32_to_bf16(val);
        }
      }
    }
  }
}

size_t tile_gemm_lds_bytes() { return size_t(NSTAGE) * (TBM + TBN) * TBK * sizeof(bf16_t); }

template <bool GATED>
static hipError_t launch_one(const TileArgs& g, int max_mtiles, hipStream_t st) {
  const int n_nt = GATED ? g.N / (TBN / 2) : (g.N + TBN - 1) / TBN;
  // one workgroup per task, up to the largest task count the routing can
  // produce (workgroups past the actual count exit at once)
  long long blocks = (long long)max_mtiles * n_nt;
  if (blocks <= 0) return hipSuccess;
  blocks = (blocks + 7) / 8 * 8;  // every XCD gets ceil(tasks / 8) slots
  const size_t lds = tile_gemm_lds_bytes();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&tile_gemm_kernel<GATED>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL((tile_gemm_kernel<GATED>), dim3((unsigned)blocks), dim3(NTHREAD), lds, st, g);
  return hipGetLastError();
}

hipError_t launch_tile_gemm(const TileArgs& g, bool gated, int max_mtiles, hipStream_t st) {
  return gated ? launch_one<true>(g, max_mtiles, st) : launch_one<false>(g, max_mtiles, st);
}

}  // namespace moe
