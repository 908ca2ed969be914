// Weight-streaming grouped GEMM for experts with few rows (decode-sized batches).
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §1.1 (SwiGLU
// experts) and §5.1 (a decode expert sees few tokens, so its cost is reading
// its weights from memory, not arithmetic).
//
// Work unit = one wave: (expert, column slice, chunk of up to 64 rows).  The
// wave streams the 128 weight rows of its slice over the whole K range, one
// 64-wide K step (16 KB, 128 contiguous bytes of each row) at a time, and
// multiplies them with the chunk's token rows, one to four 16-row tiles, so
// each weight fragment feeds up to four MFMAs.  (With 16-row chunks the shared
// expert's 256 decode rows made 16 tasks per slice that each streamed the
// slice again; at 256 tokens, timing with the shared expert cut to one chunk
// showed those 15 extra passes cost 98 us of gate/up and 39 us of down.)
//
// Copies.  Each K step goes into one of two LDS stages of the wave's own by
// buffer_load ... lds, 1 KB (8 whole 128-byte rows) per copy: the weight rows
// non-temporal (read once), the token rows cacheable (every slice reads them).
// The copies of step s + 1 are issued before step s is multiplied, so two
// steps stream per wave.  On this part a streaming read moves 7.0-7.1 TB/s
// as non-temporal LDS copies of whole 128-byte lines but about 6.1 TB/s
// cacheable or as loads into registers; the first form of this kernel loaded
// the weights straight into MFMA operand registers (64 bytes of a row per
// load instruction, which the non-temporal hint makes slower still) and took,
// at 256 tokens in A/B runs on one box, gate/up 2515 / down 1304 us against
// 2246 / 1191 us now.  Chunk c (16 bytes) of staged row r sits at position
// c ^ (r % 8), so the 16 rows an MFMA operand reads spread over the banks.
//
// Balanced persistent grid: all tasks cost the same, so with n tasks and S
// wave slots the kernel runs k = ceil(n/S) rounds on W = ceil(n/k) waves
// (wave w takes tasks w, w+W, ...), and every active wave finishes within one
// task of the others.  Dealing n tasks over all S slots instead would leave a
// partial last round whose duration is that of a full one.  Two waves per
// workgroup, one workgroup per CU.
//
// K order inside a 64-wide step: lane l feeds its row's 16-byte chunk
// 2 (l/16) + q to the q-th of two 16x16x32 MFMAs.  A and B use the same map,
// so every product pairs equal k.  Steps start at a task-dependent rotation of
// K so that concurrent waves do not all read the same column offset of their
// rows.
//
// A chunk's tile t holds rows 16 t .. 16 t + 15 of the chunk; only its active
// tiles (rows present) are copied and multiplied, the count being uniform per
// task.
//
// Column map: gated slices hold 64 output columns; weight row of tile j
// (j = 0..3 gate, 4..7 up) for MFMA column n is c0 + 4 n + j % 4, so a lane
// owns four adjacent output columns (mode 2, the backward's recompute, stores
// gate and up as well as SiLU(gate) * up).  Plain slices hold 128 columns: row
// c0 + 8 n + j, eight adjacent output columns per lane.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_async.h"

namespace moe {

namespace {

constexpr int SK = 64;                       // K per step (128 bytes of each row)
constexpr int NT = 8;                        // 16-row weight tiles per wave
constexpr int MAXT = kStreamChunk / 16;      // 16-row token tiles per task at most
constexpr int NSTG = 2;                      // LDS stages per wave
constexpr int WROWS = 16 * NT;               // weight rows per task (128)
constexpr int BSTG = WROWS * SK * 2;         // weight bytes per stage (16 KB)
constexpr int ASTG = 16 * MAXT * SK * 2;     // token-row bytes per stage (8 KB)
constexpr int STG = BSTG + ASTG;             // bytes per stage
constexpr int WPB = 2;                       // waves per workgroup
constexpr int LDS_BYTES = WPB * NSTG * STG;  // dynamic LDS per workgroup
static_assert(MAXT == 4, "the task dispatch covers 1 to 4 tiles");
static_assert(SK == 64, "one 1 KB copy holds 8 rows of 128 bytes");

constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xf00; }

// LDS position of 16-byte chunk c of a staged row r (8 chunks a row)
MOE_DEV int cpos(int r, int c) { return c ^ (r & 7); }

}  // namespace

// (expert, row base, rows, slice, first row) of a task
struct StreamTask {
  int e, row_base, m0, rows, slice;
};

template <int MODE>
__global__ __launch_bounds__(64 * WPB, 1) void stream_gemm_kernel(StreamArgs g) {
  constexpr bool GATED = MODE != 0;
  extern __shared__ __attribute__((aligned(16))) uint8_t ssm[];
  // chunk prefix, counts and offsets in LDS: the per-task expert search must
  // not wait on dependent global loads between two tasks' weight streams
  __shared__ int cs_s[kMaxStreamExperts + 1];
  __shared__ int cnt_s[kMaxStreamExperts], off_s[kMaxStreamExperts];
  for (int i = threadIdx.x; i <= g.n_exp; i += blockDim.x) cs_s[i] = g.chunk_start[i];
  for (int i = threadIdx.x; i < g.E; i += blockDim.x) {
    cnt_s[i] = g.counts[i];
    off_s[i] = g.offsets[i];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int cols = GATED ? 64 : 128;
  const int n_slices = g.N / cols;
  const int n_tasks = cs_s[g.n_exp] * n_slices;
  const int nsteps = g.K / SK;

  const int wpb = blockDim.x >> 6;
  const int slots = gridDim.x * wpb;
  const int rounds = (n_tasks + slots - 1) / slots;
  const int active = rounds > 0 ? (n_tasks + rounds - 1) / rounds : 0;
  const int wid = blockIdx.x * wpb + (threadIdx.x >> 6);
  if (wid >= active) return;  // no barriers below

  auto decode = [&](int task) {
    // task -> (expert, slice, row chunk); tasks of an expert are slice-major
    const int cidx = task / n_slices;
    int lo = 0, hi = g.n_exp - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (cs_s[mid] <= cidx) lo = mid;
      else hi = mid - 1;
    }
    StreamTask t;
    t.e = lo;
    const bool shared = lo >= g.E;
    const int cnt = shared ? g.T : cnt_s[lo];
    t.row_base = shared ? g.TK + (lo - g.E) * g.T : off_s[lo];
    const int nch = (cnt + kStreamChunk - 1) / kStreamChunk;
    const int local = task - cs_s[lo] * n_slices;
    t.slice = local / nch;
    t.m0 = (local - t.slice * nch) * kStreamChunk;
    t.rows = min(kStreamChunk, cnt - t.m0);
    return t;
  };
  // activation row of this lane in each tile of the chunk (every lane a valid
  // row of the chunk; tiles past the rows are not multiplied)
  auto a_rows = [&](const StreamTask& t, int (&r)[MAXT]) {
#pragma unroll
    for (int i = 0; i < MAXT; ++i) {
      const int m = t.m0 + min(16 * i + (lane & 15), t.rows - 1);
      r[i] = GATED ? ((t.e >= g.E) ? m : g.perm[t.row_base + m]) : t.row_base + m;
    }
  };

  // this wave's LDS stages
  uint8_t* stg0 = ssm + (threadIdx.x >> 6) * (NSTG * STG);

  // one task with NTILE active 16-row tiles.  Each K step of 64 is copied
  // into a stage by buffer_load ... lds: the 128 weight rows (16 copies of 8
  // whole 128-byte rows, non-temporal: the weights are read once) and the
  // chunk's token rows (2 copies per tile, cacheable: they are read by every
  // slice).  The copies of step s + 1 fly while step s is multiplied.
  auto run = [&](const StreamTask& cur, const int (&rws)[MAXT], int task, auto ntile_c) {
    constexpr int NTILE = decltype(ntile_c)::value;
    constexpr int CPS = 16 + 2 * NTILE;  // copies per step
    // (uniform: the buffer resources below must sit in scalar registers)
    const int e = __builtin_amdgcn_readfirstlane(cur.e);
    const int row_base = __builtin_amdgcn_readfirstlane(cur.row_base);
    const int m0 = __builtin_amdgcn_readfirstlane(cur.m0), rows = __builtin_amdgcn_readfirstlane(cur.rows);
    const int slice = __builtin_amdgcn_readfirstlane(cur.slice);
    // weight rows of this task: row of tile j (j = 0..3 gate, 4..7 up) for
    // MFMA column n is c0 + 4 n + j % 4 (gated) or c0 + 8 n + j
    const uint32_t wbytes = uint32_t(g.N) * uint32_t(g.K) * 2u;
    const __amdgpu_buffer_rsrc_t wr0 = buffer_rsrc(g.w0 + (size_t)e * g.N * g.K, wbytes);
    const __amdgpu_buffer_rsrc_t wr1 = GATED ? buffer_rsrc(g.w1 + (size_t)e * g.N * g.K, wbytes) : wr0;
    const int c0 = GATED ? slice * 64 : slice * 128;
    // token rows: x (gated, rows gathered through perm) or this expert's own
    // staged rows
    const int a_span = __builtin_amdgcn_readfirstlane(GATED ? g.T : (e >= g.E ? g.T : cnt_s[e]));
    const __amdgpu_buffer_rsrc_t ar =
        buffer_rsrc(GATED ? g.a : g.a + (size_t)row_base * g.K, uint32_t(a_span) * uint32_t(g.K) * 2u);
    // copy i of the weight rows: staged rows 8 i .. 8 i + 7; lane l: row
    // 8 i + l/8, position l%8 = chunk (l%8) ^ (row%8)
    uint32_t woff[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rho = 8 * i + (lane >> 3), j = rho >> 4, n = rho & 15;
      const int wrow = GATED ? c0 + 4 * n + (j & 3) : c0 + 8 * n + j;
      woff[i] = (uint32_t(wrow) * uint32_t(g.K) + uint32_t(cpos(rho, lane & 7) * 8)) * 2u;
    }
    // copy m of the token rows: staged rows 8 m .. 8 m + 7 (rws: this lane's
    // row of each tile is rws[t] for tile row lane%16; copy m holds tile
    // m/2's rows 8 (m%2) .. +7, the lanes' rows taken through a shuffle)
    uint32_t aoff[2 * NTILE];
#pragma unroll
    for (int m = 0; m < 2 * NTILE; ++m) {
      const int alpha = 8 * m + (lane >> 3);          // staged token row
      const int src = __shfl(rws[m >> 1], alpha & 15);  // its A row: tile m/2, row alpha%16
      const int arow_i = GATED ? src : src - row_base;
      aoff[m] = (uint32_t(arow_i) * uint32_t(g.K) + uint32_t(cpos(alpha, lane & 7) * 8)) * 2u;
    }
    auto issue = [&](int kstep, int stage) {
      uint8_t* st = stg0 + stage * STG;
      const uint32_t ko = uint32_t(kstep) * uint32_t(SK * 2);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        copy_to_lds_async16_nt((GATED && i >= 8) ? wr1 : wr0, woff[i] + ko, st + 1024 * i);
#pragma unroll
      for (int m = 0; m < 2 * NTILE; ++m) copy_to_lds_async16(ar, aoff[m] + ko, st + BSTG + 1024 * m);
    };

    f32x4 acc[NTILE][NT];
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA q of a step takes from lane l the 8 k of chunk 2 (l/16) + q of its
    // row (both operands: every product pairs equal k)
    auto frag = [&](const uint8_t* base, int r, int q) {
      return *reinterpret_cast<const bf16x8*>(base + r * (SK * 2) + cpos(r, 2 * (lane >> 4) + q) * 16);
    };
    const int rot = (task * 7) % nsteps;
    issue(rot, 0);
    for (int s = 0; s < nsteps; ++s) {
      if (s + 1 < nsteps) {
        const int k1 = rot + s + 1;
        issue(k1 >= nsteps ? k1 - nsteps : k1, (s + 1) & 1);  // into the stage of step s - 1
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(CPS));          // step s landed
      } else {
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
      }
      asm volatile("" ::: "memory");
      const uint8_t* st = stg0 + (s & 1) * STG;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bf16x8 bf[NT], af[NTILE];
#pragma unroll
        for (int j = 0; j < NT; ++j) bf[j] = frag(st, 16 * j + (lane & 15), q);
#pragma unroll
        for (int t = 0; t < NTILE; ++t) af[t] = frag(st + BSTG, 16 * t + (lane & 15), q);
#pragma unroll
        for (int t = 0; t < NTILE; ++t)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t], bf[j], acc[t][j], 0, 0, 0);
      }
      asm volatile("" ::: "memory");
    }

    // epilogue: in tile t, lane holds rows 16 t + 4*(lane/16) + v
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * t + 4 * (lane >> 4) + v;
        if (m >= m0 + rows) continue;
        bf16_t* dst = g.out + (size_t)(row_base + m) * g.N;
        const f32x4* ac = acc[t];
        if (GATED) {
          const int c = slice * 64 + 4 * (lane & 15);
          uint2 pk;
          pk.x = uint32_t(f32_to_bf16(siluf(ac[0][v]) * ac[4][v])) |
                 (uint32_t(f32_to_bf16(siluf(ac[1][v]) * ac[5][v])) << 16);
          pk.y = uint32_t(f32_to_bf16(siluf(ac[2][v]) * ac[6][v])) |
                 (uint32_t(f32_to_bf16(siluf(ac[3][v]) * ac[7][v])) << 16);
          *reinterpret_cast<uint2*>(dst + c) = pk;
          if (MODE == 2) {  // the backward keeps G and U as well
            const size_t o = (size_t)(row_base + m) * g.N + c;
            uint2 pg, pu;
            pg.x = uint32_t(f32_to_bf16(ac[0][v])) | (uint32_t(f32_to_bf16(ac[1][v])) << 16);
            pg.y = uint32_t(f32_to_bf16(ac[2][v])) | (uint32_t(f32_to_bf16(ac[3][v])) << 16);
            pu.x = uint32_t(f32_to_bf16(ac[4][v])) | (uint32_t(f32_to_bf16(ac[5][v])) << 16);
            pu.y = uint32_t(f32_to_bf16(ac[6][v])) | (uint32_t(f32_to_bf16(ac[7][v])) << 16);
            *reinterpret_cast<uint2*>(g.out_g + o) = pg;
            *reinterpret_cast<uint2*>(g.out_u + o) = pu;
          }
        } else {
          const int c = slice * 128 + 8 * (lane & 15);
          u32x4 pk;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pk[q] = uint32_t(f32_to_bf16(ac[2 * q][v])) |
                    (uint32_t(f32_to_bf16(ac[2 * q + 1][v])) << 16);
          *reinterpret_cast<u32x4*>(dst + c) = pk;
        }
      }
  };

  StreamTask cur = decode(wid);
  int cur_rows[MAXT];
  a_rows(cur, cur_rows);
  for (int task = wid; task < n_tasks; task += active) {
    // the next task's description and token rows are fetched now and arrive
    // while this task streams
    const int ntask = task + active < n_tasks ? task + active : task;
    const StreamTask nxt = decode(ntask);
    int nxt_rows[MAXT];
    a_rows(nxt, nxt_rows);
    switch ((cur.rows + 15) >> 4) {  // uniform
      case 4: run(cur, cur_rows, task, std::integral_constant<int, 4>{}); break;
      case 3: run(cur, cur_rows, task, std::integral_constant<int, 3>{}); break;
      case 2: run(cur, cur_rows, task, std::integral_constant<int, 2>{}); break;
      default: run(cur, cur_rows, task, std::integral_constant<int, 1>{}); break;
    }
    cur = nxt;
#pragma unroll
    for (int i = 0; i < MAXT; ++i) cur_rows[i] = nxt_rows[i];
  }
}

int stream_waves_per_block(int) { return WPB; }

template <int MODE>
static hipError_t launch_mode(const StreamArgs& g, int n_blocks, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&stream_gemm_kernel<MODE>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL(stream_gemm_kernel<MODE>, dim3(n_blocks), dim3(64 * WPB), LDS_BYTES, st, g);
  return hipGetLastError();
}

hipError_t launch_stream_gemm(const StreamArgs& g, int mode, int n_blocks, hipStream_t st) {
  if (g.n_exp > kMaxStreamExperts) return hipErrorInvalidValue;
  if (mode == 2 && (g.out_g == nullptr || g.out_u == nullptr)) return hipErrorInvalidValue;
  if (g.K % SK != 0) return hipErrorInvalidValue;
  if (mode == 1) return launch_mode<1>(g, n_blocks, st);
  if (mode == 2) return launch_mode<2>(g, n_blocks, st);
  return launch_mode<0>(g, n_blocks, st);
}

}  // namespace moe
