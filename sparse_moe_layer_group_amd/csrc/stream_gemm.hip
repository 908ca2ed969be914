// Weight-streaming grouped GEMM for experts with few rows (decode-sized batches).
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §1.1 (SwiGLU
// experts) and §5.1 (a decode expert sees few tokens, so its cost is reading
// its weights from memory, not arithmetic).
//
// Work unit = one wave: (expert, column slice, chunk of up to 16 rows).  The
// wave streams the 128 weight rows of its slice over the whole K range straight
// from HBM into MFMA operand registers (no LDS), one 64-wide K step (16 KB) at
// a time, and multiplies them with its token rows gathered from L2 (each token
// row is fetched once per 128 weight rows).  One 4-wave workgroup per CU:
// about 64 KB in flight per CU streams HBM fastest on MI355X; deeper pipelines
// or more waves per CU measured slower (the extra outstanding lines contend in
// L2).
//
// Balanced persistent grid: all tasks cost the same, so with n tasks and S
// wave slots the kernel runs k = ceil(n/S) rounds on W = ceil(n/k) waves
// (wave w takes tasks w, w+W, ...), and every active wave finishes within one
// task of the others.  Dealing n tasks over all S slots instead would leave a
// partial last round whose duration is that of a full one.
//
// K order inside a 64-wide step: lane l owns the 16 consecutive k starting at
// 16*(l/16) and feeds its 16-byte chunk q (k = 16*(l/16) + 8q .. +7) to the
// q-th of two 16x16x32 MFMAs.  A and B use the same map, so every product
// pairs equal k.  Steps start at a task-dependent rotation of K so that
// concurrent waves do not all read the same column offset of their rows.
//
// Column map: gated slices hold 64 output columns; weight row of tile j
// (j = 0..3 gate, 4..7 up) for lane l is c0 + 4*(l%16) + (j%4), so a lane
// owns four adjacent output columns (mode 2, the backward's recompute, stores
// gate and up as well as SiLU(gate) * up).  Plain slices hold 128 columns: row
// c0 + 8*(l%16) + j, eight adjacent output columns per lane.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int SK = 64;  // K per step
constexpr int NT = 8;   // 16-row weight tiles per wave

MOE_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Every lane loads unconditionally (rows past the expert's count read a valid
// row of the chunk and their outputs are never stored), so the compiler can
// count outstanding loads exactly.
MOE_DEV void load_step(u32x4 (&b)[NT][2], u32x4 (&a)[2], const bf16_t* const (&brow)[NT],
                       const bf16_t* arow, int koff) {
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int q = 0; q < 2; ++q) b[j][q] = *reinterpret_cast<const u32x4*>(brow[j] + koff + q * 8);
#pragma unroll
  for (int q = 0; q < 2; ++q) a[q] = *reinterpret_cast<const u32x4*>(arow + koff + q * 8);
}

MOE_DEV void mma_step(f32x4 (&acc)[NT], const u32x4 (&b)[NT][2], const u32x4 (&a)[2]) {
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int j = 0; j < NT; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[q]), as_bf16x8(b[j][q]), acc[j],
                                                       0, 0, 0);
}

}  // namespace

// (expert, row base, rows, slice, first row) of a task
struct StreamTask {
  int e, row_base, m0, rows, slice;
};

template <int MODE>
__global__ __launch_bounds__(256, 1) void stream_gemm_kernel(StreamArgs g) {
  constexpr bool GATED = MODE != 0;
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
  const int koff0 = 16 * (lane >> 4);

  const int slots = gridDim.x * 4;
  const int rounds = (n_tasks + slots - 1) / slots;
  const int active = rounds > 0 ? (n_tasks + rounds - 1) / rounds : 0;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
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
    const int nch = (cnt + 15) >> 4;
    const int local = task - cs_s[lo] * n_slices;
    t.slice = local / nch;
    t.m0 = (local - t.slice * nch) * 16;
    t.rows = min(16, cnt - t.m0);
    return t;
  };
  // activation row of this lane (every lane a valid row of the chunk)
  auto a_row = [&](const StreamTask& t) {
    const int m = t.m0 + min(lane & 15, t.rows - 1);
    if (GATED) return (t.e >= g.E) ? m : g.perm[t.row_base + m];
    return t.row_base + m;
  };

  StreamTask cur = decode(wid);
  int cur_row = a_row(cur);
  for (int task = wid; task < n_tasks; task += active) {
    // the next task's description and token row are fetched now and arrive
    // while this task streams
    const int ntask = task + active < n_tasks ? task + active : task;
    const StreamTask nxt = decode(ntask);
    const int nxt_row = a_row(nxt);

    const int e = cur.e, row_base = cur.row_base, m0 = cur.m0, rows = cur.rows;
    const int slice = cur.slice;
    const bf16_t* arow = g.a + (size_t)cur_row * g.K + koff0;
    const bf16_t* brow[NT];
    const bf16_t* w0 = g.w0 + (size_t)e * g.N * g.K;
    if (GATED) {
      const bf16_t* w1 = g.w1 + (size_t)e * g.N * g.K;
      const int c = slice * 64 + 4 * (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        brow[j] = w0 + (size_t)(c + j) * g.K + koff0;
        brow[4 + j] = w1 + (size_t)(c + j) * g.K + koff0;
      }
    } else {
      const int c = slice * 128 + 8 * (lane & 15);
#pragma unroll
      for (int j = 0; j < NT; ++j) brow[j] = w0 + (size_t)(c + j) * g.K + koff0;
    }

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int rot = (task * 7) % nsteps;
    u32x4 b[NT][2], a[2];
    for (int s = 0; s < nsteps; ++s) {
      const int k = rot + s;
      load_step(b, a, brow, arow, (k >= nsteps ? k - nsteps : k) * SK);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(acc, b, a);
      __builtin_amdgcn_sched_barrier(0);
    }

    // epilogue: lane holds rows 4*(lane/16)+t of the 16-row tile
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = m0 + 4 * (lane >> 4) + t;
      if (m >= m0 + rows) continue;
      bf16_t* dst = g.out + (size_t)(row_base + m) * g.N;
      if (GATED) {
        const int c = slice * 64 + 4 * (lane & 15);
        uint2 pk;
        pk.x = uint32_t(f32_to_bf16(siluf(acc[0][t]) * acc[4][t])) |
               (uint32_t(f32_to_bf16(siluf(acc[1][t]) * acc[5][t])) << 16);
        pk.y = uint32_t(f32_to_bf16(siluf(acc[2][t]) * acc[6][t])) |
               (uint32_t(f32_to_bf16(siluf(acc[3][t]) * acc[7][t])) << 16);
        *reinterpret_cast<uint2*>(dst + c) = pk;
        if (MODE == 2) {  // the backward keeps G and U as well
          const size_t o = (size_t)(row_base + m) * g.N + c;
          uint2 pg, pu;
          pg.x = uint32_t(f32_to_bf16(acc[0][t])) | (uint32_t(f32_to_bf16(acc[1][t])) << 16);
          pg.y = uint32_t(f32_to_bf16(acc[2][t])) | (uint32_t(f32_to_bf16(acc[3][t])) << 16);
          pu.x = uint32_t(f32_to_bf16(acc[4][t])) | (uint32_t(f32_to_bf16(acc[5][t])) << 16);
          pu.y = uint32_t(f32_to_bf16(acc[6][t])) | (uint32_t(f32_to_bf16(acc[7][t])) << 16);
          *reinterpret_cast<uint2*>(g.out_g + o) = pg;
          *reinterpret_cast<uint2*>(g.out_u + o) = pu;
        }
      } else {
        const int c = slice * 128 + 8 * (lane & 15);
        u32x4 pk;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pk[q] = uint32_t(f32_to_bf16(acc[2 * q][t])) |
                  (uint32_t(f32_to_bf16(acc[2 * q + 1][t])) << 16);
        *reinterpret_cast<u32x4*>(dst + c) = pk;
      }
    }
    cur = nxt;
    cur_row = nxt_row;
  }
}

hipError_t launch_stream_gemm(const StreamArgs& g, int mode, int n_blocks, hipStream_t st) {
  if (g.n_exp > kMaxStreamExperts) return hipErrorInvalidValue;
  if (mode == 2 && (g.out_g == nullptr || g.out_u == nullptr)) return hipErrorInvalidValue;
  if (mode == 1) hipLaunchKernelGGL(stream_gemm_kernel<1>, dim3(n_blocks), dim3(256), 0, st, g);
  else if (mode == 2) hipLaunchKernelGGL(stream_gemm_kernel<2>, dim3(n_blocks), dim3(256), 0, st, g);
  else hipLaunchKernelGGL(stream_gemm_kernel<0>, dim3(n_blocks), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace moe
