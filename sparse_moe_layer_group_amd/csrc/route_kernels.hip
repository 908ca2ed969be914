// Routing kernels for gfx950: router logits, node-limited top-K selection with
// the loss-free bias and gates, expert histogram / prefix sum / stable
// permutation, and the bias step.
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §1.3 (Eq 13, 15)
// and §1.4 (Eq 16).
#include <algorithm>

#include "common.h"
#include "lds_async.h"
#include "kernels.h"

namespace moe {

// ============================================================================
// Router logits, split over K: P[ks][t][e] = sum_{h in chunk ks} x[t][h] W_r[h][e]
//
// fp32 MFMA 16x16x4.  Block: 256 threads (4 waves), tile 32 tokens x 256
// experts; wave w owns experts [64w, 64w+64) as 2 x 4 MFMA tiles.  Each block
// walks its K chunk in steps of 32 through LDS.  Partial sums of the chunks are
// added in a fixed order by the select kernel, so the logits are deterministic
// and each float32 accumulation chain is short.
// ============================================================================

namespace {
constexpr int RB_M = 32, RB_N = 256, RB_K = 32;
constexpr int RA_STRIDE = RB_K + 2;    // A_s row stride (floats): 2 mod 32 banks
constexpr int RB_STRIDE = RB_N + 16;   // B_s row stride (floats): 16 mod 32 banks
}  // namespace

template <typename TA>
__global__ __launch_bounds__(256) void router_logits_kernel(const TA* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            float* __restrict__ P, int T, int H,
                                                            int E, int kchunk) {
  __shared__ float A_s[RB_M * RA_STRIDE];
  __shared__ float B_s[RB_K * RB_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RB_M;
  const int e0 = blockIdx.y * RB_N;
  const int ks = blockIdx.z;
  const int k_begin = ks * kchunk;
  const int k_end = min(H, k_begin + kchunk);

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = k_begin; k0 < k_end; k0 += RB_K) {
    // A: 32 x 32 -> 1024 elements, 4 per thread
    for (int i = tid; i < RB_M * RB_K; i += 256) {
      int r = i / RB_K, c = i % RB_K;
      int t = t0 + r, k = k0 + c;
      float v = (t < T && k < k_end) ? to_f32(x[(size_t)t * H + k]) : 0.f;
      A_s[r * RA_STRIDE + c] = v;
    }
    // B: 32 x 256 floats, float4 loads
    for (int i = tid; i < RB_K * RB_N / 4; i += 256) {
      int r = i / (RB_N / 4), c4 = (i % (RB_N / 4)) * 4;
      int k = k0 + r, e = e0 + c4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < k_end) {
        if ((E & 3) == 0 && e + 3 < E) {
          v = *reinterpret_cast<const float4*>(wr + (size_t)k * E + e);
        } else {
          float tmp[4] = {0.f, 0.f, 0.f, 0.f};
          for (int q = 0; q < 4; ++q)
            if (e + q < E) tmp[q] = wr[(size_t)k * E + e + q];
          v = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
        }
      }
      float* dst = &B_s[r * RB_STRIDE + c4];
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < RB_K; kk += 4) {
      float a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = A_s[(i * 16 + (lane & 15)) * RA_STRIDE + kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = B_s[(kk + (lane >> 4)) * RB_STRIDE + wave * 64 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // D layout: lane holds rows 4*(lane/16)+q, column lane%16
  float* Pk = P + (size_t)ks * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int t = t0 + i * 16 + 4 * (lane >> 4) + q;
        int e = e0 + wave * 64 + j * 16 + (lane & 15);
        if (t < T && e < E) Pk[(size_t)t * E + e] = acc[i][j][q];
      }
}


// ============================================================================
// Router logits for bfloat16 activations through bf16 MFMAs.
//
// Every float32 router weight is the exact sum of three bfloat16 parts
// (hi = top 8 significant bits, mid = next 8, lo = rest, each a truncation
// remainder), so x * w = x*hi + x*mid + x*lo exactly for a bfloat16 x and
// bf16 MFMAs give the float32 products with float32 accumulation.  The logits
// are then one bf16 GEMM with K = 3H: router_split writes, for each expert e,
// the row [hi(W_r[:,e]) | mid(W_r[:,e]) | lo(W_r[:,e])] (Wt3 [E][3H],
// K-contiguous), and the activation row is read three times.
// ============================================================================

// 64 x 64 (k, e) tile through LDS; each thread then writes 8 consecutive k of
// one expert and one part as a 16-byte vector.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                           bf16_t* __restrict__ wt3, int H,
                                                           int E) {
  __shared__ float tile[64][65];
  const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int kk = i / 64, ee = i % 64;
    const int k = k0 + kk, e = e0 + ee;
    tile[kk][ee] = (k < H && e < E) ? wr[(size_t)k * E + e] : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int ee = i / 8, kg = (i % 8) * 8;
    const int e = e0 + ee;
    if (e >= E || k0 + kg >= H) continue;  // H % 128 == 0: a group is all in or all out
    u32x4 hi4, mid4, lo4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t part[3][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float w = tile[kg + 2 * q + h][ee];
        const uint32_t u = __float_as_uint(w);
        const uint32_t hi = u & 0xffff0000u;
        const float r1 = w - __uint_as_float(hi);              // exact
        const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(mid);            // exact, fits 8 bits
        part[0][h] = hi >> 16;
        part[1][h] = mid >> 16;
        part[2][h] = __float_as_uint(r2) >> 16;
      }
      hi4[q] = part[0][0] | (part[0][1] << 16);
      mid4[q] = part[1][0] | (part[1][1] << 16);
      lo4[q] = part[2][0] | (part[2][1] << 16);
    }
    bf16_t* row = wt3 + (size_t)e * 3 * H + k0 + kg;
    *reinterpret_cast<u32x4*>(row) = hi4;
    *reinterpret_cast<u32x4*>(row + H) = mid4;
    *reinterpret_cast<u32x4*>(row + 2 * H) = lo4;
  }
}

// ---------------------------------------------------------------------------
// Router logits for large batches: an LDS-tiled bf16 GEMM over K = 3H.
// Workgroup tile 128 tokens x 256 experts, split along K into `chunks` parts
// (P[c][t][e], added in order by the select kernel).  K steps of 32 staged by
// direct global->LDS copies (buffer_load ... lds) three steps ahead into four
// stages (24 KB each);
// the activation row of step kt is x[t][kt*32 mod H ..].  Eight waves in
// 2 x 4, each 64 x 64 as 2 x 2 MFMA 32x32x16 blocks.  Staged rows are 64 bytes
// (four 16-byte chunks at chunk ^ ((row/2) % 4)).
// ---------------------------------------------------------------------------
namespace {
constexpr int RT_TBM = 128, RT_TBN = 256, RT_TBK = 32, RT_NSTAGE = 4;
constexpr int RT_NWAVE = 8, RT_WN = 4;
constexpr int RT_ASTAGE = RT_TBM * RT_TBK, RT_BSTAGE = RT_TBN * RT_TBK;  // bf16 elements
MOE_DEV int rt_swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }
}  // namespace

__global__ __launch_bounds__(512, 1) void router_tile_kernel(const bf16_t* __restrict__ x,
                                                             const bf16_t* __restrict__ wt3,
                                                             float* __restrict__ P, int T, int H,
                                                             int E, int steps_per_chunk) {
  constexpr int ACPW = RT_TBM / 16 / RT_NWAVE;   // 1 KB copies of A per wave per step
  constexpr int BCPW = RT_TBN / 16 / RT_NWAVE;
  constexpr int CPS = ACPW + BCPW;
  static_assert(ACPW >= 1 && BCPW >= 1, "tile");
  __shared__ __attribute__((aligned(16))) bf16_t As[RT_NSTAGE * RT_ASTAGE];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[RT_NSTAGE * RT_BSTAGE];
  const int t0 = blockIdx.x * RT_TBM, e0 = blockIdx.y * RT_TBN, c = blockIdx.z;
  const int nsteps_all = 3 * H / RT_TBK;
  const int kt0 = c * steps_per_chunk;
  const int nk = min(steps_per_chunk, nsteps_all - kt0);
  const int rows = min(RT_TBM, T - t0), cols = min(RT_TBN, E - e0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / RT_WN, wn = wave % RT_WN;
  const int spp = H / RT_TBK;  // steps per part

  uint32_t aoff[ACPW], boff[BCPW];
#pragma unroll
  for (int i = 0; i < ACPW; ++i) {
    const int r = 16 * (wave * ACPW + i) + (lane >> 2);
    const int t = t0 + min(r, rows - 1);
    aoff[i] = (uint32_t(t) * uint32_t(H) + uint32_t(rt_swz(r, lane & 3) * 8)) * 2u;
  }
  // buffer resources over x [T][H] and the split router rows e0.. of Wt3 [E][3H]
  const __amdgpu_buffer_rsrc_t brs =
      buffer_rsrc(wt3 + (size_t)e0 * 3 * H, uint32_t(E - e0) * uint32_t(3 * H) * 2u);
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(x, uint32_t(T) * uint32_t(H) * 2u);
#pragma unroll
  for (int i = 0; i < BCPW; ++i) {
    const int r = 16 * (wave * BCPW + i) + (lane >> 2);
    const int e = min(r, cols - 1);
    boff[i] = (uint32_t(e) * uint32_t(3 * H) + uint32_t(rt_swz(r, lane & 3) * 8)) * 2u;
  }

  auto copy_step = [&](int j) {
    const int kt = kt0 + min(j, nk - 1);
    const int part = kt / spp;
    const uint32_t ka = uint32_t((kt - part * spp) * RT_TBK * 2);
    const uint32_t kb = uint32_t(kt * RT_TBK * 2);
    const int stage = j % RT_NSTAGE;
    bf16_t* a = As + stage * RT_ASTAGE + (16 * ACPW * wave) * RT_TBK;
    bf16_t* b = Bs + stage * RT_BSTAGE + (16 * BCPW * wave) * RT_TBK;
#pragma unroll
    for (int i = 0; i < ACPW; ++i) copy_to_lds_async16(ars, aoff[i] + ka, a + 16 * i * RT_TBK);
#pragma unroll
    for (int i = 0; i < BCPW; ++i) copy_to_lds_async16(brs, boff[i] + kb, b + 16 * i * RT_TBK);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int arow0 = wm * 64 + (lane & 31), brow0 = wn * 64 + (lane & 31);
  auto frag = [&](const bf16_t* base, int row, int chunk) {
    return *reinterpret_cast<const bf16x8*>(base + row * RT_TBK + (rt_swz(row, chunk) << 3));
  };

  constexpr int VMWAIT = (RT_NSTAGE - 2) * CPS;
  constexpr int WAITIMM = (VMWAIT & 15) | ((VMWAIT >> 4) << 14) | 0x70 | 0xf00;
#pragma unroll
  for (int p = 0; p < RT_NSTAGE - 1; ++p) copy_step(p);
  for (int j = 0; j < nk; ++j) {
    __builtin_amdgcn_s_waitcnt(WAITIMM);  // this wave's copies of step j are done
    __builtin_amdgcn_s_barrier();
    copy_step(j + RT_NSTAGE - 1);
    const bf16_t* a = As + (j % RT_NSTAGE) * RT_ASTAGE;
    const bf16_t* b = Bs + (j % RT_NSTAGE) * RT_BSTAGE;
#pragma unroll
    for (int s16 = 0; s16 < RT_TBK / 16; ++s16) {
      const int ch = 2 * s16 + (lane >> 5);
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag(a, arow0 + 32 * i, ch);
#pragma unroll
      for (int i = 0; i < 2; ++i) bf[i] = frag(b, brow0 + 32 * i, ch);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[jj], acc[i][jj], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no copy left in flight
  __builtin_amdgcn_s_barrier();

  float* Pc = P + (size_t)c * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int col = wn * 64 + 32 * jj + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r < rows && col < cols) Pc[(size_t)(t0 + r) * E + e0 + col] = acc[i][jj][v];
      }
    }
}

// ============================================================================
// Node-limited selection, one wave per token.
//
// Lane l holds experts [l*epl, (l+1)*epl).  L = sum of the split-K partials in
// chunk order; s = sigmoid(L); z = s + b.  Group scores (sum of the group_topn
// largest z of each contiguous group, added from the largest down) are formed
// by lanes 0..G-1 from LDS.  topk_groups rounds of a wave arg-max keep the
// groups, topk rounds pick the experts among the kept groups' experts; one
// extra round of each measures the near-tie gaps.  Ties go to the lower index.
// Gates are the chosen s divided by their float32 sum.  Output ids ascend.
// ============================================================================

constexpr int SEL_WAVES = 4;
constexpr int SEL_MAX_E = 512;

__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ P, int ksplit,
                                                     const float* __restrict__ bias, int T, int E,
                                                     int G, int topk_groups, int topk,
                                                     int group_topn, int32_t* __restrict__ idx_out,
                                                     float* __restrict__ gate_out,
                                                     float* __restrict__ gap_out) {
  __shared__ float z_s[SEL_WAVES][SEL_MAX_E];
  __shared__ float s_s[SEL_WAVES][SEL_MAX_E];
  __shared__ int sel_s[SEL_WAVES][33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t_raw = blockIdx.x * SEL_WAVES + wave;
  const bool valid = t_raw < T;  // no early exit: the block meets at barriers below
  const int t = valid ? t_raw : T - 1;
  const int epl = (E + 63) / 64;
  const int gsz = E / G;
  float* z = z_s[wave];
  float* s = s_s[wave];

  {
    // logits: each expert's partials summed in ascending k.  Lane l reads
    // experts l, l + 64, ... (coalesced), four partials of each at a time, so
    // a token's loads are in flight together rather than one after another.
    float Lv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) Lv[j] = 0.f;
    const float* Pt = P + (size_t)t * E;
    const size_t kst = (size_t)T * E;
    int k = 0;
    for (; k + 4 <= ksplit; k += 4) {
      float v[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = 64 * j + lane;
          v[q][j] = (j < epl && e < E) ? Pt[(size_t)(k + q) * kst + e] : 0.f;
        }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) Lv[j] += v[q][j];
    }
    for (; k < ksplit; ++k) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 64 * j + lane;
        if (j < epl && e < E) Lv[j] += Pt[(size_t)k * kst + e];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = 64 * j + lane;
      if (j < epl && e < E) {
        const float sv = sigmoidf(Lv[j]);
        s[e] = sv;
        z[e] = sv + bias[e];
      }
    }
  }
  __syncthreads();

  // group scores: the sum of the group_topn largest z of each group
  float gscore = -INFINITY;
  int gidx = 0x7fffffff;
  const int lpg = gsz / epl;  // lanes per group when a lane's experts lie in one group
  const bool par = group_topn <= 2 && gsz % epl == 0 && (lpg & (lpg - 1)) == 0 && lpg <= 32 &&
                   G * lpg <= 64;
  if (par) {
    // each lane: the two largest of its experts, then merged across the
    // group's lanes (xor steps stay inside an aligned power-of-two lane group)
    float t1 = -INFINITY, t2 = -INFINITY;
    for (int j = 0; j < epl; ++j) {
      const int e = lane * epl + j;
      const float v = (e < E) ? z[e] : -INFINITY;
      if (v > t1) {
        t2 = t1;
        t1 = v;
      } else if (v > t2) {
        t2 = v;
      }
    }
    for (int off = 1; off < lpg; off <<= 1) {
      const float o1 = __shfl_xor(t1, off, kWave), o2 = __shfl_xor(t2, off, kWave);
      const float hi = fmaxf(t1, o1);
      t2 = (t1 >= o1) ? fmaxf(t2, o1) : fmaxf(t1, o2);
      t1 = hi;
    }
    const float score = group_topn == 1 ? t1 : t1 + t2;
    const float mine = __shfl(score, (lane < G ? lane : 0) * lpg, kWave);
    if (lane < G) {
      gscore = mine;
      gidx = lane;
    }
  } else if (lane < G) {
    // lane g < G scans its group keeping the group_topn largest (descending)
    float top[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int i = 0; i < gsz; ++i) {
      float v = z[lane * gsz + i];
      // insert into the descending list of length group_topn
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < group_topn && v > top[q]) {
          float tmp = top[q];
          top[q] = v;
          v = tmp;
        }
      }
    }
    float acc = top[0];
#pragma unroll
    for (int q = 1; q < 4; ++q)
      if (q < group_topn) acc += top[q];
    gscore = acc;
    gidx = lane;
  }
  // keep topk_groups groups; one more round for the gap
  uint64_t kept = 0;
  float glast = 0.f, gnext = -INFINITY;
  {
    float v = gscore;
    int i = gidx;
    for (int r = 0; r <= topk_groups && r < G; ++r) {
      float bv = v;
      int bi = i;
      wave_argmax(bv, bi);
      if (r < topk_groups) {
        kept |= (1ull << bi);
        glast = bv;
      } else {
        gnext = bv;
      }
      if (lane == bi) {
        v = -INFINITY;
        i = 0x7fffffff;
      }
    }
  }
  // expert rounds among the kept groups
  float zl[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int e = lane * epl + j;
    zl[j] = (j < epl && e < E && ((kept >> (e / gsz)) & 1ull)) ? z[e] : -INFINITY;
  }
  float elast = 0.f, enext = -INFINITY;
  for (int r = 0; r <= topk; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (zl[j] > bv) {  // lanes hold ascending ids: strict '>' keeps the lower id
        bv = zl[j];
        bi = lane * epl + j;
      }
    }
    wave_argmax(bv, bi);
    if (r < topk) {
      if (lane == 0) sel_s[wave][r] = bi;
      elast = bv;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (lane * epl + j == bi) zl[j] = -INFINITY;
    } else {
      enext = bv;
    }
  }
  __syncthreads();
  // sort the chosen ids ascending and write ids and gates
  float ssum = 0.f;
  for (int r = 0; r < topk; ++r) ssum += s[sel_s[wave][r]];
  if (valid && lane < topk) {
    int me = sel_s[wave][lane];
    int rank = 0;
    for (int r = 0; r < topk; ++r) rank += (sel_s[wave][r] < me) ? 1 : 0;
    idx_out[(size_t)t * topk + rank] = me;
    gate_out[(size_t)t * topk + rank] = s[me] / ssum;
  }
  if (valid && gap_out != nullptr && lane == 0) {
    float eg = (enext == -INFINITY) ? INFINITY : (elast - enext);
    float gg = (topk_groups >= G || gnext == -INFINITY) ? INFINITY : (glast - gnext);
    gap_out[t] = fminf(eg, gg);
  }
}

// ============================================================================
// Stable permutation by expert (integer work, deterministic).
//
// Tokens are cut into chunks of 64.  hist: per chunk, a 64-bit token mask per
// expert (LDS atomic OR, order-free) and its popcount.  scan (one block): counts,
// offsets, and each chunk's first row per expert; also the GEMM m-tile starts.
// scatter: the row of assignment (t,k) is the chunk base of its expert plus the
// number of earlier tokens of the chunk that chose the same expert.
// ============================================================================

constexpr int CHUNK = 64;

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                   int E, uint64_t* __restrict__ masks,
                                                   int32_t* __restrict__ hist) {
  __shared__ unsigned long long m_s[SEL_MAX_E];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) m_s[e] = 0ull;
  __syncthreads();
  const int t0 = c * CHUNK;
  const int nt = min(CHUNK, T - t0);
  for (int a = threadIdx.x; a < nt * K; a += blockDim.x) {
    int tl = a / K;
    int e = idx[(size_t)(t0 + tl) * K + (a % K)];
    atomicOr(&m_s[e], 1ull << tl);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    masks[(size_t)c * E + e] = m_s[e];
    hist[(size_t)c * E + e] = __popcll(m_s[e]);
  }
}

// Exclusive prefix sums of v over the block's threads in thread order (all
// threads call it; blockDim.x a multiple of 64, at most 1024).  Returns the
// exclusive sum; *total receives the block total.
MOE_DEV int block_exclusive_scan(int v, int* wave_tot /* LDS [16] */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int tw = wave_tot[w];
    before += (w < wave) ? tw : 0;
    all += tw;
  }
  __syncthreads();  // wave_tot may be reused by the next call
  *total = all;
  return before + inc - v;
}

// Work tables of the expert GEMMs over E routed experts then S shared experts
// (T rows each), both with E+S+1 entries:
//   chunk_start: prefix of ceil(rows/kStreamChunk) over experts with rows <= stream_max
//                (served by the weight-streaming GEMM);
//   mt_start:    prefix of ceil(rows/bm) over the other experts (tiled GEMM).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ hist, int nchunks,
                                                   int E, int S, int T, int K,
                                                   int32_t* __restrict__ base,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int stream_max,
                                                   int32_t* __restrict__ chunk_start, int bm,
                                                   int32_t* __restrict__ mt_start) {
  constexpr int QMAX = 8;
  __shared__ int wave_tot[16];
  __shared__ int part_s[QMAX][SEL_MAX_E];  // per expert: chunk counts of each thread's range
  __shared__ int off_s[SEL_MAX_E];
  // Q threads per expert (as many as the block holds, at most QMAX): thread
  // (q, ex) covers the contiguous chunks [c0, c1) of expert ex, so every
  // thread has few chunks, and the unrolled loops issue their independent
  // loads together (one thread walking all chunks waited on them serially)
  const int Q = min(QMAX, int(blockDim.x) / E);
  const int ex = threadIdx.x % E, q = threadIdx.x / E;
  const bool part = q < Q;
  const int c0 = part ? int((long long)q * nchunks / Q) : 0;
  const int c1 = part ? int((long long)(q + 1) * nchunks / Q) : 0;
  int psum = 0;
#pragma unroll 8
  for (int c = c0; c < c1; ++c) psum += hist[(size_t)c * E + ex];
  if (part) part_s[q][ex] = psum;
  __syncthreads();

  const int e = threadIdx.x;  // blockDim.x >= E + S + 1
  int cnt = 0;
  if (e < E)
    for (int i = 0; i < Q; ++i) cnt += part_s[i][e];
  // rows of entry e of the work tables: routed experts, then the shared ones
  const int rows = e < E ? cnt : (e < E + S ? T : 0);
  const bool str = rows <= stream_max;
  int tot;
  const int off = block_exclusive_scan(e < E ? cnt : 0, wave_tot, &tot);
  const int sa = block_exclusive_scan(str ? (rows + kStreamChunk - 1) / kStreamChunk : 0, wave_tot, &tot);
  const int sb = block_exclusive_scan(str ? 0 : (rows + bm - 1) / bm, wave_tot, &tot);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    off_s[e] = off;
  }
  if (e == E) offsets[E] = off;
  if (e <= E + S) {
    chunk_start[e] = sa;
    mt_start[e] = sb;
  }
  __syncthreads();
  // each chunk's first row per expert: the expert's offset plus the rows of
  // its earlier chunks
  if (part) {
    int run = off_s[ex];
    for (int i = 0; i < q; ++i) run += part_s[i][ex];
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
      const int h = hist[(size_t)c * E + ex];
      base[(size_t)c * E + ex] = run;
      run += h;
    }
  }
}

// Small batches (at most PERM_SMALL_T tokens): hist, scan and scatter in one
// workgroup, the chunk masks in LDS.
constexpr int PERM_SMALL_T = 512;
constexpr int PERM_SMALL_NC = PERM_SMALL_T / CHUNK;

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ idx, int T, int K, int E, int S, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ slot,
    int stream_max, int32_t* __restrict__ chunk_start, int bm, int32_t* __restrict__ mt_start) {
  __shared__ unsigned long long m_s[PERM_SMALL_NC][SEL_MAX_E];
  __shared__ int base_s[PERM_SMALL_NC][SEL_MAX_E];
  __shared__ int wave_tot[16];
  const int nc = (T + CHUNK - 1) / CHUNK;
  for (int i = threadIdx.x; i < nc * E; i += blockDim.x) m_s[i / E][i % E] = 0ull;
  __syncthreads();
  for (int a = threadIdx.x; a < T * K; a += blockDim.x) {
    const int t = a / K;
    atomicOr(&m_s[t / CHUNK][idx[a]], 1ull << (t % CHUNK));
  }
  __syncthreads();
  const int e = threadIdx.x;  // blockDim.x >= E + S + 1
  int cnt = 0;
  if (e < E)
    for (int c = 0; c < nc; ++c) cnt += __popcll(m_s[c][e]);
  const int rows = e < E ? cnt : (e < E + S ? T : 0);
  const bool str = rows <= stream_max;
  int tot;
  const int off = block_exclusive_scan(e < E ? cnt : 0, wave_tot, &tot);
  const int sa = block_exclusive_scan(str ? (rows + kStreamChunk - 1) / kStreamChunk : 0, wave_tot, &tot);
  const int sb = block_exclusive_scan(str ? 0 : (rows + bm - 1) / bm, wave_tot, &tot);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    int run = off;
    for (int c = 0; c < nc; ++c) {
      base_s[c][e] = run;
      run += __popcll(m_s[c][e]);
    }
  }
  if (e == E) offsets[E] = off;
  if (e <= E + S) {
    chunk_start[e] = sa;
    mt_start[e] = sb;
  }
  __syncthreads();
  for (int a = threadIdx.x; a < T * K; a += blockDim.x) {
    const int t = a / K, tl = t % CHUNK, c = t / CHUNK;
    const int ex = idx[a];
    const uint64_t below = (tl == 0) ? 0ull : (m_s[c][ex] & ((1ull << tl) - 1ull));
    const int row = base_s[c][ex] + __popcll(below);
    slot[a] = row;
    perm[row] = t;
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx, int T,
                                                      int K, int E,
                                                      const uint64_t* __restrict__ masks,
                                                      const int32_t* __restrict__ base,
                                                      int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ slot) {
  const int c = blockIdx.x;
  const int t0 = c * CHUNK;
  const int nt = min(CHUNK, T - t0);
  for (int a = threadIdx.x; a < nt * K; a += blockDim.x) {
    int tl = a / K;
    int t = t0 + tl;
    int e = idx[(size_t)t * K + (a % K)];
    uint64_t m = masks[(size_t)c * E + e];
    uint64_t below = (tl == 0) ? 0ull : (m & ((1ull << tl) - 1ull));
    int row = base[(size_t)c * E + e] + __popcll(below);
    slot[(size_t)t * K + (a % K)] = row;
    perm[row] = t;
  }
}

// ============================================================================
// Loss-free bias step ([V3] §1.4): one thread per expert.
// ============================================================================

__global__ void bias_update_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias,
                                   int E, long long TK, float gamma) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  long long load = (long long)counts[e] * E;
  float b = bias[e];
  if (load > TK) b = b - gamma;
  else if (load < TK) b = b + gamma;
  bias[e] = b;
}

// ============================================================================
// launchers
// ============================================================================

// K chunks of the router: about H/8 each, a multiple of 128 (H % 128 == 0)
static int router_chunk(int H) { return ((H + 7) / 8 + 127) / 128 * 128; }

// Small batches: the bf16x3 router reading W_r (float32 [H][E]) directly.
// P[ks][t][e] for one K chunk: wave tile 32 tokens x 32 experts (2 x 2 MFMA
// 16x16x32 tiles), block = 4 waves over 128 experts.  Operands are loaded
// straight from global memory in MFMA order with the 128-wide step K map of
// the streaming GEMM (lane l owns k = 32*(l/16) .. +31 of each step).  Each
// lane loads the 8 consecutive k of its expert column as float32 (W_r stride
// E) and splits them into the hi / mid / lo bfloat16 parts in registers, so
// no separate split pass runs (a split pass plus the MFMA kernel measured
// 44 us at 256 tokens, this kernel 26 us).
__global__ __launch_bounds__(256) void router_fused_kernel(const bf16_t* __restrict__ x,
                                                           const float* __restrict__ wr,
                                                           float* __restrict__ P, int T, int H,
                                                           int E, int kchunk) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32;
  const int e0 = blockIdx.y * 128 + wave * 32;
  const int ks = blockIdx.z;
  const int kb = ks * kchunk, ke = min(H, kb + kchunk);
  if (e0 >= E) return;  // whole wave; no barrier in this kernel
  const int koff = 32 * (lane >> 4);
  const bf16_t* arow[2];
  int ecol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + i * 16 + (lane & 15);
    arow[i] = (t < T) ? x + (size_t)t * H + koff : nullptr;
    ecol[i] = e0 + i * 16 + (lane & 15);
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = kb; k < ke; k += 128) {
    u32x4 a[2][4];
    float w[2][4][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        a[i][q] = arow[i] ? *reinterpret_cast<const u32x4*>(arow[i] + k + q * 8)
                          : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 8; ++r)
          w[j][q][r] = (ecol[j] < E) ? wr[(size_t)(k + koff + 8 * q + r) * E + ecol[j]] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 b[3][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t pr[3][2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float v = w[j][q][2 * h + u];
            const uint32_t hi = __float_as_uint(v) & 0xffff0000u;
            const float r1 = v - __uint_as_float(hi);              // exact
            const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
            const float r2 = r1 - __uint_as_float(mid);            // exact, fits 8 bits
            pr[0][u] = hi >> 16;
            pr[1][u] = mid >> 16;
            pr[2][u] = __float_as_uint(r2) >> 16;
          }
#pragma unroll
          for (int pp = 0; pp < 3; ++pp) b[pp][j][h] = pr[pp][0] | (pr[pp][1] << 16);
        }
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[i][q]), __builtin_bit_cast(bf16x8, b[pp][j]),
                acc[i][j], 0, 0, 0);
    }
  }
  float* Pk = P + (size_t)ks * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + i * 16 + 4 * (lane >> 4) + q;
        const int e = e0 + j * 16 + (lane & 15);
        if (t < T && e < E) Pk[(size_t)t * E + e] = acc[i][j][q];
      }
}

int router_ksplit(int H) {
  const int chunk = router_chunk(H);
  return (H + chunk - 1) / chunk;
}

// Large bf16 batches use the tiled router: K = 3H split into chunks so that
// about 256 workgroups run (at most router_ksplit(H), the partials the
// workspace holds).  Returns the number of partials written (0: not used).
static int router_tile_chunks(int T, int H, int E) {
  if (T < 2048) return 0;
  const int tiles = ((T + RT_TBM - 1) / RT_TBM) * ((E + RT_TBN - 1) / RT_TBN);
  int chunks = std::max(1, std::min(router_ksplit(H), 256 / tiles));
  const int nsteps = 3 * H / RT_TBK;
  const int spc = (nsteps + chunks - 1) / chunks;
  return (nsteps + spc - 1) / spc;  // no empty chunk
}

int router_partials(int T, int H, int E, bool x_bf16) {
  const int tc = x_bf16 ? router_tile_chunks(T, H, E) : 0;
  return tc > 0 ? tc : router_ksplit(H);
}

size_t router_split_bytes(int H, int E) { return (size_t)3 * H * E * sizeof(bf16_t); }

hipError_t launch_router(const void* x, bool x_bf16, const float* wr, bf16_t* wt3, float* P,
                         int T, int H, int E, hipStream_t st) {
  const int ks = router_ksplit(H);
  const int chunk = router_chunk(H);
  if (x_bf16) {
    const int tc = router_tile_chunks(T, H, E);
    if (tc == 0) {
      hipLaunchKernelGGL(router_fused_kernel, dim3((T + 31) / 32, (E + 127) / 128, ks), dim3(256),
                         0, st, static_cast<const bf16_t*>(x), wr, P, T, H, E, chunk);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(router_split_kernel, dim3((H + 63) / 64, (E + 63) / 64), dim3(256), 0, st,
                       wr, wt3, H, E);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nsteps = 3 * H / RT_TBK;
    const int spc = (nsteps + tc - 1) / tc;
    hipLaunchKernelGGL(router_tile_kernel,
                       dim3((T + RT_TBM - 1) / RT_TBM, (E + RT_TBN - 1) / RT_TBN, tc), dim3(512),
                       0, st, static_cast<const bf16_t*>(x), wt3, P, T, H, E, spc);
  } else {
    dim3 grid((T + RB_M - 1) / RB_M, (E + RB_N - 1) / RB_N, ks);
    hipLaunchKernelGGL(router_logits_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(x), wr, P, T, H, E, chunk);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float* P, int ksplit, const float* bias, int T, int E, int G,
                         int topk_groups, int topk, int group_topn, int32_t* idx, float* gate,
                         float* gap, hipStream_t st) {
  dim3 grid((T + SEL_WAVES - 1) / SEL_WAVES);
  hipLaunchKernelGGL(select_kernel, grid, dim3(64 * SEL_WAVES), 0, st, P, ksplit, bias, T, E, G,
                     topk_groups, topk, group_topn, idx, gate, gap);
  return hipGetLastError();
}

int perm_chunks(int T) { return (T + CHUNK - 1) / CHUNK; }

hipError_t launch_permute(const int32_t* idx, int T, int K, int E, int S, uint64_t* masks,
                          int32_t* hist, int32_t* base, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* slot, int stream_max, int32_t* chunk_start,
                          int bm, int32_t* mt_start, hipStream_t st) {
  const int nc = perm_chunks(T);
  if (T <= PERM_SMALL_T) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, st, idx, T, K, E, S, counts,
                       offsets, perm, slot, stream_max, chunk_start, bm, mt_start);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(hist_kernel, dim3(nc), dim3(256), 0, st, idx, T, K, E, masks, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, hist, nc, E, S, T, K, base, counts,
                     offsets, stream_max, chunk_start, bm, mt_start);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(nc), dim3(256), 0, st, idx, T, K, E, masks, base, perm,
                     slot);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, float* bias, int E, long long TK,
                              float gamma, hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, st, counts, bias, E,
                     TK, gamma);
  return hipGetLastError();
}

}  // namespace moe
