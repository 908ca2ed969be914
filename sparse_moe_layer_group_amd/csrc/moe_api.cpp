// C ABI of the gfx950 MoE layer library: argument validation, workspace
// carving and launch sequencing.  Every step of the layer runs in the HIP
// kernels (route_kernels.hip, gemm_kernels.hip, stream_gemm.hip,
// tile_gemm.hip, fp8_kernels.hip); this file only checks arguments and
// enqueues them on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <cstring>
#include <vector>

#include "../../include/moe.h"
#include "bwd.h"
#include "kernels.h"

namespace {

using moe::bf16_t;

struct Layout {
  size_t wt3, P, idx, gate, counts, offsets, perm, slot, gap, masks, hist, base, chunk_start,
      mt_start;
  size_t hst, yst;
  size_t hs, xq, xs;  // E4M3 weights: H scales, quantised x and its scales
  size_t bal_sn, bal_ids, bal_psum, bal_pcnt, bal_end;  // balance loss (after the routing part)
  size_t route_total, total;
};

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

size_t elem_bytes(int dt) { return dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1); }

Layout make_layout(const moe_cfg& c, int64_t T) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t E = c.n_experts, K = c.topk, S = c.n_shared, H = c.hidden, I = c.inter;
  const size_t TK = size_t(T) * K;
  const size_t nc = size_t(moe::perm_chunks(int(T)));
  L.wt3 = take(c.act_dtype == MOE_BF16 ? moe::router_split_bytes(c.hidden, c.n_experts) : 0);
  L.P = take(size_t(moe::router_ksplit(c.hidden)) * T * E * 4);
  L.idx = take(TK * 4);
  L.gate = take(TK * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(TK * 4);
  L.slot = take(TK * 4);
  L.gap = take(size_t(T) * 4);
  L.masks = take(nc * E * 8);
  L.hist = take(nc * E * 4);
  L.base = take(nc * E * 4);
  L.chunk_start = take((E + S + 1) * 4);
  L.mt_start = take((E + S + 1) * 4);
  L.route_total = off;
  const size_t rows = TK + S * size_t(T);
  const size_t es = elem_bytes(c.act_dtype);
  if (c.w_dtype == MOE_E4M3) {
    L.hst = take(rows * I);             // E4M3 codes of H
    L.hs = take(rows * (I / 128) * 4);
    L.xq = take(size_t(T) * H);
    L.xs = take(size_t(T) * (H / 128) * 4);
  } else {
    L.hst = take(rows * I * es);
  }
  L.yst = take(rows * H * es);
  L.total = off;
  // the balance loss reuses the space after the routing part
  size_t b = L.route_total;
  auto take_b = [&](size_t bytes) {
    size_t o = b;
    b += align_up(bytes);
    return o;
  };
  L.bal_sn = take_b(size_t(T) * E * 4);
  L.bal_ids = take_b(TK * 4);
  L.bal_psum = take_b(size_t(T) * E * 8);  // at most T chunk rows of E partial sums
  L.bal_pcnt = take_b(size_t(T) * E * 4);
  L.bal_end = b;
  L.total = std::max(L.total, L.bal_end);
  return L;
}

int validate_cfg(const moe_cfg* c) {
  if (c == nullptr) return MOE_ERR_NULL;
  if (c->hidden <= 0 || c->inter <= 0 || c->n_experts <= 0 || c->n_groups <= 0) return MOE_ERR_SHAPE;
  if (c->hidden % 128 != 0 || c->inter % 128 != 0) return MOE_ERR_SHAPE;
  if (c->n_experts > 512 || c->n_groups > 64 || c->n_experts % c->n_groups != 0) return MOE_ERR_SHAPE;
  const int gsz = c->n_experts / c->n_groups;
  if (c->group_topn < 1 || c->group_topn > 4 || c->group_topn > gsz) return MOE_ERR_SHAPE;
  if (c->topk_groups < 1 || c->topk_groups > c->n_groups) return MOE_ERR_SHAPE;
  if (c->topk < 1 || c->topk > 32 || c->topk > c->topk_groups * gsz) return MOE_ERR_SHAPE;
  if (c->n_shared < 0 || c->n_shared > 1) return MOE_ERR_SHAPE;
  const bool f32 = c->act_dtype == MOE_F32 && c->w_dtype == MOE_F32;
  const bool bf16 = c->act_dtype == MOE_BF16 && c->w_dtype == MOE_BF16;
  const bool fp8 = c->act_dtype == MOE_BF16 && c->w_dtype == MOE_E4M3;
  if (!f32 && !bf16 && !fp8) return MOE_ERR_DTYPE;
  // the E4M3 GEMM holds at most 128 weight scales along K per wave
  if (fp8 && (c->hidden > 16384 || c->inter > 16384)) return MOE_ERR_SHAPE;
  // one expert matrix spans less than 4 GiB (32-bit buffer ranges of the
  // tiled GEMMs), and so do the router's bf16 weight parts [E][3H]
  const int64_t wb = int64_t(elem_bytes(c->w_dtype));
  if (int64_t(c->hidden) * c->inter * wb >= (int64_t(1) << 32)) return MOE_ERR_SHAPE;
  if (int64_t(c->n_experts) * 3 * c->hidden * 2 >= (int64_t(1) << 32)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// T bounds: row counts fit int32, and T activation rows (all of x, or one
// expert's staged rows, at most T) span less than 4 GiB, the reach of the
// tiled GEMMs' 32-bit buffer ranges and offsets.
int validate_T(const moe_cfg* c, int64_t T) {
  if (T < 0) return MOE_ERR_SHAPE;
  if (T * int64_t(c->topk + c->n_shared) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  const int64_t width = std::max<int64_t>(c->hidden, c->inter) * int64_t(elem_bytes(c->act_dtype));
  if (T * width >= (int64_t(1) << 32)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// gfx950 check, cached per device
std::atomic<int> g_arch_state[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MOE_OK : MOE_ERR_DEVICE;
}

// ---------------------------------------------------------------- instrumentation

enum Slot {
  K_ROUTER = 0, K_SELECT, K_PERMUTE, K_GATEUP, K_DOWN, K_COMBINE, K_BIAS, K_QUANT, K_BAL,
  K_BWD_RECOMPUTE, K_BWD_COMBINE, K_BWD_DH, K_BWD_DX, K_BWD_WGRAD, K_BWD_ROUTER,
  K_BWD_RETILE,
  K_NSLOTS
};
const char* const kSlotNames[K_NSLOTS] = {
    "router_logits", "select",        "permute",       "gemm_gate_up",  "gemm_down",
    "combine",       "bias_update",   "quantize",      "balance_loss",  "bwd_recompute",
    "bwd_combine",   "bwd_dgrad_down", "bwd_dgrad_gate_up", "bwd_wgrad", "bwd_router_dx",
    "bwd_retile_128x1"};

struct Prof {
  bool on = false;
  std::vector<hipEvent_t> pool;
  struct Rec { int slot; hipEvent_t a, b; };
  std::vector<Rec> recs;
  double ms[K_NSLOTS] = {0};
  int n[K_NSLOTS] = {0};
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
// Instrumentation state is per host thread: calls on distinct workspaces from
// different threads stay independent with profiling on.  A thread's events
// are kept for reuse until the process ends.
thread_local Prof g_prof;

// run one launcher, bracketed by events when instrumentation is on
template <typename F> hipError_t timed(int slot, hipStream_t st, F&& f) {
  if (!g_prof.on) return f();
  hipEvent_t a = g_prof.get(), b = g_prof.get();
  if (a == nullptr || b == nullptr) {
    if (a != nullptr) g_prof.pool.push_back(a);
    if (b != nullptr) g_prof.pool.push_back(b);
    return hipErrorOutOfMemory;
  }
  hipError_t err = hipEventRecord(a, st);
  if (err == hipSuccess) err = f();
  hipError_t end = err == hipSuccess ? hipEventRecord(b, st) : err;
  if (end == hipSuccess) {
    g_prof.recs.push_back({slot, a, b});
  } else {
    g_prof.pool.push_back(a);
    g_prof.pool.push_back(b);
  }
  return err != hipSuccess ? err : end;
}

#define MOE_TRY(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

template <typename P> P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

struct RoutePtrs {
  int32_t *idx, *counts, *offsets, *perm, *slot;
  float *gate, *gap;
};

// Experts with at most this many rows go to the weight-streaming GEMM; the
// rest to the tiled GEMM.  When the average expert has <= 32 rows (decode)
// every expert streams, the shared one included.
int stream_max_rows(const moe_cfg& c, int T) {
  if (c.act_dtype != MOE_BF16 || c.w_dtype != MOE_BF16) return -1;
  const long long avg32 = (long long)T * c.topk;
  return (avg32 <= 32LL * c.n_experts) ? 0x7fffffff : 64;
}

// bf16 layers use the LDS-pipelined tiled GEMM (kTileM rows), E4M3 weights its
// block-scaled fp8 form (kTileM8 rows), the float32 layer the 64x64 tiled GEMM.
bool use_big_tiles(const moe_cfg& c) { return c.act_dtype == MOE_BF16 && c.w_dtype == MOE_BF16; }

int tile_rows(const moe_cfg& c) {
  if (c.w_dtype == MOE_E4M3) return moe::kTileM8;
  return use_big_tiles(c) ? moe::kTileM : moe::gemm_tile_m();
}

int run_route(const moe_cfg& c, int T, const void* x, const float* wr, const float* bias,
              const RoutePtrs& r, void* ws, const Layout& L, hipStream_t st) {
  const int E = c.n_experts, K = c.topk, H = c.hidden;
  float* P = at<float>(ws, L.P);
  MOE_TRY(timed(K_ROUTER, st, [&] {
    return moe::launch_router(x, c.act_dtype == MOE_BF16, wr, at<bf16_t>(ws, L.wt3), P, T, H, E,
                              st);
  }));
  MOE_TRY(timed(K_SELECT, st, [&] {
    return moe::launch_select(P, moe::router_partials(T, H, E, c.act_dtype == MOE_BF16), bias, T,
                              E, c.n_groups, c.topk_groups, K,
                              c.group_topn, r.idx, r.gate, r.gap, st);
  }));
  MOE_TRY(timed(K_PERMUTE, st, [&] {
    return moe::launch_permute(r.idx, T, K, E, c.n_shared, at<uint64_t>(ws, L.masks),
                               at<int32_t>(ws, L.hist), at<int32_t>(ws, L.base), r.counts,
                               r.offsets, r.perm, r.slot, stream_max_rows(c, T),
                               at<int32_t>(ws, L.chunk_start), tile_rows(c),
                               at<int32_t>(ws, L.mt_start), st);
  }));
  return MOE_OK;
}

RoutePtrs route_ptrs(const moe_routing* out, void* ws, const Layout& L) {
  RoutePtrs r;
  if (out != nullptr) {
    r = RoutePtrs{out->topk_idx, out->counts, out->offsets, out->perm, out->slot, out->topk_gate,
                  out->tie_gap};
  } else {
    r = RoutePtrs{at<int32_t>(ws, L.idx), at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                  at<int32_t>(ws, L.perm), at<int32_t>(ws, L.slot), at<float>(ws, L.gate),
                  at<float>(ws, L.gap)};
  }
  return r;
}

int check_routing(const moe_routing* out) {
  if (out == nullptr) return MOE_ERR_NULL;
  if (!out->topk_idx || !out->topk_gate || !out->counts || !out->offsets || !out->perm || !out->slot)
    return MOE_ERR_NULL;
  return MOE_OK;
}

std::atomic<int> g_cu_count[64];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename TE>
int run_experts(const moe_cfg& c, int T, const TE* x, const moe_experts* w, const TE* residual,
                TE* y, const RoutePtrs& r, void* ws, const Layout& L, hipStream_t st) {
  const int E = c.n_experts, K = c.topk, S = c.n_shared, H = c.hidden, I = c.inter;
  const int TK = T * K;
  const int bm = tile_rows(c);
  const int max_mt = (TK + bm - 1) / bm + E + S * ((T + bm - 1) / bm);
  TE* hst = at<TE>(ws, L.hst);
  TE* yst = at<TE>(ws, L.yst);
  const int32_t* chunk_start = at<int32_t>(ws, L.chunk_start);
  const int32_t* mt_start = at<int32_t>(ws, L.mt_start);
  const int smax = stream_max_rows(c, T);
  const bool streams = smax >= 0;
  const bool tiles = smax < T;  // an expert (or the shared one) can have up to T rows
  // persistent grid of the streaming GEMM: one workgroup per CU, fewer when
  // the largest task count the routing can produce is smaller
  auto stream_blocks = [&](int n_slices, int mode) {
    const long long chunks = (TK + moe::kStreamChunk - 1) / moe::kStreamChunk + E +
                           (long long)S * ((T + moe::kStreamChunk - 1) / moe::kStreamChunk);
    const long long waves = chunks * n_slices;
    const int wpb = moe::stream_waves_per_block(mode);
    return int(std::max<long long>(1, std::min<long long>((waves + wpb - 1) / wpb, (long long)cu_count())));
  };
  moe::GemmArgs<TE> g1{x, static_cast<const TE*>(w->w_gate), static_cast<const TE*>(w->w_up), hst,
                       r.perm, r.counts, r.offsets, mt_start, E, E + S, T, TK, I, H};
  MOE_TRY(timed(K_GATEUP, st, [&] {
    if (streams) {
      moe::StreamArgs sa{reinterpret_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(w->w_gate), static_cast<const bf16_t*>(w->w_up),
                         reinterpret_cast<bf16_t*>(hst), r.perm, r.counts, r.offsets, chunk_start,
                         E, E + S, T, TK, I, H};
      hipError_t err = moe::launch_stream_gemm(sa, 1, stream_blocks(I / 64, 1), st);
      if (err != hipSuccess || !tiles) return err;
    }
    if constexpr (std::is_same<TE, bf16_t>::value) {
      moe::TileArgs ta{reinterpret_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w->w_gate),
                       static_cast<const bf16_t*>(w->w_up), reinterpret_cast<bf16_t*>(hst), r.perm,
                       r.counts, r.offsets, mt_start, E, E + S, T, TK, I, H};
      return moe::launch_tile_gemm(ta, 1, max_mt, st);
    } else {
      return moe::launch_gemm<TE>(g1, true, max_mt, 4 * cu_count(), st);
    }
  }));
  moe::GemmArgs<TE> g2{hst, static_cast<const TE*>(w->w_down), nullptr, yst, r.perm, r.counts,
                       r.offsets, mt_start, E, E + S, T, TK, H, I};
  MOE_TRY(timed(K_DOWN, st, [&] {
    if (streams) {
      moe::StreamArgs sa{reinterpret_cast<const bf16_t*>(hst),
                         static_cast<const bf16_t*>(w->w_down), nullptr,
                         reinterpret_cast<bf16_t*>(yst), r.perm, r.counts, r.offsets, chunk_start,
                         E, E + S, T, TK, H, I};
      hipError_t err = moe::launch_stream_gemm(sa, 0, stream_blocks(H / 128, 0), st);
      if (err != hipSuccess || !tiles) return err;
    }
    if constexpr (std::is_same<TE, bf16_t>::value) {
      moe::TileArgs ta{reinterpret_cast<const bf16_t*>(hst), static_cast<const bf16_t*>(w->w_down),
                       nullptr, reinterpret_cast<bf16_t*>(yst), r.perm, r.counts, r.offsets,
                       mt_start, E, E + S, T, TK, H, I};
      return moe::launch_tile_gemm(ta, 0, max_mt, st);
    } else {
      return moe::launch_gemm<TE>(g2, false, max_mt, 4 * cu_count(), st);
    }
  }));
  MOE_TRY(timed(K_COMBINE, st, [&] {
    return moe::launch_combine<TE>(yst, r.slot, r.gate, residual, y, T, K, H, TK, S, st);
  }));
  return MOE_OK;
}

// E4M3 weights: quantise x per 1x128 slice, block-scaled gate/up GEMM with
// the SwiGLU output quantised in its epilogue, block-scaled down GEMM, combine.
int run_experts_fp8(const moe_cfg& c, int T, const bf16_t* x, const moe_experts* w,
                    const bf16_t* residual, bf16_t* y, const RoutePtrs& r, void* ws,
                    const Layout& L, hipStream_t st) {
  const int E = c.n_experts, K = c.topk, S = c.n_shared, H = c.hidden, I = c.inter;
  const int TK = T * K;
  const int bm = moe::kTileM8;
  const int max_mt = (TK + bm - 1) / bm + E + S * ((T + bm - 1) / bm);
  uint8_t* xq = at<uint8_t>(ws, L.xq);
  float* xs = at<float>(ws, L.xs);
  uint8_t* hq = at<uint8_t>(ws, L.hst);
  float* hs = at<float>(ws, L.hs);
  bf16_t* yst = at<bf16_t>(ws, L.yst);
  const int32_t* mt_start = at<int32_t>(ws, L.mt_start);
  MOE_TRY(timed(K_QUANT, st, [&] { return moe::launch_quant_1x128(x, T, H, xq, xs, st); }));
  MOE_TRY(timed(K_GATEUP, st, [&] {
    moe::TileArgs8 ta{xq, xs, static_cast<const uint8_t*>(w->w_gate),
                      static_cast<const uint8_t*>(w->w_up), w->s_gate, w->s_up, hq, nullptr, hs,
                      r.perm, r.counts, r.offsets, mt_start, E, E + S, T, TK, I, H};
    return moe::launch_tile_gemm_fp8(ta, true, max_mt, st);
  }));
  MOE_TRY(timed(K_DOWN, st, [&] {
    moe::TileArgs8 ta{hq, hs, static_cast<const uint8_t*>(w->w_down), nullptr, w->s_down, nullptr,
                      nullptr, yst, nullptr, r.perm, r.counts, r.offsets, mt_start, E, E + S, T, TK,
                      H, I};
    return moe::launch_tile_gemm_fp8(ta, false, max_mt, st);
  }));
  MOE_TRY(timed(K_COMBINE, st, [&] {
    return moe::launch_combine<bf16_t>(yst, r.slot, r.gate, residual, y, T, K, H, TK, S, st);
  }));
  return MOE_OK;
}

// ---------------------------------------------------------------- backward

// Workspace of the backward: the forward's layout (routing, H and Y staging),
// then the backward's staged rows and per-assignment buffers.
struct BwdLayout {
  Layout f;
  size_t xst, gst, ust, dyst, dgst, dust, dxst, dg, dgp, dl, dlst, wrt, dwrt, mt, mtd, total;
  // E4M3 weights
  size_t f32a, f32b, gq, gs, uq, us, dyq, dys, rowgate, dg32, du32, dgq, dgs, duq, dus;
  size_t kp, dyT, dysT, xT, xsT, hT, hsT, dgT, dgsT, duT, dusT;
};

BwdLayout make_bwd_layout(const moe_cfg& c, int64_t T) {
  BwdLayout B{};
  B.f = make_layout(c, T);
  size_t off = B.f.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t E = c.n_experts, K = c.topk, S = c.n_shared, H = c.hidden, I = c.inter;
  const size_t TK = size_t(T) * K, rows = TK + S * size_t(T);
  if (c.w_dtype == MOE_E4M3) {
    const size_t n = E + S, HB = H / 128, IB = I / 128;
    // 128x1 operands: each expert's rows rounded up to 128
    const size_t rcap = 128 * size_t(moe::f8_max_row_tiles(int(T), int(K), int(E), int(S)));
    B.f32a = take(rows * I * 4);
    B.f32b = take(rows * I * 4);
    B.gq = take(rows * I);
    B.gs = take(rows * IB * 4);
    B.uq = take(rows * I);
    B.us = take(rows * IB * 4);
    B.dyq = take(rows * H);
    B.dys = take(rows * HB * 4);
    B.rowgate = take(TK * 4);
    B.dg32 = take(rows * I * 4);
    B.du32 = take(rows * I * 4);
    B.dgq = take(rows * I);
    B.dgs = take(rows * IB * 4);
    B.duq = take(rows * I);
    B.dus = take(rows * IB * 4);
    B.dxst = take(rows * H * 2);
    B.kp = take((n + 1) * 4);
    B.dyT = take(rcap * H);
    B.dysT = take(rcap / 128 * H * 4);
    B.xT = take(rcap * H);
    B.xsT = take(rcap / 128 * H * 4);
    B.hT = take(rcap * I);
    B.hsT = take(rcap / 128 * I * 4);
    B.dgT = take(rcap * I);
    B.dgsT = take(rcap / 128 * I * 4);
    B.duT = take(rcap * I);
    B.dusT = take(rcap / 128 * I * 4);
    B.dg = take(TK * 4);
    B.dl = take(TK * 4);
    B.dlst = take(TK * 4);
    B.wrt = take(E * H * 4);
    B.dwrt = take(E * H * 4);
    B.mt = take((n + 1) * 4);
    B.total = off;
    return B;
  }
  B.xst = take(rows * H * 2);
  B.gst = take(rows * I * 2);
  B.ust = take(rows * I * 2);
  B.dyst = take(rows * H * 2);
  B.dgst = take(rows * I * 2);
  B.dust = take(rows * I * 2);
  B.dxst = take(rows * H * 2);
  B.dg = take(TK * 4);
  B.dgp = take((I / 256) * rows * 4);
  B.dl = take(TK * 4);
  B.dlst = take(TK * 4);
  B.wrt = take(E * H * 4);
  B.dwrt = take(E * H * 4);
  B.mt = take((E + S + 1) * 4);
  B.mtd = take((E + S + 1) * 4);
  B.total = off;
  return B;
}

// The backward stages its rows with 32-bit byte offsets: every staged-row
// buffer must span less than 4 GiB.
int validate_bwd(const moe_cfg* c, int64_t T) {
  if (c->act_dtype != MOE_BF16 || (c->w_dtype != MOE_BF16 && c->w_dtype != MOE_E4M3))
    return MOE_ERR_DTYPE;
  // E4M3: a tile holds the weight-block scales of up to 128 K blocks
  if (c->w_dtype == MOE_E4M3 && (c->hidden > 128 * 128 || c->inter > 128 * 128)) return MOE_ERR_SHAPE;
  if (c->hidden % 256 != 0 || c->inter % 256 != 0) return MOE_ERR_SHAPE;  // wgrad tiles of 256
  const int64_t rows = T * int64_t(c->topk + c->n_shared);
  if (rows * std::max<int64_t>(c->hidden, c->inter) * 2 >= (int64_t(1) << 32) - 256) return MOE_ERR_SHAPE;
  if (int64_t(c->hidden) * c->inter * 2 >= (int64_t(1) << 32)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// the forward's gate/up GEMM for the backward's recompute: x rows gathered through
// the permutation, H = SiLU(G) * U staged as in the forward, G and U kept as well
int run_gate_up_keep(const moe_cfg& c, int T, const bf16_t* x, const bf16_t* wg, const bf16_t* wu,
                     bf16_t* h, bf16_t* gst, bf16_t* ust, const RoutePtrs& r, void* ws,
                     const Layout& L, hipStream_t st) {
  const int E = c.n_experts, K = c.topk, S = c.n_shared, H = c.hidden, I = c.inter;
  const int TK = T * K;
  const int bm = tile_rows(c);
  const int max_mt = (TK + bm - 1) / bm + E + S * ((T + bm - 1) / bm);
  const int smax = stream_max_rows(c, T);
  const bool streams = smax >= 0, tiles = smax < T;
  if (streams) {
    const long long chunks = (TK + moe::kStreamChunk - 1) / moe::kStreamChunk + E +
                           (long long)S * ((T + moe::kStreamChunk - 1) / moe::kStreamChunk);
    const long long waves = chunks * (I / 64);
    const int wpb = moe::stream_waves_per_block(2);
    const int blocks =
        int(std::max<long long>(1, std::min<long long>((waves + wpb - 1) / wpb, (long long)cu_count())));
    moe::StreamArgs sa{x, wg, wu, h, r.perm, r.counts, r.offsets, at<int32_t>(ws, L.chunk_start),
                       E, E + S, T, TK, I, H, gst, ust};
    hipError_t err = moe::launch_stream_gemm(sa, 2, blocks, st);
    if (err != hipSuccess) return MOE_ERR_HIP;
    if (!tiles) return MOE_OK;
  }
  moe::TileArgs ta{x, wg, wu, h, r.perm, r.counts, r.offsets, at<int32_t>(ws, L.mt_start),
                   E, E + S, T, TK, I, H, gst, ust};
  return moe::launch_tile_gemm(ta, 2, max_mt, st) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int run_backward_fp8(const moe_cfg& c, int T, const bf16_t* x, const float* wr,
                     const moe_experts* w, const bf16_t* dy, bf16_t* dx, float* dwr, float* dwg,
                     float* dwu, float* dwd, void* ws, const BwdLayout& B, const RoutePtrs& r,
                     hipStream_t st);

int run_backward(const moe_cfg& c, int T, const bf16_t* x, const float* wr, const float* bias,
                 const moe_experts* w, const bf16_t* dy, bf16_t* dx, float* dwr, float* dwg,
                 float* dwu, float* dwd, void* ws, const BwdLayout& B, hipStream_t st) {
  const int E = c.n_experts, K = c.topk, S = c.n_shared, H = c.hidden, I = c.inter;
  const Layout& L = B.f;
  const RoutePtrs r = route_ptrs(nullptr, ws, L);
  int rc = run_route(c, T, x, wr, bias, r, ws, L, st);
  if (rc != MOE_OK) return rc;
  if (c.w_dtype == MOE_E4M3)
    return run_backward_fp8(c, T, x, wr, w, dy, dx, dwr, dwg, dwu, dwd, ws, B, r, st);
  moe::BwdArgs g{};
  g.x = x;
  g.perm = r.perm;
  g.counts = r.counts;
  g.offsets = r.offsets;
  g.mt = at<int32_t>(ws, B.mt);
  // 320-row data-gradient tiles from 32 routed rows per expert on average
  // (prefill: 4.29 + 7.07 -> 3.72 + 5.48 ms); 128-row tiles below (decode)
  g.mtd = int64_t(T) * K >= int64_t(32) * E ? at<int32_t>(ws, B.mtd) : nullptr;
  g.w_gate = static_cast<const bf16_t*>(w->w_gate);
  g.w_up = static_cast<const bf16_t*>(w->w_up);
  g.w_down = static_cast<const bf16_t*>(w->w_down);
  g.xst = at<bf16_t>(ws, B.xst);
  g.gst = at<bf16_t>(ws, B.gst);
  g.ust = at<bf16_t>(ws, B.ust);
  g.hst = at<bf16_t>(ws, L.hst);
  g.yst = at<bf16_t>(ws, L.yst);
  g.dyst = at<bf16_t>(ws, B.dyst);
  g.dgst = at<bf16_t>(ws, B.dgst);
  g.dust = at<bf16_t>(ws, B.dust);
  g.dxst = at<bf16_t>(ws, B.dxst);
  g.dg = at<float>(ws, B.dg);
  g.dgp = at<float>(ws, B.dgp);  // gate gradients from dH and H: Y is not recomputed
  g.dl = at<float>(ws, B.dl);
  g.dlst = at<float>(ws, B.dlst);
  g.wrt = at<float>(ws, B.wrt);
  g.dwrt = at<float>(ws, B.dwrt);
  g.dw_gate = dwg;
  g.dw_up = dwu;
  g.dw_down = dwd;
  g.E = E;
  g.n_exp = E + S;
  g.T = T;
  g.TK = T * K;
  g.K = K;
  g.H = H;
  g.I = I;
  g.wg_xcd = int64_t(T) * K <= int64_t(64) * E;  // decode-sized: at most 64 rows per expert
  const float* P = at<float>(ws, L.P);
  const int ks = moe::router_partials(T, H, E, true);
  auto stage = [&](int s) {
    return moe::launch_backward_kernels(g, P, ks, r.idx, r.slot, r.gate, wr, dy, dx, dwr, st, s);
  };
  // recompute the forward's expert intermediates from x (G, U and H in one gated
  // GEMM; Y is not needed: the gate gradients <dy, Y_k> = <dH_k, H_k> / g_k come
  // out of the dH GEMM); X rows staged for the weight gradients
  MOE_TRY(timed(K_BWD_RECOMPUTE, st, [&]() -> hipError_t {
    hipError_t err = stage(0);
    if (err != hipSuccess) return err;
    return run_gate_up_keep(c, T, x, g.w_gate, g.w_up, g.hst, g.gst, g.ust, r, ws, L, st) == MOE_OK
               ? hipSuccess
               : hipErrorLaunchFailure;
  }));
  MOE_TRY(timed(K_BWD_COMBINE, st, [&] { return stage(2); }));  // g dy, tile prefixes
  MOE_TRY(timed(K_BWD_DH, st, [&] { return stage(4); }));       // dH, dG, dU, gate-gradient sums
  MOE_TRY(timed(K_BWD_DX, st, [&] { return stage(5); }));
  MOE_TRY(timed(K_BWD_WGRAD, st, [&] { return stage(6); }));
  MOE_TRY(timed(K_BWD_ROUTER, st, [&]() -> hipError_t {
    hipError_t err = stage(3);
    if (err != hipSuccess) return err;
    if ((err = stage(7)) != hipSuccess) return err;
    return stage(8);
  }));
  return MOE_OK;
}

// E4M3 weights: every expert GEMM of the backward in E4M3 (bwd_fp8_kernels.hip);
// routing, gate gradients, dW_r and dx as on the bf16 path.
int run_backward_fp8(const moe_cfg& c, int T, const bf16_t* x, const float* wr,
                     const moe_experts* w, const bf16_t* dy, bf16_t* dx, float* dwr, float* dwg,
                     float* dwu, float* dwd, void* ws, const BwdLayout& B, const RoutePtrs& r,
                     hipStream_t st) {
  const int E = c.n_experts, K = c.topk, S = c.n_shared, H = c.hidden, I = c.inter;
  const Layout& L = B.f;
  moe::BwdArgs8 q{};
  q.x = x;
  q.dy = dy;
  q.perm = r.perm;
  q.counts = r.counts;
  q.offsets = r.offsets;
  q.slot = r.slot;
  q.gate = r.gate;
  q.xq = at<uint8_t>(ws, L.xq);
  q.xs = at<float>(ws, L.xs);
  q.w_gate = static_cast<const uint8_t*>(w->w_gate);
  q.w_up = static_cast<const uint8_t*>(w->w_up);
  q.w_down = static_cast<const uint8_t*>(w->w_down);
  q.s_gate = w->s_gate;
  q.s_up = w->s_up;
  q.s_down = w->s_down;
  q.f32a = at<float>(ws, B.f32a);
  q.f32b = at<float>(ws, B.f32b);
  q.gq = at<uint8_t>(ws, B.gq);
  q.gs = at<float>(ws, B.gs);
  q.uq = at<uint8_t>(ws, B.uq);
  q.us = at<float>(ws, B.us);
  q.hq = at<uint8_t>(ws, L.hst);
  q.hs = at<float>(ws, L.hs);
  q.yst = at<bf16_t>(ws, L.yst);
  q.dyq = at<uint8_t>(ws, B.dyq);
  q.dys = at<float>(ws, B.dys);
  q.rowgate = at<float>(ws, B.rowgate);
  q.dg32 = at<float>(ws, B.dg32);
  q.du32 = at<float>(ws, B.du32);
  q.dgq = at<uint8_t>(ws, B.dgq);
  q.dgs = at<float>(ws, B.dgs);
  q.duq = at<uint8_t>(ws, B.duq);
  q.dus = at<float>(ws, B.dus);
  q.dxst = at<bf16_t>(ws, B.dxst);
  q.mt = at<int32_t>(ws, B.mt);
  q.kp = at<int32_t>(ws, B.kp);
  q.dyT = at<uint8_t>(ws, B.dyT);
  q.dysT = at<float>(ws, B.dysT);
  q.xT = at<uint8_t>(ws, B.xT);
  q.xsT = at<float>(ws, B.xsT);
  q.hT = at<uint8_t>(ws, B.hT);
  q.hsT = at<float>(ws, B.hsT);
  q.dgT = at<uint8_t>(ws, B.dgT);
  q.dgsT = at<float>(ws, B.dgsT);
  q.duT = at<uint8_t>(ws, B.duT);
  q.dusT = at<float>(ws, B.dusT);
  q.dw_gate = dwg;
  q.dw_up = dwu;
  q.dw_down = dwd;
  q.E = E;
  q.n_exp = E + S;
  q.T = T;
  q.TK = T * K;
  q.K = K;
  q.H = H;
  q.I = I;
  // the bf16 row kernels shared with the bf16 path
  moe::BwdArgs g{};
  g.x = x;
  g.perm = r.perm;
  g.counts = r.counts;
  g.offsets = r.offsets;
  g.mt = at<int32_t>(ws, B.mt);
  g.yst = at<bf16_t>(ws, L.yst);
  g.dyst = nullptr;  // the output gradients are quantised from float32 instead
  g.dxst = q.dxst;
  g.dg = at<float>(ws, B.dg);
  g.dl = at<float>(ws, B.dl);
  g.dlst = at<float>(ws, B.dlst);
  g.wrt = at<float>(ws, B.wrt);
  g.dwrt = at<float>(ws, B.dwrt);
  g.E = E;
  g.n_exp = E + S;
  g.T = T;
  g.TK = T * K;
  g.K = K;
  g.H = H;
  g.I = I;
  const float* P = at<float>(ws, L.P);
  const int ks = moe::router_partials(T, H, E, true);
  auto stage = [&](int s) {
    return moe::launch_backward_kernels(g, P, ks, r.idx, r.slot, r.gate, wr, dy, dx, dwr, st, s);
  };
  auto stage8 = [&](int s) { return moe::launch_backward_fp8(q, st, s); };
  // recompute: Q(x), G and U cached in E4M3, H, Y
  MOE_TRY(timed(K_BWD_RECOMPUTE, st, [&]() -> hipError_t {
    hipError_t err;
    if ((err = stage8(1)) != hipSuccess) return err;
    if ((err = moe::launch_quant_1x128(x, T, H, at<uint8_t>(ws, L.xq), at<float>(ws, L.xs), st)) !=
        hipSuccess)
      return err;
    return stage8(2);
  }));
  MOE_TRY(timed(K_BWD_COMBINE, st, [&]() -> hipError_t {
    hipError_t err;
    if ((err = stage(2)) != hipSuccess) return err;  // gate gradients
    if ((err = stage(3)) != hipSuccess) return err;  // router backward
    return stage8(3);                                // Q(dY)
  }));
  MOE_TRY(timed(K_BWD_DH, st, [&] { return stage8(4); }));
  MOE_TRY(timed(K_BWD_DX, st, [&] { return stage8(5); }));
  MOE_TRY(timed(K_BWD_RETILE, st, [&] { return stage8(6); }));
  MOE_TRY(timed(K_BWD_WGRAD, st, [&] { return stage8(7); }));
  MOE_TRY(timed(K_BWD_ROUTER, st, [&]() -> hipError_t {
    hipError_t err = stage(7);
    return err != hipSuccess ? err : stage(8);
  }));
  return MOE_OK;
}

// ---------------------------------------------------------------- static scratch

// Device scratch of moe_forward_noalloc: a file-scope array that every GPU the
// library runs on holds once, from code-object load until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol): it passes the device address that
// hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[64];

// this device's address of the scratch array (looked up on its first use)
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // concurrent first calls look up the same address; any of them may store it
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return 100; }

int moe_profile_enable(int on) {
  g_prof.on = on != 0;
  return MOE_OK;
}

int moe_profile_read(double* total_ms, int32_t* launches, int n_slots) {
  for (auto& r : g_prof.recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return MOE_ERR_HIP;
    g_prof.ms[r.slot] += ms;
    g_prof.n[r.slot] += 1;
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  for (int i = 0; i < K_NSLOTS && i < n_slots; ++i) {
    if (total_ms) total_ms[i] = g_prof.ms[i];
    if (launches) launches[i] = g_prof.n[i];
  }
  if (total_ms != nullptr || launches != nullptr) {
    for (int i = 0; i < K_NSLOTS; ++i) {
      g_prof.ms[i] = 0.0;
      g_prof.n[i] = 0;
    }
  }
  return K_NSLOTS;
}

const char* moe_profile_kernel_name(int slot) {
  return (slot >= 0 && slot < K_NSLOTS) ? kSlotNames[slot] : "unknown";
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case MOE_ERR_DTYPE: return "unsupported dtype combination";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case MOE_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case MOE_ERR_TOO_LARGE:
      return "batch needs more scratch than moe_forward_noalloc's static buffer holds";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_cfg* cfg, int64_t T) {
  if (validate_cfg(cfg) != MOE_OK || validate_T(cfg, T) != MOE_OK) return 0;
  return make_layout(*cfg, T).total;
}

int moe_route(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
              const float* bias, const moe_routing* out, void* ws, size_t ws_bytes,
              void* stream) {
  int rc = validate_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if ((rc = validate_T(cfg, T)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if ((rc = check_routing(out)) != MOE_OK) return rc;
  if (x == nullptr || w_router == nullptr || bias == nullptr) return MOE_ERR_NULL;
  const Layout L = make_layout(*cfg, T);
  if (ws == nullptr || ws_bytes < L.route_total) return MOE_ERR_WORKSPACE;
  if ((rc = check_device()) != MOE_OK) return rc;
  return run_route(*cfg, int(T), x, w_router, bias, route_ptrs(out, ws, L), ws, L,
                   static_cast<hipStream_t>(stream));
}

int moe_forward(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
                const float* bias, const moe_experts* w, const void* residual, void* y,
                const moe_routing* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if ((rc = validate_T(cfg, T)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (out != nullptr && (rc = check_routing(out)) != MOE_OK) return rc;
  if (x == nullptr || w_router == nullptr || bias == nullptr || w == nullptr || y == nullptr)
    return MOE_ERR_NULL;
  if (w->w_gate == nullptr || w->w_up == nullptr || w->w_down == nullptr) return MOE_ERR_NULL;
  if (cfg->w_dtype == MOE_E4M3 && (w->s_gate == nullptr || w->s_up == nullptr || w->s_down == nullptr))
    return MOE_ERR_NULL;
  const Layout L = make_layout(*cfg, T);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if ((rc = check_device()) != MOE_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const RoutePtrs r = route_ptrs(out, ws, L);
  rc = run_route(*cfg, int(T), x, w_router, bias, r, ws, L, st);
  if (rc != MOE_OK) return rc;
  if (cfg->w_dtype == MOE_E4M3)
    return run_experts_fp8(*cfg, int(T), static_cast<const bf16_t*>(x), w,
                           static_cast<const bf16_t*>(residual), static_cast<bf16_t*>(y), r, ws, L,
                           st);
  if (cfg->act_dtype == MOE_BF16)
    return run_experts<bf16_t>(*cfg, int(T), static_cast<const bf16_t*>(x), w,
                               static_cast<const bf16_t*>(residual), static_cast<bf16_t*>(y), r,
                               ws, L, st);
  return run_experts<float>(*cfg, int(T), static_cast<const float*>(x), w,
                            static_cast<const float*>(residual), static_cast<float*>(y), r, ws, L,
                            st);
}

int moe_forward_noalloc(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
                        const float* bias, const moe_experts* w, const void* residual, void* y,
                        const moe_routing* out, void* stream) {
  int rc = validate_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if ((rc = validate_T(cfg, T)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (make_layout(*cfg, T).total > kScratchBytes) return MOE_ERR_TOO_LARGE;
  if ((rc = check_device()) != MOE_OK) return rc;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws)) != MOE_OK) return rc;
  // no timing events for this entry point: creating them would allocate
  const bool prof = g_prof.on;
  g_prof.on = false;
  rc = moe_forward(cfg, T, x, w_router, bias, w, residual, y, out, ws, kScratchBytes, stream);
  g_prof.on = prof;
  return rc;
}

size_t moe_backward_workspace_bytes(const moe_cfg* cfg, int64_t T) {
  if (validate_cfg(cfg) != MOE_OK || validate_T(cfg, T) != MOE_OK || validate_bwd(cfg, T) != MOE_OK)
    return 0;
  return make_bwd_layout(*cfg, T).total;
}

int moe_backward(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
                 const float* bias, const moe_experts* w, const void* dy, void* dx,
                 float* dw_router, float* dw_gate, float* dw_up, float* dw_down, void* ws,
                 size_t ws_bytes, void* stream) {
  int rc = validate_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if ((rc = validate_T(cfg, T)) != MOE_OK) return rc;
  if ((rc = validate_bwd(cfg, T)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || bias == nullptr || w == nullptr || dy == nullptr ||
      dx == nullptr || dw_router == nullptr || dw_gate == nullptr || dw_up == nullptr ||
      dw_down == nullptr)
    return MOE_ERR_NULL;
  if (w->w_gate == nullptr || w->w_up == nullptr || w->w_down == nullptr) return MOE_ERR_NULL;
  if (cfg->w_dtype == MOE_E4M3 && (w->s_gate == nullptr || w->s_up == nullptr || w->s_down == nullptr))
    return MOE_ERR_NULL;
  const BwdLayout B = make_bwd_layout(*cfg, T);
  if (ws == nullptr || ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  if ((rc = check_device()) != MOE_OK) return rc;
  return run_backward(*cfg, int(T), static_cast<const bf16_t*>(x), w_router, bias, w,
                      static_cast<const bf16_t*>(dy), static_cast<bf16_t*>(dx), dw_router, dw_gate,
                      dw_up, dw_down, ws, B, static_cast<hipStream_t>(stream));
}

int moe_quantize_1x128(const void* x, int64_t rows, int32_t cols, uint8_t* q, float* scales,
                       void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128 != 0) return MOE_ERR_SHAPE;
  if (rows * int64_t(cols) >= (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (x == nullptr || q == nullptr || scales == nullptr) return MOE_ERR_NULL;
  int rc = check_device();
  if (rc != MOE_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_TRY(timed(K_QUANT, st, [&] {
    return moe::launch_quant_1x128(static_cast<const bf16_t*>(x), rows, cols, q, scales, st);
  }));
  return MOE_OK;
}

int moe_balance_loss(const moe_cfg* cfg, int64_t T, int32_t seq_len, const void* x,
                     const float* w_router, float alpha, float* loss, float* f, float* p, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc = validate_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if ((rc = validate_T(cfg, T)) != MOE_OK) return rc;
  if (seq_len <= 0 || T % seq_len != 0) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || loss == nullptr) return MOE_ERR_NULL;
  const Layout L = make_layout(*cfg, T);
  if (ws == nullptr || ws_bytes < L.bal_end) return MOE_ERR_WORKSPACE;
  if ((rc = check_device()) != MOE_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = cfg->hidden, E = cfg->n_experts, Ti = int(T);
  const bool xb = cfg->act_dtype == MOE_BF16;
  float* P = at<float>(ws, L.P);
  MOE_TRY(timed(K_ROUTER, st, [&] {
    return moe::launch_router(x, xb, w_router, at<bf16_t>(ws, L.wt3), P, Ti, H, E, st);
  }));
  MOE_TRY(timed(K_BAL, st, [&] {
    return moe::launch_balance(P, moe::router_partials(Ti, H, E, xb), Ti, E, cfg->topk, seq_len,
                               alpha, at<float>(ws, L.bal_sn), at<int32_t>(ws, L.bal_ids),
                               at<double>(ws, L.bal_psum), at<int32_t>(ws, L.bal_pcnt), loss, f,
                               p, st);
  }));
  return MOE_OK;
}

int moe_bias_update(const moe_cfg* cfg, int64_t T, const int32_t* counts, float* bias,
                    float gamma, void* stream) {
  int rc = validate_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if ((rc = validate_T(cfg, T)) != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (counts == nullptr || bias == nullptr) return MOE_ERR_NULL;
  if ((rc = check_device()) != MOE_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_TRY(timed(K_BIAS, st, [&] {
    return moe::launch_bias_update(counts, bias, cfg->n_experts, (long long)T * cfg->topk, gamma,
                                   st);
  }));
  return MOE_OK;
}

}  // extern "C"
