// Complementary sequence-wise balance loss of the router.
//
// Method: "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token", §1.4 (Eq 17-20):
// for each sequence, f_i = E / (K * seq_len) * (number of its tokens whose
// top-K of the raw affinities s (no bias) holds expert i), P_i = mean over
// the sequence of s_i / sum_j s_j, loss = alpha * sum_i f_i P_i.  The top-K is
// a plain top-K over all experts, ties to the lower index.
//
// Deterministic: counts are integer (LDS atomics), P partial sums are float64
// added in token order within fixed token chunks, chunks and experts are then
// added in a fixed order.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int BAL_WAVES = 4;
constexpr int BAL_MAX_E = 512;
}  // namespace

// one wave per token: s from the router partials, s / sum(s), plain top-K ids
__global__ __launch_bounds__(64 * BAL_WAVES) void balance_token_kernel(
    const float* __restrict__ P, int ksplit, int T, int E, int K, float* __restrict__ sn,
    int32_t* __restrict__ ids) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * BAL_WAVES + wave;
  if (t >= T) return;  // whole wave; no barrier in this kernel
  const int epl = (E + 63) / 64;
  float sv[BAL_MAX_E / 64];
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < BAL_MAX_E / 64; ++j) {
    const int e = lane * epl + j;
    float v = -INFINITY;
    if (j < epl && e < E) {
      float L = 0.f;
      for (int k = 0; k < ksplit; ++k) L += P[((size_t)k * T + t) * E + e];
      v = sigmoidf(L);
      part += v;
    }
    sv[j] = v;
  }
  const float tot = wave_sum(part);
#pragma unroll
  for (int j = 0; j < BAL_MAX_E / 64; ++j) {
    const int e = lane * epl + j;
    if (j < epl && e < E) sn[(size_t)t * E + e] = sv[j] / tot;
  }
  for (int r = 0; r < K; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < BAL_MAX_E / 64; ++j)
      if (sv[j] > bv) {  // ascending ids within a lane: strict '>' keeps the lower id
        bv = sv[j];
        bi = lane * epl + j;
      }
    wave_argmax(bv, bi);
    if (lane == 0) ids[(size_t)t * K + r] = bi;
#pragma unroll
    for (int j = 0; j < BAL_MAX_E / 64; ++j)
      if (lane * epl + j == bi) sv[j] = -INFINITY;
  }
}

// block (sequence q, chunk c): counts and float64 sums of s / sum(s) over the
// chunk's tokens, in token order, for every expert
__global__ __launch_bounds__(256) void balance_chunk_kernel(const float* __restrict__ sn,
                                                            const int32_t* __restrict__ ids,
                                                            int E, int K, int seq_len, int nch,
                                                            double* __restrict__ psum,
                                                            int32_t* __restrict__ pcnt) {
  __shared__ int cnt_s[BAL_MAX_E];
  const int q = blockIdx.x, c = blockIdx.y;
  const int per = (seq_len + nch - 1) / nch;
  const int t0 = q * seq_len + c * per;
  const int t1 = q * seq_len + min(seq_len, (c + 1) * per);
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt_s[e] = 0;
  __syncthreads();
  for (int a = t0 * K + threadIdx.x; a < t1 * K; a += blockDim.x) atomicAdd(&cnt_s[ids[a]], 1);
  __syncthreads();
  const size_t o = ((size_t)q * nch + c) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double acc = 0.0;
    int t = t0;
    for (; t + 8 <= t1; t += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = sn[(size_t)(t + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += (double)v[u];
    }
    for (; t < t1; ++t) acc += (double)sn[(size_t)t * E + e];
    psum[o + e] = acc;
    pcnt[o + e] = cnt_s[e];
  }
}

// one block per sequence: chunks in order, then experts in order
__global__ __launch_bounds__(256) void balance_final_kernel(const double* __restrict__ psum,
                                                            const int32_t* __restrict__ pcnt,
                                                            int E, int K, int seq_len, int nch,
                                                            float alpha, float* __restrict__ loss,
                                                            float* __restrict__ f_out,
                                                            float* __restrict__ p_out) {
  __shared__ double term_s[BAL_MAX_E];
  const int q = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double ps = 0.0;
    long long cn = 0;
    for (int c = 0; c < nch; ++c) {
      const size_t o = ((size_t)q * nch + c) * E + e;
      ps += psum[o];
      cn += pcnt[o];
    }
    const double f = (double)cn * E / ((double)K * seq_len);
    const double p = ps / seq_len;
    term_s[e] = f * p;
    if (f_out != nullptr) f_out[(size_t)q * E + e] = (float)f;
    if (p_out != nullptr) p_out[(size_t)q * E + e] = (float)p;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int e = 0; e < E; ++e) acc += term_s[e];
    loss[q] = (float)((double)alpha * acc);
  }
}

int balance_chunks(int seq_len) { return std::max(1, std::min(32, seq_len / 128)); }

hipError_t launch_balance(const float* P, int ksplit, int T, int E, int K, int seq_len,
                          float alpha, float* sn, int32_t* ids, double* psum, int32_t* pcnt,
                          float* loss, float* f, float* p, hipStream_t st) {
  hipLaunchKernelGGL(balance_token_kernel, dim3((T + BAL_WAVES - 1) / BAL_WAVES),
                     dim3(64 * BAL_WAVES), 0, st, P, ksplit, T, E, K, sn, ids);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_seq = T / seq_len, nch = balance_chunks(seq_len);
  hipLaunchKernelGGL(balance_chunk_kernel, dim3(n_seq, nch), dim3(256), 0, st, sn, ids, E, K,
                     seq_len, nch, psum, pcnt);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(balance_final_kernel, dim3(n_seq), dim3(256), 0, st, psum, pcnt, E, K,
                     seq_len, nch, alpha, loss, f, p);
  return hipGetLastError();
}

}  // namespace moe
