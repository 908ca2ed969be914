/*
 * moe.h — C ABI of the MI355X (gfx950) DeepSeekMoE layer-forward library.
 *
 * What the library computes is the MoE layer of DeepSeek-V3 as described on
 * the page "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token" (a close reading
 * of the DeepSeek-V3 technical report):
 *   §1.3 (Eq 15)  router affinities s = sigmoid(x · W_r), float32;
 *   §1.3 / §1.4   node-limited selection: experts form n_groups contiguous
 *                 groups, a group's score is the sum of its group_topn largest
 *                 biased scores z = s + b, the topk_groups best groups are kept
 *                 and the topk largest z among their experts are chosen;
 *   §1.3 (Eq 13)  gates: the chosen experts' unbiased s renormalised to sum 1;
 *   §1.3          no token is dropped; tokens are grouped by expert;
 *   §1.1          every expert is a SwiGLU FFN hidden -> inter -> hidden;
 *   §1.3 (Eq 12)  output = shared experts' FFN + sum_k gate_k · FFN_{e_k};
 *   §1.4          loss-free bias step: b_e -= gamma if expert e's load is
 *                 above the mean, b_e += gamma if below, unchanged if equal;
 *                 and the sequence-wise balance loss (Eq 17-20);
 *   §2.2          FP8 (E4M3) weights with one float32 scale per 128x128 block,
 *                 activations quantised online per 1x128 slice, float32
 *                 accumulation with the scales applied per 128-wide K block.
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to GPU memory of the current
 *    HIP device; they are owned by the caller, which keeps them alive until the
 *    enqueued work has finished.  The library allocates no device memory and
 *    keeps no pointer after a call returns.  Struct arguments (moe_cfg,
 *    moe_routing, moe_experts) are host memory, read during the call only.
 *  - All GPU work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *    default stream) without synchronising the host.  The return status covers
 *    argument validation and launch errors; a fault while the kernels run is
 *    reported by the caller's next synchronisation.
 *  - On a validation error nothing is launched and no output is written.
 *  - T == 0 returns MOE_OK once the cfg is valid, without reading any
 *    pointer (they may be NULL) and without launching.
 *  - Results are deterministic: the same inputs give bitwise identical outputs
 *    (no floating-point atomics; integer atomics only where the result does
 *    not depend on their order).
 *  - Calls are thread-safe when they use distinct workspaces; calls sharing a
 *    workspace must be ordered on one stream.
 *  - Non-finite inputs are not checked; the results are then undefined.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum moe_dtype {
  MOE_F32 = 0,   /* IEEE binary32 */
  MOE_BF16 = 1,  /* bfloat16 */
  MOE_E4M3 = 2   /* OCP FP8 E4M3FN codes (1 byte), weights only */
};

/* status codes */
enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,       /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,      /* inconsistent or unsupported sizes */
  MOE_ERR_DTYPE = -3,      /* unsupported dtype combination */
  MOE_ERR_WORKSPACE = -4,  /* workspace NULL or smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -5,        /* a HIP runtime call or kernel launch failed */
  MOE_ERR_DEVICE = -6,     /* the current device is not a gfx950 GPU */
  MOE_ERR_TOO_LARGE = -7   /* moe_forward_noalloc: the batch needs more than
                              MOE_NOALLOC_SCRATCH_BYTES of scratch */
};

/*
 * Layer shape.  V3: hidden 7168, inter 2048, n_experts 256, n_groups 8,
 * topk_groups 4, topk 8, group_topn 2, n_shared 1.
 * Constraints (else MOE_ERR_SHAPE):
 *   n_experts % n_groups == 0, n_experts <= 512, n_groups <= 64,
 *   1 <= group_topn <= min(4, n_experts / n_groups), 1 <= topk_groups <= n_groups,
 *   1 <= topk <= min(32, topk_groups * n_experts / n_groups),
 *   n_shared in {0, 1}, hidden % 128 == 0, inter % 128 == 0,
 *   hidden * inter * sizeof(w) < 2^32, n_experts * 3 * hidden * 2 < 2^32,
 *   and for E4M3 weights hidden <= 16384, inter <= 16384.
 * T bounds (else MOE_ERR_SHAPE): T * (topk + n_shared) < 2^31 and
 *   T * max(hidden, inter) * sizeof(act) < 2^32 (the tiled GEMMs address all
 *   of x, or one expert's staged rows, with 32-bit byte offsets); at the V3
 *   shape in bf16 that is T <= 299,593.
 * Dtypes (else MOE_ERR_DTYPE): (act, w) = (F32, F32), (BF16, BF16) or (BF16, E4M3).
 */
typedef struct moe_cfg {
  int32_t hidden;       /* H: model width */
  int32_t inter;        /* I: expert intermediate width */
  int32_t n_experts;    /* E: routed experts */
  int32_t n_groups;     /* G: expert groups (nodes in the pages' deployment) */
  int32_t topk_groups;  /* groups kept per token */
  int32_t topk;         /* K: routed experts per token */
  int32_t group_topn;   /* biased scores summed per group */
  int32_t n_shared;     /* S: shared experts, always applied with weight 1 */
  int32_t act_dtype;    /* moe_dtype of x, residual and y */
  int32_t w_dtype;      /* moe_dtype of the expert weights */
} moe_cfg;

/*
 * Routing results (device pointers, caller-allocated).  Layouts:
 *   topk_idx  int32 [T][K]  chosen expert ids, ascending per token
 *   topk_gate float [T][K]  gates, same order, each row sums to 1
 *   counts    int32 [E]     assignments per expert (sum = T*K)
 *   offsets   int32 [E+1]   exclusive prefix sum of counts
 *   perm      int32 [T*K]   token id of each expert-ordered row: rows
 *                           offsets[e] .. offsets[e+1]-1 list the tokens that
 *                           chose expert e in ascending token order
 *   slot      int32 [T*K]   row of assignment t*K+k in that order
 *   tie_gap   float [T]     may be NULL: min over the token of (K-th minus
 *                           (K+1)-th eligible biased score) and (kept minus
 *                           best dropped group score); < 1e-6 marks a near-tie
 */
typedef struct moe_routing {
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* slot;
  float* tie_gap;
} moe_routing;

/*
 * Expert weights (device pointers).  Routed experts are 0..E-1; the shared
 * expert is index E.  Row-major layouts:
 *   w_gate, w_up  [E+S][I][H]   element type w_dtype
 *   w_down        [E+S][H][I]
 *   s_gate, s_up  float [E+S][I/128][H/128]   (E4M3 only, else ignored)
 *   s_down        float [E+S][H/128][I/128]   (E4M3 only, else ignored)
 * For E4M3 the weight value is code * scale of its 128x128 block.
 */
typedef struct moe_experts {
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
} moe_experts;

/* Workspace bytes that moe_route / moe_forward need for T tokens (0 on a bad cfg). */
size_t moe_workspace_bytes(const moe_cfg* cfg, int64_t T);

/*
 * Router, node-limited selection, gates and the expert permutation.
 *   x        device [T][H] act_dtype      token activations
 *   w_router device float [H][E]          expert centroids as columns
 *   bias     device float [E]             load-balancing bias (zeros for none)
 *   out      host struct of device outputs; every field but tie_gap required
 *   ws       device workspace of ws_bytes >= moe_workspace_bytes(cfg, T)
 */
int moe_route(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
              const float* bias, const moe_routing* out, void* ws, size_t ws_bytes,
              void* stream);

/*
 * The whole layer forward: moe_route followed by the routed and shared
 * SwiGLU experts and the gated combine.
 *   residual device [T][H] act_dtype or NULL; when given it is added to y
 *   y        device [T][H] act_dtype output
 *   out      NULL (routing kept in the workspace) or as in moe_route
 * Intermediate activations are rounded to bfloat16 (E4M3 with 1x128 scales
 * for E4M3 weights; float32 for the F32 configuration) and the combine
 * accumulates in float32 in ascending expert order, shared expert first.
 */
int moe_forward(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
                const float* bias, const moe_experts* w, const void* residual, void* y,
                const moe_routing* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results as moe_forward, with no workspace argument.
 * Its scratch is a static device buffer of MOE_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on every GPU it runs on until the process ends; the
 * call allocates nothing (no hipMalloc, no library allocation, no timing
 * events: moe_profile_* do not record it).
 *   Arguments as in moe_forward.  A batch whose moe_workspace_bytes(cfg, T)
 *   exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_TOO_LARGE without
 *   launching (at the V3 shape: T <= 321 in bf16, T <= 342 with E4M3 weights).
 * Every call on one GPU uses that GPU's one buffer: calls that overlap on one
 * GPU (other streams, other host threads) race and must be ordered by the
 * caller.  The buffer keeps the last call's contents; no result depends on
 * them (every scratch byte a call reads, it has written earlier in the call).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
                        const float* bias, const moe_experts* w, const void* residual, void* y,
                        const moe_routing* out, void* stream);

/*
 * Loss-free bias step on the loads of one batch.
 *   counts device int32 [E] (e.g. moe_routing.counts of the step's batch)
 *   bias   device float [E], updated in place:
 *          b_e -= gamma if counts_e * E > T * K, b_e += gamma if < , else kept
 */
int moe_bias_update(const moe_cfg* cfg, int64_t T, const int32_t* counts, float* bias,
                    float gamma, void* stream);

/*
 * Complementary sequence-wise balance loss of the router (page "02 ·
 * DeepSeek-V3", §1.4, Eq 17-20), the small loss V3 keeps beside the bias.
 * For each sequence (consecutive blocks of seq_len tokens, T % seq_len == 0):
 *   f_e = E / (K * seq_len) * (tokens whose top-K of the raw affinities s,
 *         without the bias and without the group limit, holds expert e;
 *         ties go to the lower index),
 *   P_e = mean over the sequence of s_e / sum_j s_j,
 *   loss = alpha * sum_e f_e * P_e        (the pages use alpha = 1e-4).
 *   x, w_router as in moe_route
 *   loss device float [T/seq_len]
 *   f, p device float [T/seq_len][E] each, or NULL
 *   ws   workspace of at least moe_workspace_bytes(cfg, T) bytes
 * Counts are exact; P and the loss are summed in float64 in a fixed order
 * (deterministic).  T == 0 returns MOE_OK without reading pointers.
 */
int moe_balance_loss(const moe_cfg* cfg, int64_t T, int32_t seq_len, const void* x,
                     const float* w_router, float alpha, float* loss, float* f, float* p,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the layer for one training step (page "02 · DeepSeek-V3",
 * §1.3 Eq 12-15, §1.4, §2.2): the gradients of <dy, y> for the upstream
 * gradient dy of the layer output y (the MoE branch).  The call recomputes the
 * routing and the experts' intermediates from x (the SwiGLU output is
 * recomputed, §2.2); the selection of experts is the forward's and carries no
 * gradient, and the bias takes no part in backpropagation (§1.4), so it has
 * none.  Gates are the normalised raw affinities of the chosen experts
 * (Eq 13); their gradient flows through the normalisation and the sigmoid
 * into x and W_r.
 *   x, w_router, bias, w   as in moe_forward (BF16 activations with BF16 or
 *                          E4M3 weights; other dtypes return MOE_ERR_DTYPE;
 *                          hidden and inter multiples of 256, else
 *                          MOE_ERR_SHAPE)
 *   dy        device bf16 [T][H] upstream gradient
 *   dx        device bf16 [T][H] out
 *   dw_router device float [H][E] out
 *   dw_gate, dw_up  device float [E+S][I][H] out (experts without tokens: 0)
 *   dw_down   device float [E+S][H][I] out
 *   ws        workspace of at least moe_backward_workspace_bytes(cfg, T) bytes
 * E4M3 weights (§2.2): every expert GEMM takes E4M3 operands.  The SwiGLU
 * input G, U is recomputed from x quantised in 1x128 tiles and kept as
 * 1x128 E4M3; H is recomputed from it.  The output gradients g dy and the
 * gradients dG, dU are quantised in 1x128 tiles for the data-gradient GEMMs;
 * the weight-gradient GEMMs, which contract over an expert's rows, take both
 * operands in 128x1 tiles (per column, 128 consecutive rows of the expert
 * from its first row).  Scales follow moe_quantize_1x128's rule.
 * Every output is overwritten.  Sums over tokens and experts run in a fixed
 * order (deterministic).  Staged rows use 32-bit offsets: T * (K + S) *
 * max(H, I) * 2 must stay below 4 GiB, and H * I * 2 too (else MOE_ERR_SHAPE).
 * T == 0 returns MOE_OK without reading pointers.
 */
size_t moe_backward_workspace_bytes(const moe_cfg* cfg, int64_t T);
int moe_backward(const moe_cfg* cfg, int64_t T, const void* x, const float* w_router,
                 const float* bias, const moe_experts* w, const void* dy, void* dx,
                 float* dw_router, float* dw_gate, float* dw_up, float* dw_down, void* ws,
                 size_t ws_bytes, void* stream);

/*
 * Online activation quantisation to E4M3 (page "02 · DeepSeek-V3", §2.2: one
 * scale per 1x128 tile of a token row, from the tile's max-abs value), the
 * step moe_forward applies to x when the weights are E4M3.
 *   x      device bfloat16 [rows][cols], cols % 128 == 0 (else MOE_ERR_SHAPE)
 *   q      device uint8 [rows][cols]: OCP E4M3FN codes
 *   scales device float [rows][cols/128]
 * Per slice: scale = amax / 448 in float32 (1 where that is 0); each code is
 * the float32 quotient v / scale (IEEE division) rounded to nearest, ties to
 * even, saturated at +-448.  rows == 0 returns MOE_OK without reading
 * pointers.
 */
int moe_quantize_1x128(const void* x, int64_t rows, int32_t cols, uint8_t* q, float* scales,
                       void* stream);

/*
 * Kernel timing instrumentation (off by default).  The state is per host
 * thread: moe_profile_enable switches it for the calling thread, whose
 * compute calls then record, and moe_profile_read reads that thread's record.
 * While enabled, every kernel launch (or, in moe_backward, every stage of
 * launches) of the compute entry points is bracketed by a pair of HIP events
 * on the caller's stream.
 * moe_profile_read waits for the recorded events, adds each pair's elapsed
 * time to the slot of its kernel, clears the record, and returns the number
 * of slots (at most n_slots are written to total_ms / launches, which may be
 * NULL to query the count).  moe_profile_kernel_name names a slot.
 */
int moe_profile_enable(int on);
int moe_profile_read(double* total_ms, int32_t* launches, int n_slots);
const char* moe_profile_kernel_name(int slot);

/* Static description of a status code. */
const char* moe_status_string(int status);

/* ABI version (major * 100 + minor). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
