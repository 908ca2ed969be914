"""CPU oracle for the DeepSeekMoE layer forward (DeepSeek-V3 shape).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module shares no code with it.

It is the plain, slow definition of what the layer computes, in numpy float64
(float32 where the method fixes float32: the router logits, the affinities,
the biased selection scores and the bias itself).  Sources, cited by page title
and section:

  [V3]   "02 · DeepSeek-V3: 671B 总参, 37B 激活, 14.8T token"
         (PaperTrace close reading of the DeepSeek-V3 technical report)
         §1.1 shapes; §1.3 sigmoid gating and node-limited routing (Eq 12,
         13, 15); §1.4 auxiliary-loss-free balancing (Eq 16; the bias takes
         no part in backpropagation) and the sequence-wise balance loss
         (Eq 17-20); §2.2 FP8 fine-grained quantisation and the recomputed
         SwiGLU output in the backward; §5.1 deployment (shared expert as an
         always-selected expert).
  [DEP]  "DeepSeek-V3 复盘：MoE、MLA、FP8 与低成本叙事如何验算" (audit of the
         report's cost and deployment claims; the released weights are FP8).

The display equations of [V3] are missing from the extracted text; every
formula below is rebuilt from the surrounding prose, and each reading taken
where the prose is silent is named in the docstring that uses it.

Parity status of each function (what pins it in tests/test_oracle_*.py):
  router_affinity       pinned (loop brute force; sigmoid vs scipy.expit)
  select_experts        pinned (subset-enumeration brute force; plain top-K
                        special case; group containment; bias invariants)
  gate_values           pinned (sum-to-one; bias-independence)
  permute               pinned (per-expert brute-force listing; bincount)
  expert_ffn / forward  pinned for the FFN and combine structure (scalar
                        triple-loop brute force, shared-only and single-expert
                        special cases); layer output VALUES at V3 size are
                        otherwise parity unpinned: the pages print no worked
                        example of the layer.
  bias_update           pinned (rule worked by hand from §1.4, golden file)
  sequence_balance_loss pinned (closed forms for balanced and uniform
                        affinities; sum f = E, sum P = 1; scalar-loop brute force)
  e4m3_* / quantize_1x128  pinned (all 256 codes; torch float8_e4m3fn)
  backward and its parts  pinned (central finite differences of
                        layer_fixed_routing in every input; torch CPU autograd
                        of the fixed-routing layer; zero router gradient with
                        one routed expert; linearity in dy)
  quantize_128x1        pinned (equals quantize_1x128 of the transpose)
  forward(act_quant) / expert_ffn_fp8  pinned (with the identity quantiser it
                        is the plain forward up to the float32 rounding of H;
                        scalar-loop brute force of the 1x128 quantisation of x
                        and H, with torch's float8_e4m3fn as the encoder, on
                        tiny E4M3 layers with outliers)
  backward(fp8_emulation) and expert_*_fp8  pinned (with the quantisers
                        replaced by the identity it equals the pinned backward;
                        token isolation of dx; exact column equivariance of
                        dW_down in dy; weight gradients unchanged by a
                        sub-step change of one dy element)
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, Optional, Sequence

import numpy as np

F32 = np.float32
F64 = np.float64

NEAR_TIE = 1e-6   # gap below which a selection is flagged, in biased score units


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------

def lift(a) -> np.ndarray:
    """Exact lift of a float32 / bfloat16 array (numpy or torch CPU) to float64."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu")
            if a.dtype == torch.bfloat16:
                a = a.to(torch.float32)          # exact
            a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------
# step 1: router affinities ([V3] §1.3, Eq 15)
# ----------------------------------------------------------------------------

def router_affinity(x64: np.ndarray, wr64: np.ndarray):
    """Logits and sigmoid affinities of every token for every routed expert.

    The affinity of token t for expert i is the logistic sigmoid of the dot
    product of the token with the expert's centroid (a column of the router
    weight), [V3] §1.3 Eq 15.  The logit is formed as a float64 dot product and
    rounded once to float32; the sigmoid is evaluated in float64 on that
    float32 logit and rounded to float32 (the method works in float32).

    Returns (L float32 [T][E], s float32 [T][E]).
    """
    L = (x64 @ wr64).astype(F32)
    Ld = L.astype(F64)
    s = (1.0 / (1.0 + np.exp(-Ld))).astype(F32)
    return L, s


# ----------------------------------------------------------------------------
# steps 2-3: node-limited selection and gates ([V3] §1.3, §1.4)
# ----------------------------------------------------------------------------

@dataclass
class Routing:
    idx: np.ndarray        # [T][K] int32, ascending expert id
    gate: np.ndarray       # [T][K] float32, sums to 1 per token
    z: np.ndarray          # [T][E] float32 biased scores s + b
    group_score: np.ndarray  # [T][G] float32
    groups: np.ndarray     # [T][topk_groups] int32 kept groups (rank order)
    egap: np.ndarray       # [T] float64: z of K-th minus (K+1)-th eligible expert
    ggap: np.ndarray       # [T] float64: kept-group score minus best dropped one
    flagged: np.ndarray    # [T] bool: min(egap, ggap) < NEAR_TIE


def biased_scores(s32: np.ndarray, b32: np.ndarray) -> np.ndarray:
    """Selection score z = s + b in float32.

    [V3] §1.4 (Eq 16): the per-expert bias enters the ranking only; it is added
    to the sigmoid affinity (after the sigmoid), in float32.
    """
    return (s32.astype(F32) + b32.astype(F32)[None, :]).astype(F32)


def group_scores(z32: np.ndarray, n_groups: int, group_topn: int) -> np.ndarray:
    """Score of each expert group: sum of its ``group_topn`` largest biased scores.

    [V3] §1.3: experts are spread evenly over the nodes and each node is ranked
    by the sum of its top K_r/M = 2 affinities.  Readings: groups are
    contiguous blocks of E/G expert ids; the summed scores are the biased ones
    (s + b), since the ranking of §1.4 uses s + b; the float32 sum is taken
    from the largest value down.
    """
    T, E = z32.shape
    zg = z32.reshape(T, n_groups, E // n_groups)
    top = -np.sort(-zg, axis=2)[:, :, :group_topn]
    gs = top[:, :, 0].astype(F32)
    for j in range(1, group_topn):
        gs = (gs + top[:, :, j]).astype(F32)
    return gs


def select_experts(s32: np.ndarray, b32: np.ndarray, n_groups: int, topk_groups: int,
                   topk: int, group_topn: int = 2) -> Routing:
    """Node-limited top-K selection with the loss-free bias, and the gates.

    [V3] §1.3: rank the groups by their group score, keep the best
    ``topk_groups`` (4 of 8 for V3), then take the ``topk`` (8) experts with the
    largest scores among the kept groups' experts only.  [V3] §1.4: the ranking
    uses z = s + b.  Exact ties go to the lower group / expert index.  The
    chosen experts are listed in ascending id.
    """
    T, E = s32.shape
    per = E // n_groups
    z = biased_scores(s32, b32)
    gs = group_scores(z, n_groups, group_topn)
    gorder = np.argsort(-gs, axis=1, kind="stable")        # ties: lower index first
    groups = gorder[:, :topk_groups].astype(np.int32)
    eligible = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(eligible, groups.astype(np.int64), True, axis=1)
    elig_e = np.repeat(eligible, per, axis=1)                # [T][E]
    masked = np.where(elig_e, z.astype(F64), -np.inf)
    eorder = np.argsort(-masked, axis=1, kind="stable")
    idx = np.sort(eorder[:, :topk], axis=1).astype(np.int32)

    zs = np.take_along_axis(masked, eorder, axis=1)
    n_elig = topk_groups * per
    egap = zs[:, topk - 1] - zs[:, topk] if n_elig > topk else np.full(T, np.inf)
    if topk_groups < n_groups:
        gss = np.take_along_axis(gs.astype(F64), gorder, axis=1)
        ggap = gss[:, topk_groups - 1] - gss[:, topk_groups]
    else:
        ggap = np.full(T, np.inf)
    flagged = np.minimum(egap, ggap) < NEAR_TIE
    gate = gate_values(s32, idx)
    return Routing(idx=idx, gate=gate, z=z, group_score=gs, groups=groups,
                   egap=egap, ggap=ggap, flagged=flagged)


def gate_values(s32: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gates of the chosen experts: their unbiased affinities renormalised to sum to 1.

    [V3] §1.3 (Eq 13): after the top-K choice the K affinities are normalised
    among themselves; [V3] §1.4: the bias is not part of the gate.  Computed in
    float64 from the float32 affinities and rounded to float32.
    """
    sel = np.take_along_axis(s32.astype(F64), idx.astype(np.int64), axis=1)
    return (sel / sel.sum(axis=1, keepdims=True)).astype(F32)


# ----------------------------------------------------------------------------
# step 4: permutation by expert ([V3] §1.3: no token is dropped)
# ----------------------------------------------------------------------------

@dataclass
class Perm:
    counts: np.ndarray   # [E] int32
    offsets: np.ndarray  # [E+1] int32
    perm: np.ndarray     # [T*K] int32 token id of each expert-ordered row
    slot: np.ndarray     # [T*K] int32 expert-ordered row of assignment t*K+k


def permute(idx: np.ndarray, n_experts: int) -> Perm:
    """Group the token-expert assignments by expert, keeping token order.

    Every assignment is kept (no dropping, [V3] §1.3).  Assignments are
    enumerated token-major (a = t*K + k); a stable sort by expert id lists the
    rows of each expert in ascending token order.
    """
    T, K = idx.shape
    e_of = idx.reshape(-1).astype(np.int64)
    order = np.argsort(e_of, kind="stable")
    counts = np.bincount(e_of, minlength=n_experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    slot = np.empty(T * K, dtype=np.int32)
    slot[order] = np.arange(T * K, dtype=np.int32)
    return Perm(counts=counts, offsets=offsets, perm=(order // K).astype(np.int32), slot=slot)


# ----------------------------------------------------------------------------
# step 5: SwiGLU experts and the gated combine ([V3] §1.1, §1.3 Eq 12)
# ----------------------------------------------------------------------------

def route(x64: np.ndarray, wr64: np.ndarray, b32: np.ndarray, *, n_groups: int, topk_groups: int,
          topk: int, group_topn: int = 2):
    """Steps 1-4 only: affinities, selection, gates and the expert permutation.

    Returns (L, s, Routing, Perm).
    """
    L, s = router_affinity(x64, wr64)
    r = select_experts(s, b32, n_groups, topk_groups, topk, group_topn)
    return L, s, r, permute(r.idx, wr64.shape[1])


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def expert_ffn(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on the rows of X, float64.

    [V3] §1.1: an expert is a SwiGLU block of three matrices
    (hidden -> intermediate -> hidden).  Reading: H = SiLU(X W_gate^T) * (X W_up^T),
    Y = H W_down^T with SiLU(v) = v * sigmoid(v); W_gate, W_up are
    [inter][hidden] and W_down is [hidden][inter].
    """
    G = X @ wg.T
    U = X @ wu.T
    return (silu(G) * U) @ wd.T


def expert_ffn_fp8(Xq: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                   act_quant: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> np.ndarray:
    """One SwiGLU expert on the E4M3 forward path, float64.

    [V3] §2.2: the inputs of every expert GEMM are E4M3 with one scale per
    1x128 activation tile; the products are accumulated at high precision.
    ``Xq`` holds the expert's input rows already quantised (the layer input is
    quantised once, before any expert); ``wg``, ``wu``, ``wd`` are the
    dequantised weights.  Reading: G = Xq W_gate^T and U = Xq W_up^T are exact
    products; H = SiLU(G) * U is rounded to float32 (the value a float32
    accumulator holds when it is quantised) and quantised 1x128 along the
    intermediate dimension as the down projection's input; Y = Q(H) W_down^T.
    ``act_quant`` is the quantiser (``fake_quant_1x128`` when None).
    """
    q = fake_quant_1x128 if act_quant is None else act_quant
    Hh = (silu(Xq @ wg.T) * (Xq @ wu.T)).astype(F32).astype(F64)
    return q(Hh) @ wd.T


ExpertSource = Callable[[int], Dict[str, np.ndarray]]


def dequant_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Weights stored as e4m3 codes with one float32 scale per 128x128 block, as float64."""
    v = e4m3_decode(np.asarray(codes))
    R, C = v.shape
    sc = np.asarray(scales, dtype=F64)
    return (v.reshape(R // 128, 128, C // 128, 128) * sc[:, None, :, None]).reshape(R, C)


def expert_f64(w: Dict[str, np.ndarray]):
    """(W_gate, W_up, W_down) of one expert as float64 (e4m3 codes dequantised)."""
    if "s_gate" in w:
        return (dequant_blocks(w["w_gate"], w["s_gate"]), dequant_blocks(w["w_up"], w["s_up"]),
                dequant_blocks(w["w_down"], w["s_down"]))
    return lift(w["w_gate"]), lift(w["w_up"]), lift(w["w_down"])


@dataclass
class ForwardResult:
    y: np.ndarray          # [n_tokens][H] float64 MoE branch (+ residual if given)
    tokens: np.ndarray     # token ids the rows of y belong to
    routing: Routing
    perm: Perm


def forward(x64: np.ndarray, wr64: np.ndarray, b32: np.ndarray, experts: ExpertSource, *,
            n_groups: int, topk_groups: int, topk: int, group_topn: int = 2, n_shared: int = 1,
            tokens: Optional[Sequence[int]] = None, residual: Optional[np.ndarray] = None,
            act_quant: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> ForwardResult:
    """The MoE layer output for every token (or for ``tokens`` only).

    [V3] §1.3 Eq 12: the output is the shared expert's FFN output plus the
    gate-weighted sum of the chosen routed experts' FFN outputs (plus the
    residual u_t, which is added only when ``residual`` is given).  The shared
    expert is always applied with weight 1 outside the gate normalisation
    ([V3] §5.1 treats it as a ninth, always-selected expert).  Routing always
    covers all T tokens (the permutation depends on the whole batch); expert
    FFNs are evaluated only for the requested tokens.

    ``experts(e)`` returns expert e's weights (routed 0..E-1, shared = E).
    ``act_quant`` (optional) maps a float64 activation matrix to its quantised
    value (``fake_quant_1x128`` for the E4M3 path of [V3] §2.2): it is applied
    once to the layer input x, and each expert then runs ``expert_ffn_fp8``
    with it.
    """
    T = x64.shape[0]
    E = wr64.shape[1]
    L, s = router_affinity(x64, wr64)
    r = select_experts(s, b32, n_groups, topk_groups, topk, group_topn)
    p = permute(r.idx, E)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xin = x64[tok]
    if act_quant is not None:
        xin = act_quant(xin)
    y = np.zeros((len(tok), x64.shape[1]), dtype=F64)

    def ffn(w, X):
        wg, wu, wd = expert_f64(w)
        if act_quant is None:
            return expert_ffn(X, wg, wu, wd)
        return expert_ffn_fp8(X, wg, wu, wd, act_quant)

    # routed experts in ascending id, each on the requested tokens that chose
    # it, so every token accumulates its K terms in ascending expert order
    sel = r.idx[tok]
    for e in sorted(set(int(v) for v in sel.reshape(-1))):
        jj, kk = np.nonzero(sel == e)
        Y = ffn(experts(e), xin[jj])
        y[jj] += r.gate[tok[jj], kk].astype(F64)[:, None] * Y
    for sh in range(n_shared):
        y += ffn(experts(E + sh), xin)
    if residual is not None:
        y += lift(residual)[tok]
    return ForwardResult(y=y, tokens=tok, routing=r, perm=p)


# ----------------------------------------------------------------------------
# backward of the layer for one training step ([V3] §1.3 Eq 12-15, §1.4, §2.2)
# ----------------------------------------------------------------------------
#
# The gradients are those of the scalar <dy, y> for an upstream gradient dy of
# the layer output y (the MoE branch).  Readings:
#   - the selection of experts is a discrete choice and carries no gradient;
#     the bias enters only the selection and takes no part in
#     backpropagation ([V3] §1.4 says so explicitly), so it has no gradient;
#   - the gates are the normalised raw affinities of the chosen experts
#     ([V3] §1.3 Eq 13), and their gradient flows through the normalisation
#     and the sigmoid into the router logits, hence into x and W_r;
#   - the function differentiated is the layer in float64 with the selection
#     held fixed (``layer_fixed_routing``); the selection itself is the
#     forward's (float32 scores with the bias).

def dsilu(v: np.ndarray) -> np.ndarray:
    """Derivative of SiLU(v) = v * sigmoid(v): sigmoid(v) * (1 + v * (1 - sigmoid(v)))."""
    sg = 1.0 / (1.0 + np.exp(-v))
    return sg * (1.0 + v * (1.0 - sg))


def layer_fixed_routing(x64: np.ndarray, wr64: np.ndarray, idx: np.ndarray, experts: ExpertSource,
                        n_shared: int = 1) -> np.ndarray:
    """The layer output in float64 as a smooth function of x, W_r and the
    expert weights, for a fixed choice of experts ``idx`` [T][K].

    [V3] §1.3 Eq 12, 13, 15: y_t = sum over shared experts of FFN(x_t) +
    sum_k g_tk FFN_{e_k}(x_t), g_tk = s_{t,e_k} / sum_j s_{t,e_j},
    s = sigmoid(x W_r) (no float32 rounding here).
    """
    T = x64.shape[0]
    E = wr64.shape[1]
    s = 1.0 / (1.0 + np.exp(-(x64 @ wr64)))
    ssel = np.take_along_axis(s, idx, axis=1)
    g = ssel / ssel.sum(axis=1, keepdims=True)
    y = np.zeros_like(x64)
    for e in sorted(set(int(v) for v in idx.reshape(-1))):
        jj, kk = np.nonzero(idx == e)
        wg, wu, wd = expert_f64(experts(e))
        y[jj] += g[jj, kk][:, None] * expert_ffn(x64[jj], wg, wu, wd)
    for sh in range(n_shared):
        wg, wu, wd = expert_f64(experts(E + sh))
        y += expert_ffn(x64, wg, wu, wd)
    return y


def expert_backward(X: np.ndarray, dY: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """Backward of one SwiGLU expert Y = (SiLU(X W_gate^T) * (X W_up^T)) W_down^T.

    [V3] §1.1 (the three matrices) and §2.2 (the SwiGLU input is kept and its
    output recomputed in the backward): with G = X W_gate^T, U = X W_up^T,
    A = SiLU(G), H = A * U,
      dH = dY W_down,      dW_down = dY^T H,
      dU = dH * A,         dG = dH * U * SiLU'(G),
      dX = dG W_gate + dU W_up,  dW_gate = dG^T X,  dW_up = dU^T X.
    Returns (dX, dW_gate, dW_up, dW_down), float64.
    """
    G = X @ wg.T
    U = X @ wu.T
    A = silu(G)
    Hh = A * U
    dH = dY @ wd
    dwd = dY.T @ Hh
    dU = dH * A
    dG = dH * U * dsilu(G)
    dX = dG @ wg + dU @ wu
    return dX, dG.T @ X, dU.T @ X, dwd


def expert_swiglu_input_fp8(X: np.ndarray, wg: np.ndarray, wu: np.ndarray):
    """The E4M3 path's SwiGLU input of one expert, as the backward keeps it.

    [V3] §2.2: the expert inputs are quantised in 1x128 tiles; the SwiGLU
    input is cached in E4M3 and the SwiGLU output is recomputed from that cache
    in the backward.  Reading: G = Q(X) W_gate^T and U = Q(X) W_up^T (exact
    products of the dequantised operands), each cached as Q(G), Q(U) with the
    1x128 rule along the intermediate dimension.  ``wg``, ``wu`` are the
    dequantised weights.  Returns (Q(X), Q(G), Q(U)) dequantised, float64.
    """
    Xq = fake_quant_1x128(X)
    return Xq, fake_quant_1x128(Xq @ wg.T), fake_quant_1x128(Xq @ wu.T)


def expert_output_fp8(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One expert's output recomputed on the E4M3 path from the cached SwiGLU
    input: Y = Q(SiLU(Q(G)) * Q(U)) W_down^T, the SwiGLU output quantised 1x128
    as the down projection's input ([V3] §2.2)."""
    _, Gc, Uc = expert_swiglu_input_fp8(X, wg, wu)
    return fake_quant_1x128(silu(Gc) * Uc) @ wd.T


def expert_backward_fp8(X: np.ndarray, dY: np.ndarray, wg: np.ndarray, wu: np.ndarray,
                        wd: np.ndarray):
    """Backward of one SwiGLU expert on the E4M3 path ([V3] §2.2), float64.

    The steps of ``expert_backward`` with every GEMM operand in E4M3:
      - the cached SwiGLU input Q(G), Q(U) (``expert_swiglu_input_fp8``) and
        the recomputed H = SiLU(Q(G)) * Q(U);
      - dgrad products contract over the hidden or intermediate dimension, so
        their activation operands take 1x128 tiles: dH = Q(dY) W_down,
        dX = Q(dG) W_gate + Q(dU) W_up, with dG = dH * Q(U) * SiLU'(Q(G)) and
        dU = dH * SiLU(Q(G));
      - wgrad products contract over the expert's rows (tokens), so both
        operands take 128x1 tiles, 128 consecutive rows of one column:
        dW_down = Q'(dY)^T Q'(H), dW_gate = Q'(dG)^T Q'(X), dW_up = Q'(dU)^T Q'(X)
        (Q' = ``fake_quant_128x1`` over the rows in the order given).
    The weights ``wg``, ``wu``, ``wd`` are the dequantised 128x128-block E4M3
    weights; X is the expert's input rows, dY its output gradient rows.
    Returns (dX, dW_gate, dW_up, dW_down).
    """
    _, Gc, Uc = expert_swiglu_input_fp8(X, wg, wu)
    A = silu(Gc)
    Hh = A * Uc
    dH = fake_quant_1x128(dY) @ wd
    dU = dH * A
    dG = dH * Uc * dsilu(Gc)
    dX = fake_quant_1x128(dG) @ wg + fake_quant_1x128(dU) @ wu
    dwd = fake_quant_128x1(dY).T @ fake_quant_128x1(Hh)
    Xr = fake_quant_128x1(X)
    return dX, fake_quant_128x1(dG).T @ Xr, fake_quant_128x1(dU).T @ Xr, dwd


def gate_backward(ssel: np.ndarray, dg: np.ndarray) -> np.ndarray:
    """Gradient of the router logits of the chosen experts from the gate gradients.

    [V3] §1.3 Eq 13 and 15: g_k = s_k / S with S = sum_j s_j over the chosen
    experts and s = sigmoid(L).  Then ds_j = (dg_j - sum_k dg_k g_k) / S and
    dL_j = ds_j s_j (1 - s_j); the logits of experts not chosen get no gradient.
    ``ssel`` and ``dg`` are [T][K]; returns dL [T][K].
    """
    S = ssel.sum(axis=1, keepdims=True)
    g = ssel / S
    ds = (dg - (dg * g).sum(axis=1, keepdims=True)) / S
    return ds * ssel * (1.0 - ssel)


@dataclass
class BackwardResult:
    dx: np.ndarray                 # [len(tokens)][H] float64
    tokens: np.ndarray             # token ids the rows of dx belong to
    dw_router: np.ndarray          # [H][E] float64 (columns of router_cols, others 0)
    dw: Dict[int, tuple]           # expert id -> (dW_gate, dW_up, dW_down), float64
    dgate: np.ndarray              # [T][K] float64 gate gradients (rows of grad_tokens)
    dlogit: np.ndarray             # [T][K] float64 logit gradients of the chosen experts
    routing: Routing
    perm: Perm


def backward(x64: np.ndarray, wr64: np.ndarray, b32: np.ndarray, experts: ExpertSource,
             dy64: np.ndarray, *, n_groups: int, topk_groups: int, topk: int, group_topn: int = 2,
             n_shared: int = 1, tokens: Optional[Sequence[int]] = None,
             grad_experts: Optional[Sequence[int]] = None,
             router_cols: Optional[Sequence[int]] = None,
             fp8_emulation: bool = False) -> BackwardResult:
    """Gradients of <dy, y> w.r.t. x, W_r and every expert's three matrices.

    Steps, in the order of the forward they reverse ([V3] §1.3 Eq 12-15):
      1. route as the forward does (selection with the bias, [V3] §1.4);
      2. per chosen expert, its output Y_k(x_t) and the gate gradient
         dg_tk = <dy_t, Y_k(x_t)> (Eq 12);
      3. logit gradients of the chosen experts through the gate
         normalisation and the sigmoid (``gate_backward``);
      4. router: dx_t += sum_k dL_tk W_r[:, e_k]; dW_r[:, e] = sum over the
         assignments (t, k) to e of dL_tk x_t;
      5. each expert's backward with dY = g_tk dy_t on its rows (the shared
         expert: dY = dy_t on every row), dx_t += its dX rows (``expert_backward``).
    Float64 throughout on float64 affinities s = sigmoid(x W_r).

    Subsets for large shapes: ``tokens`` (rows of dx), ``grad_experts``
    (experts whose weight gradients are formed; shared = E), ``router_cols``
    (columns of dW_r).  Gate and logit gradients are formed for the tokens
    these need.  Defaults: everything.

    ``fp8_emulation``: the E4M3 path of [V3] §2.2 (weights given as E4M3 codes
    and 128x128 block scales): expert outputs from ``expert_output_fp8`` and
    expert gradients from ``expert_backward_fp8``; an expert's rows are its
    tokens in ascending order (shared: all tokens), the row order of its
    128x1 tiles.  Without it, the weights are dequantised and the activations
    stay exact.
    """
    ffn_out = expert_output_fp8 if fp8_emulation else expert_ffn
    ffn_bwd = expert_backward_fp8 if fp8_emulation else expert_backward
    T, H = x64.shape
    E = wr64.shape[1]
    L, s32, r, p = route(x64, wr64, b32, n_groups=n_groups, topk_groups=topk_groups, topk=topk,
                         group_topn=group_topn)
    idx = r.idx.astype(np.int64)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    gexp = list(range(E + n_shared)) if grad_experts is None else [int(e) for e in grad_experts]
    rcols = list(range(E)) if router_cols is None else [int(e) for e in router_cols]

    # tokens whose logit gradients are needed: rows of dx, and every token
    # routed to a column of dW_r
    need = set(int(t) for t in tok)
    for e in rcols:
        need.update(int(t) for t in np.nonzero((idx == e).any(axis=1))[0])
    need = np.array(sorted(need), dtype=np.int64)

    s = 1.0 / (1.0 + np.exp(-(x64 @ wr64)))
    ssel = np.take_along_axis(s, idx, axis=1)
    g = ssel / ssel.sum(axis=1, keepdims=True)

    # step 2: gate gradients of the needed tokens
    dg = np.zeros((T, topk), dtype=F64)
    if len(need):
        sel = idx[need]
        for e in sorted(set(int(v) for v in sel.reshape(-1))):
            jj, kk = np.nonzero(sel == e)
            wg, wu, wd = expert_f64(experts(e))
            Y = ffn_out(x64[need[jj]], wg, wu, wd)
            dg[need[jj], kk] = np.einsum("rh,rh->r", dy64[need[jj]], Y)
    # step 3
    dL = np.zeros((T, topk), dtype=F64)
    dL[need] = gate_backward(ssel[need], dg[need])

    # step 4: router
    dx = np.zeros((len(tok), H), dtype=F64)
    for k in range(topk):
        dx += dL[tok, k][:, None] * wr64[:, idx[tok, k]].T
    dwr = np.zeros((H, E), dtype=F64)
    for e in rcols:
        tt, kk = np.nonzero(idx == e)
        dwr[:, e] = (dL[tt, kk][:, None] * x64[tt]).sum(axis=0)

    # step 5: experts.  Weight gradients need all rows of the expert; dx needs
    # the rows of the requested tokens.
    pos = {int(t): i for i, t in enumerate(tok)}
    dw = {}
    sel_tok = idx[tok]
    shared_ids = set(range(E, E + n_shared))   # every token's rows: they always reach dx
    for e in sorted(set(int(v) for v in sel_tok.reshape(-1)) | set(gexp) | shared_ids):
        wg, wu, wd = expert_f64(experts(e))
        if e >= E:                                  # shared: every token, dY = dy
            rows = np.arange(T) if e in gexp else tok
            dY = dy64[rows]
        else:
            tt, kk = np.nonzero(idx == e)
            if e not in gexp:                       # only the requested tokens' rows
                keep = np.isin(tt, tok)
                tt, kk = tt[keep], kk[keep]
            rows = tt
            dY = g[tt, kk][:, None] * dy64[tt]
        if len(rows) == 0:
            if e in gexp:
                dw[e] = (np.zeros_like(wg), np.zeros_like(wu), np.zeros_like(wd))
            continue
        dX, dwg, dwu, dwd = ffn_bwd(x64[rows], dY, wg, wu, wd)
        if e in gexp:
            dw[e] = (dwg, dwu, dwd)
        for i, t in enumerate(rows):
            j = pos.get(int(t))
            if j is not None:
                dx[j] += dX[i]
    return BackwardResult(dx=dx, tokens=tok, dw_router=dwr, dw=dw, dgate=dg, dlogit=dL,
                          routing=r, perm=p)


# ----------------------------------------------------------------------------
# step 6: auxiliary-loss-free bias update ([V3] §1.4)
# ----------------------------------------------------------------------------

def bias_update(b32: np.ndarray, counts: np.ndarray, T: int, K: int, gamma: float) -> np.ndarray:
    """One loss-free balancing step on the bias.

    [V3] §1.4: at the end of a step the load of each expert over the whole
    batch is counted; an overloaded expert's bias drops by gamma and an
    underloaded one's rises by gamma (a sign update).  Reading: the mean load
    is T*K/E; overloaded means count > mean, underloaded count < mean, and an
    expert at exactly the mean keeps its bias.  Compared as count*E vs T*K in
    integers; the update is one float32 add.
    """
    b = np.asarray(b32, dtype=F32).copy()
    E = b.shape[0]
    c = np.asarray(counts, dtype=np.int64)
    g = F32(gamma)
    over = c * E > T * K
    under = c * E < T * K
    b[over] = (b[over] - g).astype(F32)
    b[under] = (b[under] + g).astype(F32)
    return b


def load_ratio(counts: np.ndarray) -> float:
    """Max over mean per-expert load."""
    c = np.asarray(counts, dtype=F64)
    return float(c.max() / c.mean())


# ----------------------------------------------------------------------------
# complementary sequence-wise balance loss ([V3] §1.4, Eq 17-20)
# ----------------------------------------------------------------------------

@dataclass
class BalanceLoss:
    loss: np.ndarray   # [n_seq] float64: alpha * sum_i f_i P_i
    f: np.ndarray      # [n_seq][E] float64: selection frequency, mean 1 over experts
    P: np.ndarray      # [n_seq][E] float64: mean normalised affinity
    gap: np.ndarray    # [T] float32: K-th minus (K+1)-th raw affinity of each token


def sequence_balance_loss(s32: np.ndarray, topk: int, seq_len: int, alpha: float) -> BalanceLoss:
    """The small sequence-wise balance loss V3 keeps beside the bias.

    [V3] §1.4 (Eq 17-20): for each sequence of seq_len tokens,
      f_i = E / (K * seq_len) * #{t : expert i is in the top-K of token t's
            raw affinities s_t (the bias is not involved)},
      P_i = mean over the sequence of s_{i,t} / sum_j s_{j,t},
      loss = alpha * sum_i f_i * P_i.
    Readings: the top-K is a plain top-K over all experts (no group limit)
    with ties going to the lower index; sequences are consecutive blocks of
    seq_len tokens.
    """
    s = np.asarray(s32, dtype=F32)
    T, E = s.shape
    assert T % seq_len == 0
    order = np.argsort(-s.astype(F64), axis=1, kind="stable")   # descending, lower index first
    top = order[:, :topk]
    kth = np.take_along_axis(s, order[:, topk - 1:topk], axis=1)[:, 0]
    nxt = (np.take_along_axis(s, order[:, topk:topk + 1], axis=1)[:, 0] if topk < E
           else np.full(T, -np.inf, dtype=F32))
    gap = (kth.astype(F64) - nxt.astype(F64)).astype(F32)
    sel = np.zeros((T, E), dtype=np.int64)
    np.put_along_axis(sel, top, 1, axis=1)
    sn = s.astype(F64) / s.astype(F64).sum(axis=1, keepdims=True)
    n_seq = T // seq_len
    counts = sel.reshape(n_seq, seq_len, E).sum(axis=1)
    f = counts.astype(F64) * E / (topk * seq_len)
    P = sn.reshape(n_seq, seq_len, E).mean(axis=1)
    loss = alpha * (f * P).sum(axis=1)
    return BalanceLoss(loss=loss, f=f, P=P, gap=gap)


# ----------------------------------------------------------------------------
# FP8 E4M3 fine-grained quantisation ([V3] §2.2)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """Value of each OCP E4M3FN code (1 sign, 4 exponent bits biased by 7, 3 mantissa bits).

    Exponent field 0 holds subnormals m * 2^-9; field 15 with mantissa 7 is NaN
    (the format has no infinities).
    """
    c = np.asarray(c, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = (c & 0x7).astype(F64)
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(ef.astype(F64) - 7.0))
    val = np.where((ef == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


_E4M3_VALUES = _e4m3_value(np.arange(256))   # the 256 codes' values, looked up by code


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3FN code (``_e4m3_value``), float64."""
    return _E4M3_VALUES[np.asarray(codes).astype(np.uint8)]


def e4m3_quantize(v) -> np.ndarray:
    """Round float32 values to E4M3FN codes: nearest, ties to even, saturating at +-448.

    Values below the smallest subnormal half-step round to signed zero.
    """
    a = np.asarray(v, dtype=F64)
    sign = (np.signbit(a)).astype(np.int64) << 7
    mag = np.abs(a)
    # binade exponent for normals (min normal 2^-6); spacing 2^(e-3); subnormal spacing 2^-9
    _, ex = np.frexp(np.where(mag > 0, mag, 1.0))    # mag = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    step = np.exp2(e.astype(F64) - 3.0)
    q = np.round(mag / step) * step                   # np.round: half to even
    q = np.minimum(q, E4M3_MAX)
    # encode
    _, qex = np.frexp(np.where(q > 0, q, 1.0))
    qe = qex - 1
    normal = q >= 2.0 ** -6
    ef = np.where(normal, qe + 7, 0)
    mant = np.where(normal, np.round((q / np.exp2(qe.astype(F64)) - 1.0) * 8.0),
                    np.round(q / 2.0 ** -9))
    code = sign | (ef.astype(np.int64) << 3) | mant.astype(np.int64)
    return code.astype(np.uint8)


def _tile_scale(amax: np.ndarray) -> np.ndarray:
    """amax / 448 in float32; 1 where that is zero (an all-zero tile, or a
    max-abs so small that the quotient underflows)."""
    sc = (np.asarray(amax, dtype=F32) / F32(448.0)).astype(F32)
    return np.where(sc > 0, sc, F32(1.0)).astype(F32)


def quantize_1x128(a: np.ndarray):
    """Per-row, per-128-column online quantisation of an activation matrix.

    [V3] §2.2: activations are grouped in 1x128 tiles (one token, 128
    channels); each tile's scale comes from its current max-abs value and the
    values are stored as E4M3.  Reading: scale = amax / 448 in float32 (1 for an
    all-zero tile, and wherever amax / 448 rounds to zero); code = RNE(v / scale)
    computed in float32.

    Returns (codes uint8 [R][C], scales float32 [R][C/128]).
    """
    a32 = np.asarray(a, dtype=F32)
    R, C = a32.shape
    t = a32.reshape(R, C // 128, 128)
    scale = _tile_scale(np.abs(t).max(axis=2))
    ratio = (t / scale[:, :, None]).astype(F32)
    return e4m3_quantize(ratio).reshape(R, C), scale


def dequantize_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    R, C = codes.shape
    return (e4m3_decode(codes).reshape(R, C // 128, 128) * scales.astype(F64)[:, :, None]).reshape(R, C)


def fake_quant_1x128(a: np.ndarray) -> np.ndarray:
    """Quantise then dequantise (float64 result): the emulation mode's activation map."""
    q, s = quantize_1x128(np.asarray(a, dtype=F64).astype(F32))
    return dequantize_1x128(q, s)


def quantize_128x1(a: np.ndarray):
    """Per-column, per-128-row quantisation: the 128x1 tiles of [V3] §2.2.

    A product that contracts over tokens (a weight gradient) needs its scales
    to run along the tokens, so each tile is 128 consecutive rows of one
    column.  Same rule as ``quantize_1x128``: scale = amax / 448 in float32 (1
    where that is zero), code = RNE(v / scale) in float32.  Rows are grouped
    from the first; a last partial group holds the remaining rows (zero
    padding would change neither its amax nor any product).

    Returns (codes uint8 [R][C], scales float32 [ceil(R/128)][C]).
    """
    a32 = np.asarray(a, dtype=F32)
    R, C = a32.shape
    codes = np.zeros((R, C), dtype=np.uint8)
    scales = np.ones((-(-R // 128), C), dtype=F32)
    for blk in range(scales.shape[0]):
        t = a32[128 * blk:128 * (blk + 1)]
        sc = _tile_scale(np.abs(t).max(axis=0))
        scales[blk] = sc
        codes[128 * blk:128 * (blk + 1)] = e4m3_quantize((t / sc[None, :]).astype(F32))
    return codes, scales


def fake_quant_128x1(a: np.ndarray) -> np.ndarray:
    """``quantize_128x1`` then dequantise (float64 result)."""
    q, sc = quantize_128x1(np.asarray(a, dtype=F64).astype(F32))
    rows = np.repeat(sc.astype(F64), 128, axis=0)[:q.shape[0]]
    return e4m3_decode(q) * rows


# ----------------------------------------------------------------------------
# error metric
# ----------------------------------------------------------------------------

def max_row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||y_t - ref_t||_2 / ||ref_t||_2."""
    y = np.asarray(y, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return float(np.max(num / np.maximum(den, 1e-300)))
