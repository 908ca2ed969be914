"""Each plausible mistake planted in the oracle (on the CPU) must fail a pin.

The mistakes are patched into the oracle module for the duration of one call
of an existing pin test; the test then must raise AssertionError.
"""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as M
from tests import test_oracle_backward as TBW
from tests import test_oracle_backward_fp8 as TB8
from tests import test_oracle_balance as TB
from tests import test_oracle_ffn as TF
from tests import test_oracle_fp8 as T8
from tests import test_oracle_fp8_forward as T8F
from tests import test_oracle_routing as TR


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(M, name, fn)
    monkeypatch.setattr(oracle, name, fn)


_orig = {n: getattr(M, n) for n in ("group_scores", "biased_scores", "gate_values", "permute",
                                     "expert_ffn", "bias_update", "router_affinity",
                                     "e4m3_quantize", "select_experts",
                                     "sequence_balance_loss", "dsilu", "gate_backward",
                                     "expert_backward", "expert_swiglu_input_fp8",
                                     "expert_ffn_fp8", "forward")}


def m_group_top1(z, n_groups, group_topn):
    return _orig["group_scores"](z, n_groups, 1)


def m_no_bias(s, b):
    return s.astype(np.float32)


def m_gate_biased(s, idx):
    return _orig["gate_values"]((s + np.float32(0.1)).astype(np.float32), idx)


def m_gate_all_experts(s, idx):
    sel = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), axis=1)
    return (sel / s.astype(np.float64).sum(axis=1, keepdims=True)).astype(np.float32)


def m_perm_reversed(idx, E):
    p = _orig["permute"](idx, E)
    for e in range(E):
        a, b = p.offsets[e], p.offsets[e + 1]
        p.perm[a:b] = p.perm[a:b][::-1].copy()
    return p


def m_ffn_swapped(X, wg, wu, wd):
    return _orig["expert_ffn"](X, wu, wg, wd)


def m_bias_sign(b, counts, T, K, gamma):
    return _orig["bias_update"](b, counts, T, K, -gamma)


def m_bias_ge(b, counts, T, K, gamma):
    bb = np.asarray(b, np.float32).copy()
    c = np.asarray(counts) * len(bb)
    bb[c >= T * K] -= np.float32(gamma)
    bb[c < T * K] += np.float32(gamma)
    return bb.astype(np.float32)


def m_sigmoid_sign(x, wr):
    L, s = _orig["router_affinity"](x, wr)
    return L, (1.0 / (1.0 + np.exp(L.astype(np.float64)))).astype(np.float32)


def m_round_away(v):
    a = np.asarray(v, np.float64)
    return _orig["e4m3_quantize"](a + np.sign(a) * np.abs(a) * 2.0 ** -20)


def m_select_ascending(s, b, n_groups, topk_groups, topk, group_topn=2):
    return _orig["select_experts"](-s, -b, n_groups, topk_groups, topk, group_topn)


def m_bal_raw_P(s, K, seq_len, alpha):
    r = _orig["sequence_balance_loss"](s, K, seq_len, alpha)
    T, E = s.shape
    P = np.asarray(s, np.float64).reshape(T // seq_len, seq_len, E).mean(axis=1)
    return M.BalanceLoss(loss=alpha * (r.f * P).sum(axis=1), f=r.f, P=P, gap=r.gap)


def m_bal_no_scale(s, K, seq_len, alpha):
    r = _orig["sequence_balance_loss"](s, K, seq_len, alpha)
    f = r.f * K / s.shape[1]
    return M.BalanceLoss(loss=alpha * (f * r.P).sum(axis=1), f=f, P=r.P, gap=r.gap)


def m_bal_smallest(s, K, seq_len, alpha):
    r = _orig["sequence_balance_loss"](s, K, seq_len, alpha)
    f = _orig["sequence_balance_loss"]((1 - np.asarray(s, np.float32)), K, seq_len, alpha).f
    return M.BalanceLoss(loss=alpha * (f * r.P).sum(axis=1), f=f, P=r.P, gap=r.gap)


def m_dsilu_sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def m_gate_bwd_uncentred(ssel, dg):
    S = ssel.sum(axis=1, keepdims=True)
    return dg / S * ssel * (1.0 - ssel)


def m_expert_bwd_swapped(X, dY, wg, wu, wd):
    dX, dwg, dwu, dwd = _orig["expert_backward"](X, dY, wg, wu, wd)
    return dX, dwu, dwg, dwd


def m_fp8_wgrad_dy_1x128(X, dY, wg, wu, wd):
    # dW_down from 1x128 tiles of dY (the dgrad grouping) instead of 128x1
    _, Gc, Uc = _orig["expert_swiglu_input_fp8"](X, wg, wu)
    A = M.silu(Gc)
    dH = M.fake_quant_1x128(dY) @ wd
    dU, dG = dH * A, dH * Uc * M.dsilu(Gc)
    dX = M.fake_quant_1x128(dG) @ wg + M.fake_quant_1x128(dU) @ wu
    Xr = M.fake_quant_128x1(X)
    return (dX, M.fake_quant_128x1(dG).T @ Xr, M.fake_quant_128x1(dU).T @ Xr,
            M.fake_quant_1x128(dY).T @ M.fake_quant_128x1(A * Uc))


def m_fp8_dgrad_dy_exact(X, dY, wg, wu, wd):
    # dH from the unquantised dY
    _, Gc, Uc = _orig["expert_swiglu_input_fp8"](X, wg, wu)
    A = M.silu(Gc)
    dH = dY @ wd
    dU, dG = dH * A, dH * Uc * M.dsilu(Gc)
    dX = M.fake_quant_1x128(dG) @ wg + M.fake_quant_1x128(dU) @ wu
    Xr = M.fake_quant_128x1(X)
    return (dX, M.fake_quant_128x1(dG).T @ Xr, M.fake_quant_128x1(dU).T @ Xr,
            M.fake_quant_128x1(dY).T @ M.fake_quant_128x1(A * Uc))


def m_q128x1_per_row(a):
    # amax taken along each row of a tile instead of down each column
    a32 = np.asarray(a, dtype=np.float32)
    R, C = a32.shape
    codes = np.zeros((R, C), dtype=np.uint8)
    scales = np.ones((-(-R // 128), C), dtype=np.float32)
    for blk in range(scales.shape[0]):
        t = a32[128 * blk:128 * (blk + 1)]
        amax = np.abs(t).max(axis=1, keepdims=True)
        sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        scales[blk] = sc.max()
        codes[128 * blk:128 * (blk + 1)] = M.e4m3_quantize((t / sc).astype(np.float32))
    return codes, scales


def m_fp8_quant_u_not_h(Xq, wg, wu, wd, act_quant=None):
    # the up projection quantised instead of the SwiGLU output
    q = M.fake_quant_1x128 if act_quant is None else act_quant
    return (M.silu(Xq @ wg.T) * q(Xq @ wu.T)).astype(np.float32).astype(np.float64) @ wd.T


def m_fp8_h_128x1(Xq, wg, wu, wd, act_quant=None):
    # H quantised in 128x1 tiles (down the token rows) instead of 1x128
    Hh = (M.silu(Xq @ wg.T) * (Xq @ wu.T)).astype(np.float32).astype(np.float64)
    return M.fake_quant_128x1(Hh) @ wd.T


def m_fp8_no_input_quant(*a, **kw):
    # the layer input x left unquantised (only H goes through the quantiser)
    q = kw.get("act_quant")
    if q is not None:
        H = a[0].shape[1]
        kw["act_quant"] = lambda v: v if v.shape[1] == H else q(v)
    return _orig["forward"](*a, **kw)


CASES = [
    ("group_scores", m_group_top1, TR.test_selection_matches_subset_enumeration, (0,)),
    ("biased_scores", m_no_bias, TR.test_large_bias_forces_and_excludes_experts, ()),
    ("gate_values", m_gate_biased, TR.test_bias_changes_selection_not_gate_values, ()),
    ("gate_values", m_gate_all_experts, TR.test_gates_sum_to_one_and_are_positive, ()),
    ("permute", m_perm_reversed, TR.test_permutation_matches_per_expert_listing, ()),
    ("expert_ffn", m_ffn_swapped, TF.test_expert_ffn_matches_scalar_loops, ()),
    ("bias_update", m_bias_sign, TR.test_bias_update_golden_example, ()),
    ("bias_update", m_bias_ge, TR.test_bias_update_golden_example, ()),
    ("router_affinity", m_sigmoid_sign, TR.test_sigmoid_matches_scipy_expit, ()),
    ("e4m3_quantize", m_round_away, T8.test_midpoints_round_to_even_and_saturate, ()),
    ("select_experts", m_select_ascending, TR.test_plain_topk_when_all_groups_kept, ()),
    ("sequence_balance_loss", m_bal_raw_P, TB.test_balanced_selection_gives_alpha, ()),
    ("sequence_balance_loss", m_bal_no_scale, TB.test_balanced_selection_gives_alpha, ()),
    ("sequence_balance_loss", m_bal_smallest, TB.test_concentrated_routing_is_penalised, ()),
    ("dsilu", m_dsilu_sigmoid, TBW.test_directional_derivatives_match_finite_differences, ("x",)),
    ("gate_backward", m_gate_bwd_uncentred, TBW.test_directional_derivatives_match_finite_differences,
     ("w_router",)),
    ("expert_backward", m_expert_bwd_swapped, TBW.test_gradients_match_torch_autograd, ()),
    ("expert_backward_fp8", m_fp8_wgrad_dy_1x128,
     TB8.test_doubling_a_dy_column_doubles_that_row_of_dw_down, ()),
    ("expert_backward_fp8", m_fp8_dgrad_dy_exact,
     TB8.test_a_substep_change_of_dy_moves_no_weight_gradient, ()),
    ("quantize_128x1", m_q128x1_per_row, TB8.test_quantize_128x1_is_1x128_of_the_transpose, ()),
    ("expert_ffn_fp8", m_fp8_quant_u_not_h, T8F.test_emulation_matches_scalar_loop_quantisation,
     (T8F.FP8_TINY,)),
    ("expert_ffn_fp8", m_fp8_h_128x1, T8F.test_emulation_matches_scalar_loop_quantisation,
     (T8F.FP8_TINY,)),
    ("forward", m_fp8_no_input_quant, T8F.test_emulation_matches_scalar_loop_quantisation,
     (T8F.FP8_TINY,)),
]


@pytest.mark.parametrize("name,fn,pin,args", CASES, ids=[f"{c[0]}:{c[1].__name__}" for c in CASES])
def test_planted_mistake_fails_a_pin(monkeypatch, name, fn, pin, args):
    _patch(monkeypatch, name, fn)
    with pytest.raises(AssertionError):
        pin(*args)


def test_dropped_shared_expert_fails_combine_pin(monkeypatch):
    orig_forward = M.forward

    def no_shared(*a, **kw):
        kw["n_shared"] = 0
        return orig_forward(*a, **kw)

    monkeypatch.setattr(M, "forward", no_shared)
    monkeypatch.setattr(oracle, "forward", no_shared)
    with pytest.raises(AssertionError):
        TF.test_layer_output_matches_bruteforce_combine()
