"""Pins of the oracle's routing steps (router, node-limited selection, gates,
permutation, bias update) against brute force, library routines, invariants
and the pages' stated rules.  CPU only."""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle as O
import synthetic as S
from tests import bruteforce as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_inputs(T=64, seed_cfg="tiny"):
    c = S.get_config(seed_cfg, T=T)
    x = O.lift(S.gen_x(c))
    wr = O.lift(S.gen_router(c))
    b = S.gen_bias(c).numpy()
    return c, x, wr, b


def _route(c, x, wr, b):
    return O.route(x, wr, b, n_groups=c.n_groups, topk_groups=c.topk_groups, topk=c.topk,
                   group_topn=c.group_topn)


# --------------------------------------------------------------------------- router


def test_router_logits_match_loop_bruteforce():
    c, x, wr, b = _tiny_inputs(T=6)
    L, s = O.router_affinity(x, wr)
    Lb = BF.logits_loop(x, wr)
    # both are a float64 sum rounded once to float32; summation order may move
    # the rounding boundary by at most one float32 ulp
    assert np.all(np.abs(L.astype(np.float64) - Lb) <= np.spacing(np.abs(Lb)))


def test_sigmoid_matches_scipy_expit():
    c, x, wr, b = _tiny_inputs()
    L, s = O.router_affinity(x, wr)
    ref = scipy.special.expit(L.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(s, ref)
    assert np.all((s > 0) & (s < 1))


# --------------------------------------------------------------------------- selection


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_selection_matches_subset_enumeration(seed):
    c = S.get_config("tiny", seed=seed)
    x = O.lift(S.gen_x(c))
    wr = O.lift(S.gen_router(c))
    b = S.gen_bias(c).numpy()
    L, s, r, p = _route(c, x, wr, b)
    checked = 0
    for t in range(c.T):
        if r.flagged[t]:
            continue
        idx, groups, gs = BF.select_enumerate(r.z[t], c.n_groups, c.topk_groups, c.topk, c.group_topn)
        assert list(r.idx[t]) == idx, t
        assert sorted(r.groups[t]) == groups, t
        np.testing.assert_allclose(r.group_score[t].astype(np.float64), gs, rtol=0, atol=1e-7)
        checked += 1
    assert checked >= c.T - 2


def test_selection_at_v3_shape_matches_enumeration_on_sample():
    # V3 grouping: 256 experts in 8 groups of 32, keep 4, top-8 (C(128,8) is
    # too many subsets, so the expert stage enumerates the greedy-equivalent
    # top-8 through pairwise exchange optimality instead)
    c = S.get_config("decode", T=32)
    x = O.lift(S.gen_x(c))
    wr = O.lift(S.gen_router(c))
    b = (np.arange(256, dtype=np.float32) % 7 - 3) * np.float32(0.002)
    L, s, r, p = _route(c, x, wr, b)
    for t in range(c.T):
        if r.flagged[t]:
            continue
        z = r.z[t].astype(np.float64)
        gs = [max(z[g * 32 + i] + z[g * 32 + j] for i in range(32) for j in range(i + 1, 32))
              for g in range(8)]
        gs_rank = sorted(range(8), key=lambda g: (-gs[g], g))
        kept = sorted(gs_rank[:4])
        assert sorted(r.groups[t]) == kept
        elig = [e for g in kept for e in range(g * 32, g * 32 + 32)]
        chosen = set(int(e) for e in r.idx[t])
        assert chosen <= set(elig)
        # exchange optimality: no unchosen eligible expert beats a chosen one
        worst_in = min(z[e] for e in chosen)
        best_out = max(z[e] for e in elig if e not in chosen)
        assert worst_in > best_out


def test_plain_topk_when_all_groups_kept():
    # special case: keeping every group reduces the method to a plain top-K of z
    c, x, wr, b = _tiny_inputs()
    L, s = O.router_affinity(x, wr)
    r = O.select_experts(s, b, n_groups=4, topk_groups=4, topk=4)
    z = (s + b[None, :]).astype(np.float32)
    ref = np.sort(np.argsort(-z.astype(np.float64), axis=1, kind="stable")[:, :4], axis=1)
    np.testing.assert_array_equal(r.idx, ref)
    r1 = O.select_experts(s, b, n_groups=1, topk_groups=1, topk=4, group_topn=2)
    np.testing.assert_array_equal(r1.idx, ref)


def test_selected_experts_inside_kept_groups_v3():
    c = S.get_config("prefill", T=512)
    x = O.lift(S.gen_x(c))
    wr = O.lift(S.gen_router(c))
    b = S.gen_bias(c).numpy()
    L, s, r, p = _route(c, x, wr, b)
    grp = r.idx // 32
    for t in range(c.T):
        assert set(grp[t]) <= set(r.groups[t])
        assert len(set(grp[t])) <= 4
    assert r.idx.shape == (512, 8)
    assert np.all(np.diff(r.idx, axis=1) > 0)          # ascending, distinct


def test_exact_ties_go_to_lower_index():
    s = np.full((1, 16), 0.5, dtype=np.float32)
    b = np.zeros(16, dtype=np.float32)
    r = O.select_experts(s, b, n_groups=4, topk_groups=2, topk=4)
    assert list(r.groups[0]) == [0, 1]
    assert list(r.idx[0]) == [0, 1, 2, 3]
    assert r.flagged[0]


# --------------------------------------------------------------------------- gates


def test_gates_sum_to_one_and_are_positive():
    for name, T in (("tiny", 64), ("decode", 64)):
        c, x, wr, b = _tiny_inputs(T=T, seed_cfg=name)
        L, s, r, p = _route(c, x, wr, b)
        assert np.all(np.abs(r.gate.astype(np.float64).sum(axis=1) - 1.0) <= 1e-6)
        assert np.all(r.gate > 0)


def test_bias_changes_selection_not_gate_values():
    c, x, wr, b = _tiny_inputs()
    L, s = O.router_affinity(x, wr)
    r0 = O.select_experts(s, np.zeros(16, np.float32), 4, 2, 4)
    r1 = O.select_experts(s, b, 4, 2, 4)
    assert np.any(r0.idx != r1.idx)               # the bias moves some selections
    same = np.all(r0.idx == r1.idx, axis=1)
    assert same.sum() > 0
    np.testing.assert_array_equal(r0.gate[same], r1.gate[same])
    # gates depend on the unbiased affinities only: proportional to s of the chosen
    sel = np.take_along_axis(s.astype(np.float64), r1.idx.astype(np.int64), axis=1)
    ratio = r1.gate.astype(np.float64) / sel
    assert np.all(np.abs(ratio / ratio[:, :1] - 1.0) < 1e-6)


def test_large_bias_forces_and_excludes_experts():
    c, x, wr, b = _tiny_inputs()
    L, s = O.router_affinity(x, wr)
    b2 = np.zeros(16, np.float32)
    b2[[5, 6, 9, 11]] = 10.0           # groups 1 and 2
    b2[0] = -10.0
    r = O.select_experts(s, b2, 4, 2, 4)
    assert np.all(r.idx == np.array([5, 6, 9, 11]))
    ref = s[:, [5, 6, 9, 11]].astype(np.float64)
    np.testing.assert_allclose(r.gate, ref / ref.sum(axis=1, keepdims=True), rtol=1e-7)


def test_raising_bias_never_drops_an_expert():
    c, x, wr, b = _tiny_inputs()
    L, s = O.router_affinity(x, wr)
    r = O.select_experts(s, b, 4, 2, 4)
    for e in range(16):
        bb = b.copy()
        bb[e] = np.float32(bb[e] + np.float32(0.05))
        r2 = O.select_experts(s, bb, 4, 2, 4)
        had = np.any(r.idx == e, axis=1) & ~r.flagged & ~r2.flagged
        has = np.any(r2.idx == e, axis=1)
        assert np.all(has[had])


# --------------------------------------------------------------------------- permutation


def test_permutation_matches_per_expert_listing():
    c, x, wr, b = _tiny_inputs()
    L, s, r, p = _route(c, x, wr, b)
    T, K = r.idx.shape
    assert p.counts.sum() == T * K                       # nothing dropped
    np.testing.assert_array_equal(p.counts, np.bincount(r.idx.ravel(), minlength=16))
    rows = []
    for e in range(16):
        toks = [t for t in range(T) if e in list(r.idx[t])]
        assert list(p.perm[p.offsets[e]:p.offsets[e + 1]]) == toks
        rows += toks
    assert len(rows) == T * K
    # slot is the inverse: assignment t*K+k sits at row slot, whose token is t
    for t in range(T):
        for k in range(K):
            row = p.slot[t * K + k]
            assert p.perm[row] == t
            assert p.offsets[r.idx[t, k]] <= row < p.offsets[r.idx[t, k] + 1]
    assert sorted(p.slot.tolist()) == list(range(T * K))


# --------------------------------------------------------------------------- bias update


def test_bias_update_golden_example():
    g = json.load(open(os.path.join(GOLDEN, "bias_update_example.json")))
    for st in g["steps"]:
        out = O.bias_update(np.array(st["bias_in"], np.float32), np.array(st["counts"]), g["T"], g["K"],
                            g["gamma"])
        assert out.dtype == np.float32
        np.testing.assert_allclose(out, st["bias_out"], rtol=0, atol=1e-9)
    # from zero the step is exactly the float32 gamma
    out = O.bias_update(np.zeros(4, np.float32), np.array([4, 0, 2, 2]), 4, 2, 1e-3)
    assert out[0] == -np.float32(1e-3) and out[1] == np.float32(1e-3) and out[2] == 0.0


def test_bias_update_moves_toward_balance_on_skew():
    c = S.get_config("skew", T=512)
    x = O.lift(S.gen_x(c))
    wr = O.lift(S.gen_router(c))
    b = np.zeros(256, np.float32)
    L, s, r, p = _route(c, x, wr, b)
    ratio0 = O.load_ratio(p.counts)
    assert ratio0 > 5.0                              # Zipf offsets skew the load
    b1 = O.bias_update(b, p.counts, c.T, c.topk, c.gamma)
    hot = int(np.argmax(p.counts))
    assert b1[hot] < 0
    assert np.all(np.abs(b1) == np.float32(1e-3)) or np.any(p.counts * 256 == c.T * 8)
    assert O.load_ratio(np.full(256, 16)) == 1.0
    assert O.load_ratio(p.counts) >= 1.0


# --------------------------------------------------------------------------- goldens from the pages


def test_v3_shapes_and_parameter_count():
    g = json.load(open(os.path.join(GOLDEN, "v3_layer_shapes.json")))
    c = S.get_config("decode")
    assert (c.hidden, c.inter, c.n_experts, c.n_shared, c.topk) == (
        g["hidden"], g["expert_intermediate"], g["routed_experts"], g["shared_experts"],
        g["routed_per_token"])
    assert c.topk_groups == g["max_nodes_per_token"] and c.n_groups == g["nodes"]
    assert c.n_experts // c.n_groups == g["gpus"] // g["nodes"] * g["experts_per_gpu"]
    assert c.group_topn == g["top_affinities_per_node"]
    w = S.gen_expert(c, 0)
    n = sum(v.numel() for v in w.values())
    assert n == S.expert_param_count(c)
    assert n == 44_040_192
    assert round(n / 1e6, 1) == g["expert_params_millions_rounded"]
    active = g["active_experts_per_layer"] * n
    assert active == 396_361_728
    assert round(active / 1e6) == g["active_expert_params_per_layer_millions_rounded"]
    assert round(active * g["moe_layers"] / 1e9, 1) == g["active_expert_params_all_layers_billions_rounded"]
    # bf16 bytes of all 257 experts of one layer
    assert 257 * n * 2 == 22_636_658_688
