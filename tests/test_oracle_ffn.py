"""Pins of the oracle's expert FFN and gated combine (brute force and special
cases).  CPU only."""
import numpy as np

import oracle as O
import synthetic as S
from tests import bruteforce as BF


def _tiny(T=64):
    c = S.get_config("tiny", T=T)
    x = O.lift(S.gen_x(c))
    wr = O.lift(S.gen_router(c))
    b = S.gen_bias(c).numpy()
    ex = {e: {k: v.numpy() for k, v in S.gen_expert(c, e).items()} for e in range(c.E + c.S)}
    return c, x, wr, b, ex


def _fwd(c, x, wr, b, ex, **kw):
    return O.forward(x, wr, b, lambda e: ex[e], n_groups=c.n_groups, topk_groups=c.topk_groups,
                     topk=c.topk, group_topn=c.group_topn, n_shared=c.n_shared, **kw)


def test_expert_ffn_matches_scalar_loops():
    c, x, wr, b, ex = _tiny()
    for e in (0, 7, 16):
        wg, wu, wd = O.expert_f64(ex[e])
        Y = O.expert_ffn(x[:3], wg, wu, wd)
        for t in range(3):
            ref = BF.swiglu_loop(x[t], wg, wu, wd)
            np.testing.assert_allclose(Y[t], ref, rtol=1e-12, atol=1e-12)


def test_layer_output_matches_bruteforce_combine():
    c, x, wr, b, ex = _tiny()
    res = _fwd(c, x, wr, b, ex, tokens=[0, 5, 33, 63])
    r = res.routing
    for j, t in enumerate(res.tokens):
        ref = BF.swiglu_loop(x[t], *O.expert_f64(ex[c.E]))          # shared, weight 1
        for k in range(c.topk):
            e = int(r.idx[t, k])
            ref = ref + float(r.gate[t, k]) * BF.swiglu_loop(x[t], *O.expert_f64(ex[e]))
        np.testing.assert_allclose(res.y[j], ref, rtol=1e-11, atol=1e-11)


def test_token_subset_equals_full_rows():
    c, x, wr, b, ex = _tiny()
    full = _fwd(c, x, wr, b, ex)
    sub = _fwd(c, x, wr, b, ex, tokens=[3, 17, 40])
    np.testing.assert_allclose(sub.y, full.y[[3, 17, 40]], rtol=1e-13, atol=1e-13)


def test_zero_routed_experts_leaves_shared_expert_only():
    c, x, wr, b, ex = _tiny()
    ex0 = {e: dict(w) for e, w in ex.items()}
    for e in range(c.E):
        ex0[e]["w_down"] = np.zeros_like(ex0[e]["w_down"])
    res = _fwd(c, x, wr, b, ex0, tokens=[0, 1, 2])
    for j in range(3):
        ref = BF.swiglu_loop(x[j], *O.expert_f64(ex[c.E]))
        np.testing.assert_allclose(res.y[j], ref, rtol=1e-12, atol=1e-12)


def test_single_expert_single_choice_is_the_ffn():
    # one routed expert, K = 1, no shared expert: gate is 1 and y = FFN(x)
    c, x, wr, b, ex = _tiny()
    wr1 = wr[:, :1]
    res = O.forward(x[:4], wr1, np.zeros(1, np.float32), lambda e: ex[e], n_groups=1, topk_groups=1,
                    topk=1, group_topn=1, n_shared=0)
    assert np.all(res.routing.gate == 1.0)
    for t in range(4):
        np.testing.assert_allclose(res.y[t], BF.swiglu_loop(x[t], *O.expert_f64(ex[0])), rtol=1e-12,
                                   atol=1e-12)


def test_output_is_linear_in_down_projections():
    c, x, wr, b, ex = _tiny()
    ex2 = {e: dict(w, w_down=w["w_down"] * 2.0) for e, w in ex.items()}
    y1 = _fwd(c, x, wr, b, ex, tokens=range(8)).y
    y2 = _fwd(c, x, wr, b, ex2, tokens=range(8)).y
    np.testing.assert_array_equal(y2, 2.0 * y1)


def test_residual_is_added_when_given():
    c, x, wr, b, ex = _tiny()
    y1 = _fwd(c, x, wr, b, ex, tokens=[1, 2]).y
    y2 = _fwd(c, x, wr, b, ex, tokens=[1, 2], residual=x).y
    np.testing.assert_allclose(y2 - y1, x[[1, 2]], rtol=0, atol=1e-12)


def test_silu_special_values():
    v = np.array([0.0, 40.0, -40.0, 1.0])
    out = O.silu(v)
    assert out[0] == 0.0 and abs(out[1] - 40.0) < 1e-12 and abs(out[2]) < 1e-15
    assert abs(out[3] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
