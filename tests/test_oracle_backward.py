"""Pins of the oracle's layer backward (page "02 · DeepSeek-V3", §1.3 Eq 12-15,
§1.4, §2.2).  CPU only.

- Central finite differences of ``layer_fixed_routing`` (float64) along random
  directions in x, W_r and each expert matrix: the difference quotient equals
  <gradient, direction> up to O(eps^2).
- torch CPU autograd (float64) of the fixed-routing layer: every element of
  every gradient.
- One routed expert per token: the gate is identically 1, so the router gets
  exactly zero gradient.
- Linearity in dy; a uniform bias shift (same selection) changes no gradient.
"""
import numpy as np
import pytest

import oracle as O
from tests import test_oracle_ffn as TF


def _bwd(c, x, wr, b, ex, dy, **kw):
    return O.backward(x, wr, b, lambda e: ex[e], dy, n_groups=c.n_groups,
                      topk_groups=c.topk_groups, topk=c.topk, group_topn=c.group_topn,
                      n_shared=c.n_shared, **kw)


def _setup(T=16, seed=7, **cfg):
    c, x, wr, b, ex = TF._tiny(T)
    if cfg:
        c = c.with_(**cfg)
    dy = np.random.default_rng(seed).standard_normal(x.shape)
    return c, x, wr, b, ex, dy


def _f64_experts(ex):
    return {e: {k: O.lift(v) for k, v in w.items()} for e, w in ex.items()}


def test_fixed_routing_layer_matches_forward():
    c, x, wr, b, ex, dy = _setup()
    fw = TF._fwd(c, x, wr, b, ex)
    y = O.layer_fixed_routing(x, wr, fw.routing.idx.astype(np.int64), lambda e: ex[e], c.n_shared)
    # the forward rounds logits and affinities to float32; nothing else differs
    err = np.abs(y - fw.y).max() / np.abs(fw.y).max()
    assert err < 1e-6, err


@pytest.mark.parametrize("which", ["x", "w_router", "w_gate", "w_up", "w_down", "shared_w_down"])
def test_directional_derivatives_match_finite_differences(which):
    c, x, wr, b, ex, dy = _setup()
    res = _bwd(c, x, wr, b, ex, dy)
    idx = res.routing.idx.astype(np.int64)
    ex64 = _f64_experts(ex)
    rng = np.random.default_rng(11)
    e = int(idx[0, 0]) if not which.startswith("shared") else c.E
    name = which.replace("shared_", "")

    def loss(xx, ww, ee):
        return float((dy * O.layer_fixed_routing(xx, ww, idx, lambda k: ee[k], c.n_shared)).sum())

    if which == "x":
        v = rng.standard_normal(x.shape)
        an = float((res.dx * v).sum())
        f = lambda h: loss(x + h * v, wr, ex64)
    elif which == "w_router":
        v = rng.standard_normal(wr.shape) / 16
        an = float((res.dw_router * v).sum())
        f = lambda h: loss(x, wr + h * v, ex64)
    else:
        j = {"w_gate": 0, "w_up": 1, "w_down": 2}[name]
        v = rng.standard_normal(ex64[e][name].shape) / 16
        an = float((res.dw[e][j] * v).sum())

        def f(h):
            ee = dict(ex64)
            ee[e] = dict(ex64[e])
            ee[e][name] = ex64[e][name] + h * v
            return loss(x, wr, ee)
    eps = 1e-5
    fd = (f(eps) - f(-eps)) / (2 * eps)
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_gradients_match_torch_autograd():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    c, x, wr, b, ex, dy = _setup(T=24)
    res = _bwd(c, x, wr, b, ex, dy)
    idx = torch.tensor(res.routing.idx.astype(np.int64))
    X = torch.tensor(x, requires_grad=True)
    WR = torch.tensor(wr, requires_grad=True)
    W = {e: [torch.tensor(m, requires_grad=True) for m in O.expert_f64(ex[e])]
         for e in range(c.E + c.n_shared)}
    s = torch.sigmoid(X @ WR)
    ssel = s.gather(1, idx)
    g = ssel / ssel.sum(dim=1, keepdim=True)

    def ffn(Xe, w):
        return (F.silu(Xe @ w[0].T) * (Xe @ w[1].T)) @ w[2].T
    y = ffn(X, W[c.E])
    for e in range(c.E):
        mask = (idx == e)
        ge = (g * mask).sum(dim=1, keepdim=True)
        y = y + ge * ffn(X, W[e])
    np.testing.assert_allclose(y.detach().numpy(), O.layer_fixed_routing(
        x, wr, idx.numpy(), lambda e: ex[e], c.n_shared), rtol=1e-12, atol=1e-12)
    (torch.tensor(dy) * y).sum().backward()
    np.testing.assert_allclose(res.dx, X.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(res.dw_router, WR.grad.numpy(), rtol=1e-10, atol=1e-11)
    for e in range(c.E + c.n_shared):
        for j in range(3):
            np.testing.assert_allclose(res.dw[e][j], W[e][j].grad.numpy(), rtol=1e-10, atol=1e-11,
                                       err_msg=f"expert {e} matrix {j}")


def test_one_routed_expert_gives_no_router_gradient():
    c, x, wr, b, ex, dy = _setup(topk=1, topk_groups=4)
    res = _bwd(c, x, wr, b, ex, dy)
    assert np.all(res.dlogit == 0.0)
    assert np.all(res.dw_router == 0.0)


def test_backward_is_linear_in_dy():
    c, x, wr, b, ex, dy = _setup()
    dy2 = np.random.default_rng(3).standard_normal(x.shape)
    a = _bwd(c, x, wr, b, ex, dy)
    bb = _bwd(c, x, wr, b, ex, dy2)
    ab = _bwd(c, x, wr, b, ex, 2.0 * dy + dy2)
    np.testing.assert_allclose(ab.dx, 2 * a.dx + bb.dx, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(ab.dw_router, 2 * a.dw_router + bb.dw_router, rtol=1e-10, atol=1e-11)
    for e in a.dw:
        for j in range(3):
            np.testing.assert_allclose(ab.dw[e][j], 2 * a.dw[e][j] + bb.dw[e][j], rtol=1e-10, atol=1e-11)


def test_uniform_bias_shift_changes_no_gradient():
    c, x, wr, b, ex, dy = _setup()
    a = _bwd(c, x, wr, b, ex, dy)
    s = _bwd(c, x, wr, (b + np.float32(0.25)).astype(np.float32), ex, dy)
    assert np.array_equal(a.routing.idx, s.routing.idx)
    np.testing.assert_array_equal(a.dx, s.dx)
    np.testing.assert_array_equal(a.dw_router, s.dw_router)


@pytest.mark.parametrize("gexp", [[3, "shared"], [3], []])
def test_subsets_equal_full_result(gexp):
    c, x, wr, b, ex, dy = _setup()
    gexp = [c.E if e == "shared" else e for e in gexp]
    full = _bwd(c, x, wr, b, ex, dy)
    sub = _bwd(c, x, wr, b, ex, dy, tokens=[2, 9], grad_experts=gexp, router_cols=[5])
    np.testing.assert_allclose(sub.dx, full.dx[[2, 9]], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sub.dw_router[:, 5], full.dw_router[:, 5], rtol=1e-12, atol=1e-13)
    for e in gexp:
        for j in range(3):
            np.testing.assert_allclose(sub.dw[e][j], full.dw[e][j], rtol=1e-12, atol=1e-13)
