"""Pins of the oracle's E4M3 backward emulation (page "02 · DeepSeek-V3",
§2.2: 1x128 activation tiles, 128x1 tiles where a product contracts over
tokens, the SwiGLU input cached in E4M3 and its output recomputed).  CPU only.

- ``quantize_128x1`` is ``quantize_1x128`` of the transpose (that quantiser is
  pinned against all 256 codes and torch's float8_e4m3fn).
- With both quantisers replaced by the identity, the emulation is the plain
  backward, which finite differences and torch autograd pin.
- Token isolation: 1x128 tiles never mix tokens, so one token's dy moves no
  other token's dx.
- 128x1 tiles of dY: doubling one column of dy doubles exactly that row of
  every dW_down (its tile scales double, its codes stay) and leaves the other
  rows bit for bit.
- Quantisation absorbs a change below one E4M3 step of an element that is no
  tile's maximum: every weight gradient stays bit for bit, while the exact
  backward moves.
"""
import numpy as np
import pytest

import oracle as O
import oracle.moe_oracle as M
from tests import test_oracle_backward as TBW


def _bwd(c, x, wr, b, ex, dy, **kw):
    return TBW._bwd(c, x, wr, b, ex, dy, fp8_emulation=True, **kw)


def test_quantize_128x1_is_1x128_of_the_transpose():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((300, 256)).astype(np.float32)
    a[:, 5] = 0.0                      # an all-zero column: scale 1, codes 0
    a[17, 9] = 4000.0                  # an outlier in the first row tile of column 9
    a[250:, 11] *= 1e-30               # a tiny last tile
    q, s = O.quantize_128x1(a)
    assert q.shape == (300, 256) and s.shape == (3, 256)
    at = np.zeros((256, 384), dtype=np.float32)
    at[:, :300] = a.T
    qt, st = O.quantize_1x128(at)
    np.testing.assert_array_equal(q, qt[:, :300].T)
    np.testing.assert_array_equal(s, st.T)


def test_identity_quantisers_give_the_exact_backward(monkeypatch):
    c, x, wr, b, ex, dy = TBW._setup(T=24)
    ref = TBW._bwd(c, x, wr, b, ex, dy)
    ident = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    monkeypatch.setattr(M, "fake_quant_1x128", ident)
    monkeypatch.setattr(M, "fake_quant_128x1", ident)
    got = _bwd(c, x, wr, b, ex, dy)
    np.testing.assert_allclose(got.dx, ref.dx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got.dw_router, ref.dw_router, rtol=1e-12, atol=1e-14)
    for e in ref.dw:
        for g, r in zip(got.dw[e], ref.dw[e]):
            np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-14)


def test_one_tokens_dy_moves_no_other_tokens_dx():
    c, x, wr, b, ex, dy = TBW._setup(T=24)
    base = _bwd(c, x, wr, b, ex, dy, grad_experts=[])
    dy2 = dy.copy()
    dy2[5] = 30.0 * np.random.default_rng(11).standard_normal(dy.shape[1])
    got = _bwd(c, x, wr, b, ex, dy2, grad_experts=[])
    others = np.arange(c.T) != 5
    np.testing.assert_array_equal(got.dx[others], base.dx[others])
    assert not np.array_equal(got.dx[5], base.dx[5])


def test_doubling_a_dy_column_doubles_that_row_of_dw_down():
    c, x, wr, b, ex, dy = TBW._setup(T=24)
    h0 = 37
    base = _bwd(c, x, wr, b, ex, dy)
    dy2 = dy.copy()
    dy2[:, h0] *= 2.0
    got = _bwd(c, x, wr, b, ex, dy2)
    rest = np.arange(c.hidden) != h0
    n = 0
    for e, (_, _, dwd) in base.dw.items():
        gd = got.dw[e][2]
        np.testing.assert_array_equal(gd[h0], 2.0 * dwd[h0])
        np.testing.assert_array_equal(gd[rest], dwd[rest])
        n += bool(np.any(dwd[h0] != 0))
    assert n >= 4


def _quiet_element(c, x, wr, b, dy, t0):
    """A column h of token t0 whose dy value is the maximum of none of the
    tiles holding it: its 1x128 slice, and the 128x1 column tile of dY in
    every expert t0 is routed to (the shared expert's included)."""
    _, _, r, _ = O.route(x, wr, b, n_groups=c.n_groups, topk_groups=c.topk_groups, topk=c.topk,
                         group_topn=c.group_topn)
    s = 1.0 / (1.0 + np.exp(-(x @ wr)))
    ssel = np.take_along_axis(s, r.idx.astype(np.int64), axis=1)
    g = ssel / ssel.sum(axis=1, keepdims=True)
    order = np.argsort(np.abs(dy[t0]))
    for h in order[len(order) // 4:]:           # skip the smallest (sub-normal codes)
        sl = slice(128 * (h // 128), 128 * (h // 128) + 128)
        if np.abs(dy[t0, sl]).max() == abs(dy[t0, h]):
            continue
        ok = np.abs(dy[:, h]).max() > abs(dy[t0, h])           # shared: dY = dy
        for k, e in enumerate(r.idx[t0]):
            tt, kk = np.nonzero(r.idx == e)
            col = np.abs(g[tt, kk] * dy[tt, h])
            ok &= col.max() > abs(g[t0, k] * dy[t0, h])
        if ok:
            return int(h)
    raise AssertionError("no quiet element")


def test_a_substep_change_of_dy_moves_no_weight_gradient():
    c, x, wr, b, ex, dy = TBW._setup(T=24)
    t0 = 3
    h0 = _quiet_element(c, x, wr, b, dy, t0)
    dy2 = dy.copy()
    dy2[t0, h0] *= 1.0 + 1e-5                   # far below an E4M3 step, above float32's
    base = _bwd(c, x, wr, b, ex, dy)
    got = _bwd(c, x, wr, b, ex, dy2)
    for e in base.dw:
        for gm, bm in zip(got.dw[e], base.dw[e]):
            np.testing.assert_array_equal(gm, bm)
    exact0 = TBW._bwd(c, x, wr, b, ex, dy)
    exact1 = TBW._bwd(c, x, wr, b, ex, dy2)
    assert not np.array_equal(exact0.dw[c.E][2], exact1.dw[c.E][2])


@pytest.mark.parametrize("T", [24, 200])
def test_emulation_stays_within_e4m3_error_of_the_exact_backward(T):
    c, x, wr, b, ex, dy = TBW._setup(T=T)
    ref = TBW._bwd(c, x, wr, b, ex, dy)
    got = _bwd(c, x, wr, b, ex, dy)
    rel = lambda a, r: np.linalg.norm(a - r) / np.linalg.norm(r)  # noqa: E731
    errs = [rel(got.dx, ref.dx), rel(got.dw_router, ref.dw_router)]
    errs += [rel(gm, rm) for e in ref.dw for gm, rm in zip(got.dw[e], ref.dw[e])
             if np.linalg.norm(rm) > 0]
    # E4M3 keeps 3 mantissa bits (relative step 2^-3 .. 2^-4): each product sees
    # a few percent, never the exact result and never an order-one error
    assert 1e-3 < min(errs) and max(errs) < 0.15, (min(errs), max(errs))
