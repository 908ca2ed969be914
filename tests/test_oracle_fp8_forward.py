"""Pins of the oracle's E4M3 forward emulation (``forward(act_quant=...)``,
``expert_ffn_fp8``), the reference of the GPU path's E4M3 output gates.

Page "02 · DeepSeek-V3", §2.2: the inputs of the expert GEMMs are E4M3 with one
scale per 1x128 activation tile (the layer input x, and the SwiGLU output H
ahead of the down projection), weights are E4M3 per 128x128 block, and the
products are accumulated at high precision.  Pins:
  - with the identity quantiser the emulation is the plain (pinned) forward,
    up to the float32 rounding of H;
  - on tiny E4M3 layers with outliers, every token equals a scalar-loop
    brute force that quantises x and H slice by slice with torch's
    float8_e4m3fn encoder (tests/bruteforce.py), for one slice of H per row
    (inter 128) and for two (inter 256).
CPU only."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests import bruteforce as BF


def _layer(**kw):
    c = S.get_config("tiny").with_(**kw)
    x = O.lift(S.gen_x(c))
    wr = O.lift(S.gen_router(c))
    b = S.gen_bias(c).numpy()
    ex = {e: {k: v.numpy() for k, v in S.gen_expert(c, e).items()} for e in range(c.E + c.S)}
    return c, x, wr, b, ex


def _fwd(c, x, wr, b, ex, **kw):
    return O.forward(x, wr, b, lambda e: ex[e], n_groups=c.n_groups, topk_groups=c.topk_groups,
                     topk=c.topk, group_topn=c.group_topn, n_shared=c.n_shared, **kw)


# tiny E4M3 layers: bf16 activations, E4M3 weights, 2% outliers x50 so that
# many 1x128 slices of x carry one
FP8_TINY = dict(act_dtype="bf16", w_dtype="e4m3", outlier_p=0.02, outlier_mult=50.0)


@pytest.mark.parametrize("kw", [{}, FP8_TINY])
def test_identity_quantiser_reduces_to_plain_forward(kw):
    c, x, wr, b, ex = _layer(**kw)
    plain = _fwd(c, x, wr, b, ex)
    ident = _fwd(c, x, wr, b, ex, act_quant=lambda a: np.asarray(a, np.float64))
    err = O.max_row_rel_err(ident.y, plain.y)
    assert err <= 1e-6, err                 # float32 rounding of H only
    np.testing.assert_array_equal(ident.routing.idx, plain.routing.idx)


@pytest.mark.parametrize("kw", [FP8_TINY, dict(FP8_TINY, hidden=384, inter=256)])
def test_emulation_matches_scalar_loop_quantisation(kw):
    c, x, wr, b, ex = _layer(**kw)
    tokens = [0, 9, 33, c.T - 1]
    res = _fwd(c, x, wr, b, ex, tokens=tokens, act_quant=O.fake_quant_1x128)
    r = res.routing
    for j, t in enumerate(tokens):
        ref = BF.swiglu_fp8_loop(x[t], *O.expert_f64(ex[c.E]))         # shared, weight 1
        for k in range(c.topk):
            e = int(r.idx[t, k])
            ref = ref + float(r.gate[t, k]) * BF.swiglu_fp8_loop(x[t], *O.expert_f64(ex[e]))
        err = np.linalg.norm(res.y[j] - ref) / np.linalg.norm(ref)
        assert err <= 1e-9, (t, err)


def test_quantisation_is_visible_at_this_size():
    """The pins above can see a quantisation step: the emulation differs from
    the plain forward by far more than their tolerance (E4M3 keeps 3 mantissa
    bits), and quantising only H or only x each gives a different answer."""
    c, x, wr, b, ex = _layer(**FP8_TINY)
    plain = _fwd(c, x, wr, b, ex).y
    emu = _fwd(c, x, wr, b, ex, act_quant=O.fake_quant_1x128).y
    err = O.max_row_rel_err(emu, plain)
    assert 5e-3 < err < 0.2, err
    H = c.hidden
    only_h = _fwd(c, x, wr, b, ex,
                  act_quant=lambda a: a if a.shape[1] == H else O.fake_quant_1x128(a)).y
    assert O.max_row_rel_err(only_h, emu) > 1e-3
