"""GPU parity of the layer backward (page "02 · DeepSeek-V3", §1.3 Eq 12-15,
§1.4, §2.2) against the oracle on the same seeded inputs.

The GPU recomputes G, U, H and Y and stages them, and the gradients dY, dG,
dU and dX, in bfloat16 (relative rounding up to 2^-9 each); every sum runs in
float32.  The oracle is float64 on the same bf16 inputs and upstream gradient.
Bars:
  - dx: max over tokens of ||dx_gpu - dx_ref|| / ||dx_ref|| <= 2e-2;
  - every expert's dW_gate, dW_up, dW_down: ||D||_F / ||R||_F <= 2e-2;
  - dW_r: ||D||_F / ||R||_F <= 2e-2;
  - two calls bitwise identical.
Measured at the mid shapes: about 4e-3 for each (bf16 staging, a few 2^-9).
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import sparse_moe_layer_group_amd as moe
import synthetic as S
from tests.conftest import gpu_available
from tests.gpu_common import DEV, GpuInputs, cpu_expert_source, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = 2e-2


def _dy(c, seed=99):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((c.T, c.hidden), generator=g).to(torch.bfloat16)


def _run(gi, dy_cpu):
    c = gi.c
    n = c.n_experts + c.n_shared
    dy = dy_cpu.to(DEV)
    dx = torch.empty_like(gi.x)
    dwr = torch.empty((c.hidden, c.n_experts), dtype=torch.float32, device=DEV)
    dwg = torch.empty((n, c.inter, c.hidden), dtype=torch.float32, device=DEV)
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((n, c.hidden, c.inter), dtype=torch.float32, device=DEV)
    ws = moe.alloc_backward_workspace(gi.cfg, c.T, DEV)
    moe.backward(gi.cfg, gi.x, gi.wr, gi.b, gi.ex, dy, dx, dwr, dwg, dwu, dwd, ws)
    torch.cuda.synchronize()
    del ws
    return dx, dwr, dwg, dwu, dwd


def _oracle(c, dy_cpu, **kw):
    return O.backward(O.lift(S.gen_x(c, device="cpu")), O.lift(S.gen_router(c, "cpu")),
                      S.gen_bias(c, "cpu").numpy(), cpu_expert_source(c), O.lift(dy_cpu),
                      n_groups=c.n_groups, topk_groups=c.topk_groups, topk=c.topk,
                      group_topn=c.group_topn, n_shared=c.n_shared, **kw)


def _rel_f(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _row_rel(a, b):
    return (np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300))


# mid T=3000: 293-454 rows per expert (two 320-row data-gradient tiles for some,
# weight-gradient K loops with ragged tails); T=300: the large-tile data-gradient
# kernel with one tile; T=65 and 1: the 128-row kernel
# mid T=3000 and mid_skew T=800 take the persistent weight-gradient kernel (more
# than 64 rows per routed expert); mid_skew T=800 has two experts without rows
# (all-zero gradient tiles) and one with 792 rows (25 k-steps); mid T=800 without
# a shared expert: no shared rows, tiles or gradients anywhere in the backward
@pytest.mark.parametrize("name,T,kw", [("mid", 300, {}), ("mid", 65, {}), ("mid", 1, {}),
                                       ("mid_skew", 300, {}), ("mid", 3000, {}), ("mid_skew", 800, {}),
                                       ("mid", 800, {"n_shared": 0})])
def test_backward_parity(name, T, kw):
    c = S.get_config(name, T=T, **kw)
    say(f"backward parity: {name} T={T} {kw}")
    gi = GpuInputs(c)
    dy = _dy(c)
    dx, dwr, dwg, dwu, dwd = _run(gi, dy)
    ref = _oracle(c, dy)
    ex = row = float(_row_rel(dx.float().cpu().numpy(), ref.dx).max())
    wr_err = _rel_f(dwr.cpu().numpy(), ref.dw_router)
    worst = 0.0
    for e, (g, u, d) in ref.dw.items():
        if not np.any(g) and not np.any(d):
            assert float(dwg[e].abs().max()) == 0.0 and float(dwd[e].abs().max()) == 0.0
            continue
        for got, want in ((dwg[e], g), (dwu[e], u), (dwd[e], d)):
            worst = max(worst, _rel_f(got.cpu().numpy(), want))
    say(f"{name} T={T}: dx max row rel {ex:.3e}; dW max rel {worst:.3e}; dW_r rel {wr_err:.3e}")
    assert row <= TOL
    assert worst <= TOL
    assert wr_err <= TOL


def test_backward_is_deterministic():
    c = S.get_config("mid", T=300)
    gi = GpuInputs(c)
    dy = _dy(c)
    a = _run(gi, dy)
    b = _run(gi, dy)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_backward_with_an_underflowed_gate():
    """A chosen expert whose float32 sigmoid underflows to 0 (gate exactly 0).

    The GPU forms dg_k = <dH_k, H_k> / g_k from the data-gradient GEMM; at g_k =
    0 it takes dg_k = 0, which leaves every logit gradient as the true <dy, Y_k>
    would (dg_k enters them only through g_k dg_k and s_k (1 - s_k)).  Inputs:
    mid_skew (x[:, 0] = 1), expert 5's router column -120 e_0 (logit -120 for
    every token: float32 sigmoid 0, float64 7.7e-53), its bias +10 (chosen by
    every token).  The oracle runs in float64 on the same inputs."""
    c = S.get_config("mid_skew", T=800)
    say(f"backward, underflowed gate: mid_skew T={c.T}")
    e0 = 5
    wr = S.gen_router(c, "cpu").clone()
    wr[:, e0] = 0.0
    wr[0, e0] = -120.0
    b = S.gen_bias(c, "cpu").clone()
    b[e0] = 10.0
    gi = GpuInputs(c)
    gi.wr = wr.to(DEV)
    gi.b = b.to(DEV)
    counts = gi.run_route()["counts"].cpu().numpy()
    assert counts[e0] == c.T
    dy = _dy(c)
    dx, dwr, dwg, dwu, dwd = _run(gi, dy)
    assert bool(torch.isfinite(dx.float()).all()) and bool(torch.isfinite(dwr).all())
    ref = O.backward(O.lift(S.gen_x(c, device="cpu")), O.lift(wr), b.numpy(), cpu_expert_source(c),
                     O.lift(dy), n_groups=c.n_groups, topk_groups=c.topk_groups, topk=c.topk,
                     group_topn=c.group_topn, n_shared=c.n_shared, grad_experts=[e0, c.n_experts])
    rows = _row_rel(dx.float().cpu().numpy(), ref.dx)
    wr_err = _rel_f(dwr.cpu().numpy(), ref.dw_router)
    sh = c.n_experts
    mats = [_rel_f(got[sh].cpu().numpy(), want) for got, want in zip((dwg, dwu, dwd), ref.dw[sh])]
    say(f"underflowed gate: dx max row rel {rows.max():.3e}; dW_r rel {wr_err:.3e}; shared dW max "
        f"rel {max(mats):.3e}")
    assert rows.max() <= TOL and wr_err <= TOL and max(mats) <= TOL
    # expert e0's gradients carry the factor g = 0 (float64: 1e-53 of the others)
    for got, want in zip((dwg, dwu, dwd), ref.dw[e0]):
        assert float(got[e0].abs().max()) == 0.0 and float(np.abs(want).max()) < 1e-40


@pytest.mark.parametrize("seed", [None, 21])   # the workload's own seed, and one more
@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_v3_backward_sampled(name, seed):
    c = S.get_config(name) if seed is None else S.get_config(name, seed=seed)
    say(f"V3 backward {name}: T={c.T}, seed {c.seed}")
    gi = GpuInputs(c)
    dy = _dy(c)
    dx, dwr, dwg, dwu, dwd = _run(gi, dy)
    out = gi.run_route()
    counts = out["counts"].cpu().numpy()
    busiest = int(np.argmax(counts))
    experts = [busiest, int(np.argmin(counts))]
    if name == "decode":
        experts.append(c.n_experts)  # the shared expert (every token's rows)
    tokens = [0, c.T // 2, c.T - 1]
    # a dW_r column needs the full forward of every token routed to its expert
    # (their K experts each): one lightly loaded column at decode only; the
    # mid-size cases check all of dW_r
    rcols = [int(np.argmin(counts))] if name == "decode" else []
    ref = _oracle(c, dy, tokens=tokens, grad_experts=experts, router_cols=rcols)
    dxe = _row_rel(dx[tokens].float().cpu().numpy(), ref.dx)
    errs = {}
    for e in experts:
        g, u, d = ref.dw[e]
        errs[e] = max(_rel_f(dwg[e].cpu().numpy(), g), _rel_f(dwu[e].cpu().numpy(), u),
                      _rel_f(dwd[e].cpu().numpy(), d))
    wr = max([_rel_f(dwr[:, e].cpu().numpy(), ref.dw_router[:, e]) for e in rcols] + [0.0])
    say(f"V3 {name}: dx rows {np.round(dxe, 5).tolist()}, dW {dict((k, round(v, 5)) for k, v in errs.items())}"
        f" (counts {[int(counts[e]) if e < c.n_experts else c.T for e in experts]}), dW_r {wr:.3e}")
    assert dxe.max() <= TOL
    assert max(errs.values()) <= TOL
    assert wr <= TOL
    del gi, dx, dwr, dwg, dwu, dwd
    gc.collect()
    torch.cuda.empty_cache()
