"""Layer output at the largest batch the library accepts for the V3 shape.

Page "02 · DeepSeek-V3": §1.3 (every token is routed and computed, whatever
the batch: no token dropping), §1.1 / Eq 12 (the layer output), §2.2 (the
E4M3 path).  With bf16 activations the entry points accept T up to 299,593:
x then spans 299,593 * 7168 * 2 bytes, just under 4 GiB, the bound of the
tiled GEMMs' 32-bit buffer ranges over x.  The staged expert rows (34 GB of Y,
11 GB of H) lie far past 4 GiB, so every down GEMM's range must start at its
own expert.  At this T each routed expert has about 9,400 rows (30 row tiles)
and the shared expert 299,593.

Checked on the GPU's run of the whole batch:
  - the permutation (counts, offsets, perm, slot) bit-exact against the
    oracle's permutation of the GPU's own selection (every token);
  - for sampled tokens, selection (unflagged), gates (1e-6) and output rows
    against the float64 oracle routed on those tokens alone (a token's
    routing and FFN do not depend on the other tokens): the first, middle and
    last tokens, the tokens of the last staged row of the four highest
    experts (the ends of the staging buffers), a row of each of several late
    row tiles of the shared expert, and random tokens.
Bars as at the other V3 shapes: max row-relative error 2e-2 (bf16), 6e-2
against the oracle's E4M3 layer (E4M3 weights).
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import sparse_moe_layer_group_amd as moe
import synthetic as S
from tests.conftest import gpu_available
from tests.gpu_common import DEV, OUT_TOL, SEL_TOL_GATE, GpuInputs, row_errors, say
from tests.test_gpu_v3_full import ExpertsAhead

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900),
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

T_MAX = 299593           # (2^32 - 1) // (7168 * 2): x of the V3 shape in bf16 under 4 GiB


def _sample(p, T, K, E, rng):
    tok = {0, 1, T // 2, T - 1}
    for e in range(E - 4, E):                  # last staged rows of the highest experts
        tok.add(int(p.perm[p.offsets[e] + p.counts[e] - 1]))
    for m in (T - 1, T - 321, T - 3200, T - 32000, 100000):   # late shared-expert row tiles
        tok.add(int(m))                        # the shared expert's row m is token m
    tok |= set(rng.choice(T, 12, replace=False).tolist())
    return np.array(sorted(tok), dtype=np.int64)


@pytest.mark.parametrize("name", ["prefill", "fp8"])
def test_largest_accepted_batch(name):
    c = S.get_config(name, T=T_MAX)
    cfg = moe.cfg_from(c)
    assert moe.workspace_bytes(cfg, T_MAX) > 0 and moe.workspace_bytes(cfg, T_MAX + 1) == 0
    assert T_MAX * c.hidden * 2 < 2 ** 32 <= (T_MAX + 1) * c.hidden * 2
    say(f"max batch {name}: T={T_MAX}, workspace {moe.workspace_bytes(cfg, T_MAX) / 2**30:.1f} GiB")
    gi = GpuInputs(c)
    y, out = gi.run_forward()
    idx = out["topk_idx"].cpu().numpy()
    gate = out["topk_gate"].cpu().numpy()
    got = {k: out[k].cpu().numpy() for k in ("counts", "offsets", "perm", "slot")}
    x_cpu = gi.x.cpu()
    host = {k: v.cpu() for k, v in gi.ex.items()}
    b = gi.b.cpu().numpy()
    try:
        E, K = c.n_experts, c.topk
        p = O.permute(idx, E)
        for k in got:
            assert np.array_equal(got[k], getattr(p, k)), f"{name}: {k} differs at T={T_MAX}"
        say(f"max batch {name}: permutation bit-exact; rows per expert "
            f"{int(p.counts.min())}..{int(p.counts.max())}")
        tok = _sample(p, T_MAX, K, E, np.random.default_rng(5))
        y_s = y[torch.from_numpy(tok).to(DEV)].float().cpu().numpy()
        x64 = O.lift(x_cpu[torch.from_numpy(tok)])
        wr64 = O.lift(S.gen_router(c, "cpu"))
        used = sorted(set(int(e) for e in idx[tok].reshape(-1)))
        src = ExpertsAhead(host, used + [E])
        e4m3 = c.w_dtype == "e4m3"
        try:
            ref = O.forward(x64, wr64, b, src, n_groups=c.n_groups, topk_groups=c.topk_groups,
                            topk=c.topk, group_topn=c.group_topn, n_shared=c.n_shared,
                            act_quant=O.fake_quant_1x128 if e4m3 else None)
        finally:
            src.close()
        r = ref.routing
        ok = ~r.flagged
        assert np.array_equal(idx[tok][ok], r.idx[ok]), f"{name}: selection differs"
        gerr = float(np.abs(gate[tok][ok] - r.gate[ok]).max())
        assert gerr <= SEL_TOL_GATE, gerr
        err = row_errors(y_s, ref.y)[ok]
        say(f"max batch {name}: {err.size} sampled rows (tokens {tok[:6].tolist()}...), "
            f"gate err {gerr:.2e}, max row err {err.max():.4e}, median {np.median(err):.4e}")
        assert err.size >= 16
        assert err.max() <= OUT_TOL["e4m3" if e4m3 else "bf16"]
    finally:
        del gi, y, out, host, x_cpu
        gc.collect()
        torch.cuda.empty_cache()
