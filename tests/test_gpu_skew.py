"""The skewed-routing workload on the GPU: 200 steps of the loss-free bias
update (page "02 · DeepSeek-V3", §1.4) at the V3 shape, T=4096, with router
logits offset per expert by a centred log-Zipf(1.2) profile.

Every step: the GPU's bias update is bit-exact against the oracle's rule
applied to the GPU's own counts.  At steps 0, 100 and 199: the GPU's routing
(selection, gates, counts, permutation) against the oracle on the same batch
and bias.  The max/mean expert load must fall as the bias adapts.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_moe_layer_group_amd as moe
import synthetic as S
from tests.conftest import gpu_available
from tests.gpu_common import DEV, check_routing, oracle_route, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def test_skew_200_bias_steps():
    c = S.get_config("skew")
    assert c.steps == 200 and c.T == 4096
    cfg = moe.cfg_from(c)
    wr = S.gen_router(c, DEV)
    b = torch.zeros(c.n_experts, dtype=torch.float32, device=DEV)
    ws = moe.alloc_workspace(cfg, c.T, DEV)
    out = moe.alloc_routing(cfg, c.T, DEV)
    b_ref = np.zeros(c.n_experts, np.float32)
    ratios = []
    for step in range(c.steps):
        x = S.gen_x(c, step=step, device=DEV)
        moe.route(cfg, x, wr, b, out, ws)
        counts = out["counts"].cpu().numpy()
        if step in (0, 100, 199):
            L, s, r, p = oracle_route(c, S.gen_x(c, step=step, device="cpu"), b_ref)
            check_routing(c, out, r, f"skew step {step}")
        moe.bias_update(cfg, c.T, out["counts"], b, c.gamma)
        b_ref = O.bias_update(b_ref, counts, c.T, c.topk, c.gamma)
        got = b.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), b_ref.view(np.uint32)), f"bias differs at step {step}"
        ratios.append(O.load_ratio(counts))
    say("skew: max/mean load at steps 0/25/50/100/150/199: " +
        " ".join(f"{ratios[i]:.2f}" for i in (0, 25, 50, 100, 150, 199)))
    assert ratios[0] > 10 and ratios[-1] < ratios[0] / 4
