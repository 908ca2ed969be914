"""GPU parity of the sequence-wise balance loss (page "02 · DeepSeek-V3",
§1.4, Eq 17-20) against the oracle on the same seeded inputs.

Bars: per-expert selection counts (f * K * seq_len / E) exact on sequences
without a near-tie (K-th minus (K+1)-th raw affinity < 1e-6) and within the
number of near-tie tokens otherwise; P within 1e-6 absolute; the loss within
1e-5 relative (1e-4 absolute of alpha when it is not bitwise defined by ties);
two calls bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_moe_layer_group_amd as moe
import synthetic as S
from tests.conftest import gpu_available
from tests.gpu_common import DEV, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

ALPHA = 1e-4


def _run(c, seq_len):
    cfg = moe.cfg_from(c)
    x = S.gen_x(c, device=DEV)
    wr = S.gen_router(c, DEV)
    n_seq = c.T // seq_len
    loss = torch.empty(n_seq, dtype=torch.float32, device=DEV)
    f = torch.empty((n_seq, c.n_experts), dtype=torch.float32, device=DEV)
    p = torch.empty((n_seq, c.n_experts), dtype=torch.float32, device=DEV)
    ws = moe.alloc_workspace(cfg, c.T, DEV)
    moe.balance_loss(cfg, x, wr, seq_len, ALPHA, loss, ws, f=f, p=p)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), f.cpu().numpy(), p.cpu().numpy()


@pytest.mark.parametrize("name,T,seq_len", [("tiny", 64, 16), ("tiny", 64, 64), ("mid", 300, 100),
                                            ("mid", 300, 1), ("decode", 256, 256),
                                            ("skew", 4096, 1024), ("prefill", 8192, 4096)])
def test_balance_loss_parity(name, T, seq_len):
    c = S.get_config(name, T=T)
    loss, f, p = _run(c, seq_len)
    _, s = O.router_affinity(O.lift(S.gen_x(c, device="cpu")), O.lift(S.gen_router(c, "cpu")))
    ref = O.sequence_balance_loss(s, c.topk, seq_len, ALPHA)
    scale = c.topk * seq_len / c.n_experts
    cnt = np.rint(f.astype(np.float64) * scale).astype(np.int64)
    cnt_ref = np.rint(ref.f * scale).astype(np.int64)
    near = (ref.gap < 1e-6).reshape(-1, seq_len).sum(axis=1)
    for q in range(T // seq_len):
        diff = int(np.abs(cnt[q] - cnt_ref[q]).sum())
        assert diff <= 2 * near[q], (q, diff, int(near[q]))
    assert np.abs(p - ref.P).max() <= 1e-6
    ok = near == 0
    if ok.any():
        rel = np.abs(loss[ok] - ref.loss[ok]) / np.abs(ref.loss[ok])
        assert rel.max() <= 1e-5, rel.max()
    assert np.abs(loss - ref.loss).max() <= 1e-4 * ALPHA * seq_len
    say(f"balance loss {name} T={T} seq_len={seq_len}: loss/alpha {np.round(loss[:4] / ALPHA, 4).tolist()} "
        f"(oracle {np.round(ref.loss[:4] / ALPHA, 4).tolist()}), near-ties {int(near.sum())}")


def test_balance_loss_is_deterministic():
    c = S.get_config("skew", T=2048)
    a = _run(c, 2048)
    b = _run(c, 2048)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_skewed_routing_raises_the_loss():
    # the Zipf-offset router concentrates tokens on a few experts: against the
    # same batch under the unskewed router, the hottest expert's frequency and
    # the loss both rise
    c = S.get_config("skew", T=1024)
    loss, f, p = _run(c, 1024)
    loss0, f0, p0 = _run(c.with_(zipf_s=None), 1024)
    say(f"balance loss / alpha: skewed {loss[0] / ALPHA:.4f}, unskewed {loss0[0] / ALPHA:.4f}; "
        f"max f {f[0].max():.2f} vs {f0[0].max():.2f}")
    assert loss[0] > 1.5 * loss0[0]
    assert f[0].max() > 10 and f0[0].max() < 3
