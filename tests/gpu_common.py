"""Shared helpers of the GPU parity tests: input upload, oracle comparison."""
import sys

import numpy as np
import torch

import oracle as O
import sparse_moe_layer_group_amd as moe
import synthetic as S

DEV = "cuda"
SEL_TOL_GATE = 1e-6
OUT_TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class GpuInputs:
    """Seeded inputs of one configuration resident on the GPU."""

    def __init__(self, c, step=0, T=None):
        if T is not None:
            c = c.with_(T=T)
        self.c = c
        self.cfg = moe.cfg_from(c)
        self.x = S.gen_x(c, step=step, device=DEV)
        self.wr = S.gen_router(c, device=DEV)
        self.b = S.gen_bias(c, device=DEV)
        self.ex = S.gen_experts(c, device=DEV)
        self.T = c.T

    def run_forward(self, residual=None, out=None):
        y = torch.empty_like(self.x)
        if out is None:
            out = moe.alloc_routing(self.cfg, self.T, DEV)
        ws = moe.alloc_workspace(self.cfg, self.T, DEV)
        moe.forward(self.cfg, self.x, self.wr, self.b, self.ex, y, ws, residual=residual, out=out)
        torch.cuda.synchronize()
        return y, out

    def run_route(self, x=None, b=None):
        x = self.x if x is None else x
        b = self.b if b is None else b
        out = moe.alloc_routing(self.cfg, x.shape[0], DEV)
        ws = moe.alloc_workspace(self.cfg, x.shape[0], DEV)
        moe.route(self.cfg, x, self.wr, b, out, ws)
        torch.cuda.synchronize()
        return out


def cpu_expert_source(c):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = S.gen_expert(c, e, "cpu")   # torch CPU tensors; the oracle lifts them
        return cache[e]
    return get


def oracle_route(c, x_cpu, b_np):
    return O.route(O.lift(x_cpu), O.lift(S.gen_router(c, "cpu")), b_np, n_groups=c.n_groups,
                   topk_groups=c.topk_groups, topk=c.topk, group_topn=c.group_topn)


def check_routing(c, out, ref_r, label=""):
    """Four-part routing parity: selection (unflagged tokens), gates, and the
    permutation recomputed by the oracle from the GPU's own selection."""
    T, K, E = out["topk_idx"].shape[0], c.topk, c.n_experts
    idx = out["topk_idx"].cpu().numpy()
    gate = out["topk_gate"].cpu().numpy()
    ok = ~ref_r.flagged
    flagged = np.nonzero(ref_r.flagged)[0]
    mism = np.nonzero(np.any(idx != ref_r.idx, axis=1) & ok)[0]
    assert mism.size == 0, f"{label}: selection differs on unflagged tokens {mism[:10]}"
    gerr = float(np.abs(gate[ok] - ref_r.gate[ok]).max()) if ok.any() else 0.0
    assert gerr <= SEL_TOL_GATE, f"{label}: gate error {gerr}"
    # every token: valid selection (distinct ascending ids inside <= topk_groups groups)
    assert np.all(np.diff(idx, axis=1) > 0) and idx.min() >= 0 and idx.max() < E
    per = E // c.n_groups
    ngroups = np.array([len(set(row // per)) for row in idx])
    assert np.all(ngroups <= c.topk_groups)
    assert np.all(np.abs(gate.astype(np.float64).sum(axis=1) - 1.0) <= 1e-6)
    # permutation: bit-exact against the oracle applied to the GPU selection
    p = O.permute(idx, E)
    for name in ("counts", "offsets", "perm", "slot"):
        got = out[name].cpu().numpy()
        assert np.array_equal(got, getattr(p, name)), f"{label}: {name} differs"
    if "tie_gap" in out:
        gap = out["tie_gap"].cpu().numpy()
        # the GPU's own gap agrees with the oracle's to float32 rounding of s
        both = np.minimum(ref_r.egap, ref_r.ggap)
        fin = np.isfinite(both)
        assert np.all(np.abs(gap[fin] - both[fin]) < 1e-5)
    say(f"{label}: routing ok: {T} tokens, {flagged.size} near-ties flagged {flagged[:8].tolist()}, "
        f"gate err {gerr:.2e}")
    return p


def row_errors(y_gpu, y_ref):
    y = y_gpu.astype(np.float64)
    num = np.linalg.norm(y - y_ref, axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    return num / den
