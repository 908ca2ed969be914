"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module is shared by the CPU oracle tests and by the GPU path's tests and
benchmark. It holds no step of the layer's arithmetic: only random numbers,
tensor shapes, dtype rounding and the offline weight encoding that the layer
receives as input.

Random numbers come from one counter-based generator, SplitMix64 (Steele, Lea
and Flood, "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014):
element ``i`` of stream ``key`` is ``mix64(key + (i + 1) * 0x9E3779B97F4A7C15)``
with the paper's 64-bit finaliser.  The same torch integer code runs on the CPU
and on a GPU device, so both produce identical bits for the same
``(seed, tensor id, index)``; a GPU test checks that.

* Normal variates: inverse-CDF lookup.  The top 20 output bits index a table of
  Phi^-1((j + 1/2) / 2^20), computed in float64 and rounded to float32.
* Uniform variates on (0, 1): 23 output bits ``v`` give ``(2v + 1) * 2^-24``,
  which is exact in float32.
* Bernoulli(p): the low 20 bits compared with ``round(p * 2^20)``.

Stream keys: ``mix64(seed << 40 | tensor_id << 32 | index)`` with tensor ids
0 x (index = step), 1 router weights, 2 bias, 3 gate, 4 up, 5 down
(index = expert id, the shared expert is id E), 6 Zipf rank permutation,
7 outlier masks (index = tensor_id << 20 | sub-index).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np
import torch

__all__ = [
    "MoEConfig", "CONFIGS", "get_config", "normal", "uniform01", "bernoulli",
    "gen_x", "gen_router", "gen_bias", "gen_expert", "gen_experts",
    "zipf_offsets", "expert_param_count",
]

# ----------------------------------------------------------------------------
# configurations (shapes from the V3 description: hidden 7168, 256 routed
# experts in 8 groups plus 1 shared, intermediate 2048, 8 routed per token)
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class MoEConfig:
    name: str
    seed: int
    T: int
    hidden: int
    inter: int
    n_experts: int
    n_groups: int
    topk_groups: int
    topk: int
    group_topn: int = 2
    n_shared: int = 1
    act_dtype: str = "bf16"        # "f32" | "bf16"
    w_dtype: str = "bf16"          # "f32" | "bf16" | "e4m3"
    bias_kind: str = "zero"        # "zero" | "uniform"
    bias_range: float = 0.0
    router_scale: float = 1.0      # multiplies the N(0, 1/H) router init
    zipf_s: Optional[float] = None  # skewed routing: centred log-Zipf offsets
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    gamma: float = 1e-3
    steps: int = 1                 # bias-update steps for the skew workload

    @property
    def E(self) -> int:
        return self.n_experts

    @property
    def S(self) -> int:
        return self.n_shared

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


_V3 = dict(hidden=7168, inter=2048, n_experts=256, n_groups=8, topk_groups=4, topk=8,
           group_topn=2, n_shared=1)

CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig(name="tiny", seed=0, T=64, hidden=256, inter=128, n_experts=16,
                      n_groups=4, topk_groups=2, topk=4, group_topn=2, n_shared=1,
                      act_dtype="f32", w_dtype="f32", bias_kind="uniform",
                      bias_range=0.05),
    "decode": MoEConfig(name="decode", seed=1, T=256, **_V3),
    "prefill": MoEConfig(name="prefill", seed=2, T=8192, bias_kind="uniform",
                         bias_range=0.01, **_V3),
    "skew": MoEConfig(name="skew", seed=3, T=4096, zipf_s=1.2, steps=200, **_V3),
    "fp8": MoEConfig(name="fp8", seed=4, T=4096, w_dtype="e4m3", outlier_p=1e-3,
                     outlier_mult=50.0, **_V3),
    # reduced width, same routing structure: spans several GEMM tiles with
    # ragged tails and is small enough for a full-output oracle comparison
    "mid": MoEConfig(name="mid", seed=5, T=300, hidden=1024, inter=256, n_experts=64,
                     n_groups=8, topk_groups=4, topk=8, group_topn=2, n_shared=1,
                     bias_kind="uniform", bias_range=0.02),
    "mid_skew": MoEConfig(name="mid_skew", seed=7, T=300, hidden=1024, inter=256, n_experts=64,
                          n_groups=8, topk_groups=4, topk=8, group_topn=2, n_shared=1,
                          zipf_s=1.2),
    "mid_fp8": MoEConfig(name="mid_fp8", seed=6, T=300, hidden=1024, inter=256, n_experts=64,
                         n_groups=8, topk_groups=4, topk=8, group_topn=2, n_shared=1,
                         w_dtype="e4m3", outlier_p=1e-3, outlier_mult=50.0),
}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg


def expert_param_count(cfg: MoEConfig) -> int:
    """Parameters of one SwiGLU expert as generated (three matrices)."""
    return 2 * cfg.inter * cfg.hidden + cfg.hidden * cfg.inter


# ----------------------------------------------------------------------------
# SplitMix64 on torch int64 (wrap-around arithmetic, logical shifts by masking)
# ----------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def _s64(c: int) -> int:
    c &= _M64
    return c - (1 << 64) if c >= (1 << 63) else c


_GAMMA = 0x9E3779B97F4A7C15
_MUL1 = 0xBF58476D1CE4E5B9
_MUL2 = 0x94D049BB133111EB


def _mix64_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * _MUL1) & _M64
    z = ((z ^ (z >> 27)) * _MUL2) & _M64
    return z ^ (z >> 31)


def _mix64_(z: torch.Tensor) -> torch.Tensor:
    """In-place SplitMix64 finaliser on an int64 tensor."""
    t = torch.empty_like(z)
    torch.bitwise_right_shift(z, 30, out=t)
    t.bitwise_and_((1 << 34) - 1)
    z.bitwise_xor_(t)
    z.mul_(_s64(_MUL1))
    torch.bitwise_right_shift(z, 27, out=t)
    t.bitwise_and_((1 << 37) - 1)
    z.bitwise_xor_(t)
    z.mul_(_s64(_MUL2))
    torch.bitwise_right_shift(z, 31, out=t)
    t.bitwise_and_((1 << 33) - 1)
    z.bitwise_xor_(t)
    return z


def stream_key(seed: int, tensor_id: int, index: int) -> int:
    assert 0 <= seed < (1 << 24) and 0 <= tensor_id < 256 and 0 <= index < (1 << 32)
    return _mix64_int((seed << 40) | (tensor_id << 32) | index)


def _raw(key: int, start: int, n: int, device) -> torch.Tensor:
    """Raw 64-bit outputs start..start+n-1 of the stream (int64 tensor)."""
    z = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z.mul_(_s64(_GAMMA)).add_(_s64(key))
    return _mix64_(z)


_NORMAL_BITS = 20
_TABLES: Dict[str, torch.Tensor] = {}


def _normal_table(device) -> torch.Tensor:
    dev = str(torch.device(device))
    if dev not in _TABLES:
        if "cpu" not in _TABLES:
            from scipy.special import ndtri
            j = np.arange(1 << _NORMAL_BITS, dtype=np.float64)
            tab = ndtri((j + 0.5) / float(1 << _NORMAL_BITS)).astype(np.float32)
            _TABLES["cpu"] = torch.from_numpy(tab)
        _TABLES[dev] = _TABLES["cpu"].to(device)
    return _TABLES[dev]


def normal(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """n standard-normal float32 variates of stream ``key``."""
    z = _raw(key, start, n, device)
    z.bitwise_right_shift_(64 - _NORMAL_BITS)
    z.bitwise_and_((1 << _NORMAL_BITS) - 1)
    return _normal_table(device)[z]


def uniform01(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """n float32 variates on (0, 1), each exactly (2v + 1) * 2^-24."""
    z = _raw(key, start, n, device)
    z.bitwise_right_shift_(41)
    z.bitwise_and_((1 << 23) - 1)
    u = z.to(torch.float32)
    return u.mul_(2.0).add_(1.0).mul_(2.0 ** -24)


def bernoulli(key: int, n: int, p: float, device="cpu", start: int = 0) -> torch.Tensor:
    z = _raw(key, start, n, device)
    z.bitwise_and_((1 << 20) - 1)
    return z < int(round(p * (1 << 20)))


# ----------------------------------------------------------------------------
# tensors of one configuration
# ----------------------------------------------------------------------------

_TID_X, _TID_WR, _TID_B, _TID_G, _TID_U, _TID_D, _TID_ZIPF, _TID_OUT = range(8)


def _f32(v: float) -> float:
    return float(np.float32(v))


def _round_act(v: torch.Tensor, cfg: MoEConfig) -> torch.Tensor:
    if cfg.act_dtype == "f32":
        return v
    if cfg.act_dtype == "bf16":
        return v.to(torch.bfloat16)
    raise ValueError(cfg.act_dtype)


def _apply_outliers(v: torch.Tensor, cfg: MoEConfig, tid: int, sub: int, start: int = 0) -> torch.Tensor:
    """Multiply a Bernoulli(outlier_p) subset of entries by outlier_mult."""
    if cfg.outlier_p <= 0.0:
        return v
    m = bernoulli(stream_key(cfg.seed, _TID_OUT, (tid << 20) | sub), v.numel(), cfg.outlier_p,
                  v.device, start=start).view(v.shape)
    return torch.where(m, v * _f32(cfg.outlier_mult), v)


def gen_x(cfg: MoEConfig, step: int = 0, device="cpu", rows: Optional[slice] = None) -> torch.Tensor:
    """Token activations u_t, [T][hidden], x ~ N(0, 1) (skew: column 0 set to 1).

    ``rows`` selects a contiguous token range; its values equal the same rows
    of the full tensor.
    """
    T, H = cfg.T, cfg.hidden
    r0 = 0 if rows is None or rows.start is None else rows.start
    r1 = T if rows is None or rows.stop is None else rows.stop
    v = normal(stream_key(cfg.seed, _TID_X, step), (r1 - r0) * H, device, start=r0 * H).view(r1 - r0, H)
    v = _apply_outliers(v, cfg, _TID_X, step, start=r0 * H)
    if cfg.zipf_s is not None:
        v[:, 0] = 1.0
    return _round_act(v, cfg).contiguous()


def zipf_offsets(cfg: MoEConfig) -> np.ndarray:
    """Per-expert logit offsets for skewed routing: centred log-Zipf(s) pmf.

    A seeded permutation assigns each expert a rank r_e in 1..E; the offset is
    -s*ln(r_e) minus its mean over ranks, rounded to float32.
    """
    E = cfg.n_experts
    keys = _raw(stream_key(cfg.seed, _TID_ZIPF, 0), 0, E, "cpu").numpy()
    order = np.argsort(keys, kind="stable")
    rank = np.empty(E, dtype=np.int64)
    rank[order] = np.arange(1, E + 1)
    logp = -cfg.zipf_s * np.log(rank.astype(np.float64))
    mean = np.mean(-cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64)))
    return (logp - mean).astype(np.float32)


def gen_router(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """Router weights (expert centroids as columns), [hidden][E] float32, N(0, scale^2/hidden)."""
    H, E = cfg.hidden, cfg.n_experts
    w = normal(stream_key(cfg.seed, _TID_WR, 0), H * E, device).view(H, E)
    w.mul_(_f32(cfg.router_scale / math.sqrt(H)))
    if cfg.zipf_s is not None:
        w[0, :] = torch.from_numpy(zipf_offsets(cfg)).to(device)
    return w.contiguous()


def gen_bias(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """Initial load-balancing bias b, [E] float32."""
    E = cfg.n_experts
    if cfg.bias_kind == "zero":
        return torch.zeros(E, dtype=torch.float32, device=device)
    u = uniform01(stream_key(cfg.seed, _TID_B, 0), E, "cpu")
    b = (u * 2.0 - 1.0) * _f32(cfg.bias_range)
    return b.to(device)


def _e4m3_blocks(master: torch.Tensor):
    """Offline weight encoding: one float32 scale per 128x128 block, codes e4m3fn.

    scale = fl32(amax / 448) (1 if the block is all zero); code = RNE(fl32(v / scale)).
    Divisions are float64 tensor-by-tensor divisions (torch divides by a scalar
    on the GPU through a reciprocal), so CPU and GPU give identical encodings.
    Returns (uint8 codes with the master's shape, scales [rows/128][cols/128]).
    """
    R, C = master.shape
    blk = master.view(R // 128, 128, C // 128, 128)
    amax = blk.abs().amax(dim=(1, 3)).to(torch.float64)
    d448 = torch.full_like(amax, 448.0)
    scale = torch.where(amax > 0, amax / d448, torch.ones_like(amax)).to(torch.float32)
    ratio = (blk.to(torch.float64) / scale.to(torch.float64)[:, None, :, None]).to(torch.float32)
    q = ratio.to(torch.float8_e4m3fn)
    return q.view(torch.uint8).view(R, C).contiguous(), scale.contiguous()


def gen_expert(cfg: MoEConfig, e: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Weights of expert ``e`` (0..E-1 routed, E = shared).

    w_gate, w_up: [inter][hidden]; w_down: [hidden][inter]; each entry
    N(0, 1/fan_in).  float32 / bf16 / e4m3 codes (uint8) per ``cfg.w_dtype``;
    e4m3 also returns s_gate, s_up [inter/128][hidden/128] and
    s_down [hidden/128][inter/128].
    """
    H, I = cfg.hidden, cfg.inter
    out: Dict[str, torch.Tensor] = {}
    for name, tid, shape, fan_in in (("w_gate", _TID_G, (I, H), H), ("w_up", _TID_U, (I, H), H),
                                     ("w_down", _TID_D, (H, I), I)):
        v = normal(stream_key(cfg.seed, tid, e), shape[0] * shape[1], device).view(*shape)
        v.mul_(_f32(1.0 / math.sqrt(fan_in)))
        v = _apply_outliers(v, cfg, tid, e)
        if cfg.w_dtype == "f32":
            out[name] = v
        elif cfg.w_dtype == "bf16":
            out[name] = v.to(torch.bfloat16)
        elif cfg.w_dtype == "e4m3":
            q, s = _e4m3_blocks(v)
            out[name] = q
            out["s" + name[1:]] = s
        else:
            raise ValueError(cfg.w_dtype)
        del v
    return out


def gen_experts(cfg: MoEConfig, device="cpu") -> Dict[str, torch.Tensor]:
    """All E + S experts stacked: w_gate/w_up [E+S][I][H], w_down [E+S][H][I] (+ scales)."""
    n = cfg.n_experts + cfg.n_shared
    first = gen_expert(cfg, 0, device)
    out = {k: torch.empty((n,) + tuple(v.shape), dtype=v.dtype, device=device) for k, v in first.items()}
    for k, v in first.items():
        out[k][0].copy_(v)
    del first
    for e in range(1, n):
        for k, v in gen_expert(cfg, e, device).items():
            out[k][e].copy_(v)
    return out
