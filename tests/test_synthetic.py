"""The seeded input generator: determinism, published SplitMix64 outputs,
distribution sanity, row slicing.  CPU only."""
import numpy as np
import torch

import synthetic as S


def test_splitmix64_published_sequence():
    # SplitMix64 started from state 0 (Steele, Lea & Flood 2014)
    z = S._raw(0, 0, 3, "cpu").tolist()
    got = [v & ((1 << 64) - 1) for v in z]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_same_seed_same_bits_and_streams_differ():
    c = S.get_config("tiny")
    a, b = S.gen_x(c), S.gen_x(c)
    assert torch.equal(a, b)
    assert not torch.equal(S.gen_x(c, step=1), a)
    e3, e4 = S.gen_expert(c, 3), S.gen_expert(c, 4)
    assert not torch.equal(e3["w_gate"], e4["w_gate"])
    assert not torch.equal(e3["w_gate"], e3["w_up"])


def test_normal_and_uniform_moments():
    v = S.normal(S.stream_key(9, 0, 0), 1 << 21)
    assert abs(v.mean().item()) < 3e-3 and abs(v.std().item() - 1.0) < 3e-3
    u = S.uniform01(S.stream_key(9, 2, 0), 1 << 20)
    assert u.min().item() > 0 and u.max().item() < 1 and abs(u.mean().item() - 0.5) < 2e-3
    m = S.bernoulli(S.stream_key(9, 7, 0), 1 << 22, 1e-3)
    assert abs(m.float().mean().item() - 1e-3) < 1e-4


def test_row_slices_equal_full_tensor():
    for name in ("fp8", "skew"):
        c = S.get_config(name, T=12)
        full = S.gen_x(c)
        assert torch.equal(full[3:7], S.gen_x(c, rows=slice(3, 7)))


def test_config_recipes():
    c = S.get_config("skew", T=8)
    x = S.gen_x(c)
    assert torch.all(x[:, 0] == 1.0)
    wr = S.gen_router(c)
    off = S.zipf_offsets(c)
    assert torch.equal(wr[0], torch.from_numpy(off))
    assert abs(float(off.astype(np.float64).mean())) < 1e-5
    assert 5.4 < off.max() < 5.5 and -1.19 < off.min() < -1.17
    b = S.gen_bias(S.get_config("prefill"))
    assert b.abs().max().item() <= 0.01 and b.abs().max().item() > 0.009
    assert torch.all(S.gen_bias(S.get_config("decode")) == 0)
    w = S.gen_expert(S.get_config("tiny"), 0)
    assert w["w_gate"].shape == (128, 256) and w["w_down"].shape == (256, 128)
    assert abs(w["w_down"].std().item() * np.sqrt(128) - 1.0) < 0.05


def test_e4m3_weight_encoding_shapes():
    c = S.get_config("fp8", hidden=256, inter=128)
    w = S.gen_expert(c, 0)
    assert w["w_gate"].dtype == torch.uint8 and w["s_gate"].shape == (1, 2)
    assert w["w_down"].shape == (256, 128) and w["s_down"].shape == (2, 1)
    codes = w["w_gate"].view(torch.float8_e4m3fn).to(torch.float32)
    assert not torch.isnan(codes).any()
    assert codes.abs().max().item() == 448.0
