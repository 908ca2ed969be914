"""moe_forward_noalloc, the entry point with the library's static device
scratch, against moe_forward with a caller workspace: same inputs, bitwise
identical outputs and routing (the two run the same kernels), on two calls in
a row with the second batch smaller than the first, and a batch beyond the
static scratch rejected without launching.  Calls go through the C ABI
(ctypes), as every GPU test here does."""
import ctypes

import pytest
import torch

import sparse_moe_layer_group_amd as moe
import synthetic as S
from tests.conftest import gpu_available
from tests.gpu_common import DEV, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _pair(c, T, residual):
    """moe_forward (workspace) and moe_forward_noalloc on the first T tokens."""
    cc = c.with_(T=T)
    cfg = moe.cfg_from(cc)
    x = S.gen_x(cc, device=DEV)
    wr = S.gen_router(cc, device=DEV)
    b = S.gen_bias(cc, device=DEV)
    ex = _pair.experts.setdefault(c.name, S.gen_experts(cc, device=DEV))
    res = x.flip(0).contiguous() if residual else None
    y_ref = torch.empty_like(x)
    out_ref = moe.alloc_routing(cfg, T, DEV)
    moe.forward(cfg, x, wr, b, ex, y_ref, moe.alloc_workspace(cfg, T, DEV), residual=res,
                out=out_ref)
    y = torch.full_like(x, float("nan"))
    out = moe.alloc_routing(cfg, T, DEV)
    moe.forward_noalloc(cfg, x, wr, b, ex, y, residual=res, out=out)
    y_int = torch.full_like(x, float("nan"))   # routing kept in the scratch
    moe.forward_noalloc(cfg, x, wr, b, ex, y_int, residual=res)
    torch.cuda.synchronize()
    return y_ref, out_ref, y, out, y_int


_pair.experts = {}


@pytest.mark.parametrize("name,T0,T1", [("mid", 300, 37), ("decode", 256, 64), ("mid_fp8", 300, 129),
                                        ("tiny", 64, 5)])
def test_noalloc_matches_forward_on_two_calls(name, T0, T1):
    c = S.get_config(name)
    for i, T in enumerate((T0, T1)):
        say(f"noalloc: {name} call {i} T={T}")
        y_ref, out_ref, y, out, y_int = _pair(c, T, residual=(i == 1))
        assert torch.equal(y, y_ref), f"{name} T={T}: output differs"
        assert torch.equal(y_int, y_ref), f"{name} T={T}: output with internal routing differs"
        for k in ("topk_idx", "topk_gate", "counts", "offsets", "perm", "slot", "tie_gap"):
            assert torch.equal(out[k], out_ref[k]), f"{name} T={T}: {k} differs"
    _pair.experts.pop(name, None)
    torch.cuda.empty_cache()


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    c = S.get_config("decode")
    cfg = moe.cfg_from(c)
    T = 322                                       # workspace 64.3 MiB > 64 MiB
    assert moe.workspace_bytes(cfg, T) > moe.NOALLOC_SCRATCH_BYTES >= moe.workspace_bytes(cfg, 321)
    one = ctypes.c_void_p(1)
    ex = moe._Experts(1, 1, 1, None, None, None)
    rc = moe.lib().moe_forward_noalloc(ctypes.byref(cfg), T, one, one, one, ctypes.byref(ex), None,
                                       one, None, None)
    assert rc == -7 and "static" in moe.status_string(rc)
