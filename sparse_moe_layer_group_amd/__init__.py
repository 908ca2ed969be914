"""Python binding of the gfx950 DeepSeekMoE layer library (``libmoe_mi355x.so``).

Argument marshalling only: torch tensors supply device memory and the current
stream; every step of the layer runs in the library's HIP kernels.  There is no
fallback: if the library is missing or the GPU is not a gfx950 device, calls
raise.

Entry points mirror the C ABI in ``include/moe.h``: :func:`workspace_bytes`,
:func:`route`, :func:`forward`, :func:`bias_update`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

__all__ = ["F32", "BF16", "E4M3", "MoeError", "lib", "lib_path", "make_cfg", "cfg_from",
           "workspace_bytes", "alloc_workspace", "alloc_routing", "route", "forward",
           "forward_noalloc", "NOALLOC_SCRATCH_BYTES",
           "bias_update", "quantize_1x128", "balance_loss", "backward", "backward_workspace_bytes",
           "alloc_backward_workspace", "profile_enable", "profile_read",
           "status_string", "abi_version", "EXPORTED_SYMBOLS"]

F32, BF16, E4M3 = 0, 1, 2
_DT_NAME = {"f32": F32, "bf16": BF16, "e4m3": E4M3}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16, E4M3: torch.uint8}

EXPORTED_SYMBOLS = ("moe_workspace_bytes", "moe_route", "moe_forward", "moe_bias_update",
                    "moe_profile_enable", "moe_profile_read", "moe_profile_kernel_name",
                    "moe_status_string", "moe_abi_version", "moe_quantize_1x128",
                    "moe_balance_loss", "moe_backward", "moe_backward_workspace_bytes",
                    "moe_forward_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20    # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libmoe_mi355x.so")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "inter", "n_experts", "n_groups",
                                              "topk_groups", "topk", "group_topn", "n_shared",
                                              "act_dtype", "w_dtype")]


class _Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_gate", "counts", "offsets",
                                               "perm", "slot", "tie_gap")]


class _Experts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up",
                                               "s_down")]


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m sparse_moe_layer_group_amd.build`")
        L = ctypes.CDLL(path)
        P, I64, SZ, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(_Cfg), I64]
        L.moe_workspace_bytes.restype = SZ
        L.moe_route.argtypes = [ctypes.POINTER(_Cfg), I64, P, P, P, ctypes.POINTER(_Routing), P, SZ, P]
        L.moe_route.restype = I32
        L.moe_forward.argtypes = [ctypes.POINTER(_Cfg), I64, P, P, P, ctypes.POINTER(_Experts), P, P,
                                  ctypes.POINTER(_Routing), P, SZ, P]
        L.moe_forward.restype = I32
        L.moe_forward_noalloc.argtypes = [ctypes.POINTER(_Cfg), I64, P, P, P,
                                          ctypes.POINTER(_Experts), P, P, ctypes.POINTER(_Routing),
                                          P]
        L.moe_forward_noalloc.restype = I32
        L.moe_bias_update.argtypes = [ctypes.POINTER(_Cfg), I64, P, P, ctypes.c_float, P]
        L.moe_bias_update.restype = I32
        L.moe_status_string.argtypes = [I32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = I32
        L.moe_profile_enable.argtypes = [I32]
        L.moe_profile_enable.restype = I32
        L.moe_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32),
                                       I32]
        L.moe_profile_read.restype = I32
        L.moe_balance_loss.argtypes = [ctypes.POINTER(_Cfg), I64, ctypes.c_int32, P, P,
                                       ctypes.c_float, P, P, P, P, SZ, P]
        L.moe_balance_loss.restype = I32
        L.moe_backward_workspace_bytes.argtypes = [ctypes.POINTER(_Cfg), I64]
        L.moe_backward_workspace_bytes.restype = SZ
        L.moe_backward.argtypes = [ctypes.POINTER(_Cfg), I64, P, P, P, ctypes.POINTER(_Experts), P,
                                   P, P, P, P, P, P, SZ, P]
        L.moe_backward.restype = I32
        L.moe_quantize_1x128.argtypes = [P, I64, ctypes.c_int32, P, P, P]
        L.moe_quantize_1x128.restype = I32
        L.moe_profile_kernel_name.argtypes = [I32]
        L.moe_profile_kernel_name.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def profile_enable(on: bool = True) -> None:
    """Bracket every kernel launch with HIP events on the caller's stream."""
    lib().moe_profile_enable(1 if on else 0)


def profile_read() -> Dict[str, tuple]:
    """{kernel name: (total ms, launches)} since the last read; clears the record."""
    L = lib()
    n = L.moe_profile_read(None, None, 0)
    if n < 0:
        raise MoeError(n, "moe_profile_read")
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    rc = L.moe_profile_read(ms, cnt, n)
    if rc < 0:
        raise MoeError(rc, "moe_profile_read")
    return {L.moe_profile_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().moe_abi_version())


def make_cfg(hidden: int, inter: int, n_experts: int, n_groups: int, topk_groups: int, topk: int,
             group_topn: int = 2, n_shared: int = 1, act_dtype=BF16, w_dtype=BF16) -> _Cfg:
    act = _DT_NAME.get(act_dtype, act_dtype)
    wdt = _DT_NAME.get(w_dtype, w_dtype)
    return _Cfg(hidden, inter, n_experts, n_groups, topk_groups, topk, group_topn, n_shared, act,
                wdt)


def cfg_from(obj) -> _Cfg:
    """moe_cfg from any object with the same attribute names (dtypes as names or codes)."""
    return make_cfg(obj.hidden, obj.inter, obj.n_experts, obj.n_groups, obj.topk_groups, obj.topk,
                    obj.group_topn, obj.n_shared, obj.act_dtype, obj.w_dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _check(t: torch.Tensor, name: str, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_bytes(cfg: _Cfg, T: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg), int(T)))


def alloc_workspace(cfg: _Cfg, T: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(cfg, T)
    if n == 0 and T > 0:
        raise MoeError(-2, "workspace_bytes")
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def alloc_routing(cfg: _Cfg, T: int, device="cuda", tie_gap: bool = True) -> Dict[str, torch.Tensor]:
    K, E = cfg.topk, cfg.n_experts
    i32 = dict(dtype=torch.int32, device=device)
    out = {
        "topk_idx": torch.empty((T, K), **i32),
        "topk_gate": torch.empty((T, K), dtype=torch.float32, device=device),
        "counts": torch.empty((E,), **i32),
        "offsets": torch.empty((E + 1,), **i32),
        "perm": torch.empty((T * K,), **i32),
        "slot": torch.empty((T * K,), **i32),
    }
    if tie_gap:
        out["tie_gap"] = torch.empty((T,), dtype=torch.float32, device=device)
    return out


def _routing_struct(cfg: _Cfg, T: int, out: Dict[str, torch.Tensor]) -> _Routing:
    K, E = cfg.topk, cfg.n_experts
    for name, dt, shp in (("topk_idx", torch.int32, (T, K)), ("topk_gate", torch.float32, (T, K)),
                          ("counts", torch.int32, (E,)), ("offsets", torch.int32, (E + 1,)),
                          ("perm", torch.int32, (T * K,)), ("slot", torch.int32, (T * K,))):
        _check(out.get(name), name, dt, shp)
    gap = out.get("tie_gap")
    if gap is not None:
        _check(gap, "tie_gap", torch.float32, (T,))
    return _Routing(*[out[n].data_ptr() if out.get(n) is not None else None
                      for n in ("topk_idx", "topk_gate", "counts", "offsets", "perm", "slot",
                                "tie_gap")])


def route(cfg: _Cfg, x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
          out: Dict[str, torch.Tensor], ws: torch.Tensor, stream=None) -> None:
    """moe_route: router, node-limited selection, gates and expert permutation into ``out``."""
    T = x.shape[0]
    _check(x, "x", _TORCH_DT[cfg.act_dtype], (T, cfg.hidden))
    _check(w_router, "w_router", torch.float32, (cfg.hidden, cfg.n_experts))
    _check(bias, "bias", torch.float32, (cfg.n_experts,))
    r = _routing_struct(cfg, T, out)
    rc = lib().moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(r),
                         _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream))
    if rc != 0:
        raise MoeError(rc, "moe_route")


def _forward_args(cfg: _Cfg, x, w_router, bias, experts, y, residual, out):
    """Checked pointer arguments shared by moe_forward and moe_forward_noalloc."""
    T = x.shape[0]
    H, I, n = cfg.hidden, cfg.inter, cfg.n_experts + cfg.n_shared
    adt, wdt = _TORCH_DT[cfg.act_dtype], _TORCH_DT[cfg.w_dtype]
    _check(x, "x", adt, (T, H))
    _check(y, "y", adt, (T, H))
    if residual is not None:
        _check(residual, "residual", adt, (T, H))
    _check(w_router, "w_router", torch.float32, (H, cfg.n_experts))
    _check(bias, "bias", torch.float32, (cfg.n_experts,))
    _check(experts.get("w_gate"), "w_gate", wdt, (n, I, H))
    _check(experts.get("w_up"), "w_up", wdt, (n, I, H))
    _check(experts.get("w_down"), "w_down", wdt, (n, H, I))
    if cfg.w_dtype == E4M3:
        _check(experts.get("s_gate"), "s_gate", torch.float32, (n, I // 128, H // 128))
        _check(experts.get("s_up"), "s_up", torch.float32, (n, I // 128, H // 128))
        _check(experts.get("s_down"), "s_down", torch.float32, (n, H // 128, I // 128))
    ex = _Experts(*[experts[k].data_ptr() if experts.get(k) is not None else None
                    for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")])
    r = _routing_struct(cfg, T, out) if out is not None else None
    return ex, r


def forward(cfg: _Cfg, x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
            experts: Dict[str, torch.Tensor], y: torch.Tensor, ws: torch.Tensor,
            residual: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None,
            stream=None) -> None:
    """moe_forward: the whole layer into ``y`` (routing into ``out`` when given)."""
    ex, r = _forward_args(cfg, x, w_router, bias, experts, y, residual, out)
    rc = lib().moe_forward(ctypes.byref(cfg), x.shape[0], _ptr(x), _ptr(w_router), _ptr(bias),
                           ctypes.byref(ex), _ptr(residual), _ptr(y),
                           ctypes.byref(r) if r is not None else None, _ptr(ws),
                           ws.numel() if ws is not None else 0, _stream(stream))
    if rc != 0:
        raise MoeError(rc, "moe_forward")


def forward_noalloc(cfg: _Cfg, x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
                    experts: Dict[str, torch.Tensor], y: torch.Tensor,
                    residual: Optional[torch.Tensor] = None,
                    out: Optional[Dict[str, torch.Tensor]] = None, stream=None) -> None:
    """moe_forward_noalloc: moe_forward with the library's static device scratch (no workspace)."""
    ex, r = _forward_args(cfg, x, w_router, bias, experts, y, residual, out)
    rc = lib().moe_forward_noalloc(ctypes.byref(cfg), x.shape[0], _ptr(x), _ptr(w_router),
                                   _ptr(bias), ctypes.byref(ex), _ptr(residual), _ptr(y),
                                   ctypes.byref(r) if r is not None else None, _stream(stream))
    if rc != 0:
        raise MoeError(rc, "moe_forward_noalloc")


def backward_workspace_bytes(cfg: _Cfg, T: int) -> int:
    """moe_backward_workspace_bytes (0: unsupported configuration)."""
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(cfg), int(T)))


def alloc_backward_workspace(cfg: _Cfg, T: int, device) -> torch.Tensor:
    n = backward_workspace_bytes(cfg, T)
    if n == 0:
        raise MoeError(-2, "moe_backward_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def backward(cfg: _Cfg, x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
             experts: Dict[str, torch.Tensor], dy: torch.Tensor, dx: torch.Tensor,
             dw_router: torch.Tensor, dw_gate: torch.Tensor, dw_up: torch.Tensor,
             dw_down: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """moe_backward: gradients of <dy, y> into dx, dw_router and the expert weight gradients."""
    T = x.shape[0]
    H, I, E, n = cfg.hidden, cfg.inter, cfg.n_experts, cfg.n_experts + cfg.n_shared
    adt, wdt = _TORCH_DT[cfg.act_dtype], _TORCH_DT[cfg.w_dtype]
    for t, name in ((x, "x"), (dy, "dy"), (dx, "dx")):
        _check(t, name, adt, (T, H))
    _check(w_router, "w_router", torch.float32, (H, E))
    _check(bias, "bias", torch.float32, (E,))
    _check(experts.get("w_gate"), "w_gate", wdt, (n, I, H))
    _check(experts.get("w_up"), "w_up", wdt, (n, I, H))
    _check(experts.get("w_down"), "w_down", wdt, (n, H, I))
    _check(dw_router, "dw_router", torch.float32, (H, E))
    _check(dw_gate, "dw_gate", torch.float32, (n, I, H))
    _check(dw_up, "dw_up", torch.float32, (n, I, H))
    _check(dw_down, "dw_down", torch.float32, (n, H, I))
    if cfg.w_dtype == E4M3:
        _check(experts.get("s_gate"), "s_gate", torch.float32, (n, I // 128, H // 128))
        _check(experts.get("s_up"), "s_up", torch.float32, (n, I // 128, H // 128))
        _check(experts.get("s_down"), "s_down", torch.float32, (n, H // 128, I // 128))
    ex = _Experts(*[experts[k].data_ptr() if experts.get(k) is not None else None
                    for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")])
    rc = lib().moe_backward(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(bias),
                            ctypes.byref(ex), _ptr(dy), _ptr(dx), _ptr(dw_router), _ptr(dw_gate),
                            _ptr(dw_up), _ptr(dw_down), _ptr(ws),
                            ws.numel() if ws is not None else 0, _stream(stream))
    if rc != 0:
        raise MoeError(rc, "moe_backward")


def balance_loss(cfg: _Cfg, x: torch.Tensor, w_router: torch.Tensor, seq_len: int, alpha: float,
                 loss: torch.Tensor, ws: torch.Tensor, f: Optional[torch.Tensor] = None,
                 p: Optional[torch.Tensor] = None, stream=None) -> None:
    """moe_balance_loss: sequence-wise balance loss per sequence of seq_len tokens into ``loss``."""
    T = x.shape[0]
    H, E = cfg.hidden, cfg.n_experts
    _check(x, "x", _TORCH_DT[cfg.act_dtype], (T, H))
    _check(w_router, "w_router", torch.float32, (H, E))
    n_seq = T // seq_len if seq_len > 0 else 0
    _check(loss, "loss", torch.float32, (n_seq,))
    for t, name in ((f, "f"), (p, "p")):
        if t is not None:
            _check(t, name, torch.float32, (n_seq, E))
    rc = lib().moe_balance_loss(ctypes.byref(cfg), T, int(seq_len), _ptr(x), _ptr(w_router),
                                ctypes.c_float(alpha), _ptr(loss), _ptr(f), _ptr(p), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream))
    if rc != 0:
        raise MoeError(rc, "moe_balance_loss")


def quantize_1x128(x: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """moe_quantize_1x128: bf16 [R][C] -> E4M3 codes (uint8 [R][C]) and float32 scales [R][C/128]."""
    R, C = x.shape
    _check(x, "x", torch.bfloat16, (R, C))
    _check(q, "q", torch.uint8, (R, C))
    _check(scales, "scales", torch.float32, (R, C // 128))
    rc = lib().moe_quantize_1x128(_ptr(x), int(R), int(C), _ptr(q), _ptr(scales), _stream(stream))
    if rc != 0:
        raise MoeError(rc, "moe_quantize_1x128")


def bias_update(cfg: _Cfg, T: int, counts: torch.Tensor, bias: torch.Tensor, gamma: float,
                stream=None) -> None:
    """moe_bias_update: loss-free balancing step on ``bias`` in place."""
    _check(counts, "counts", torch.int32, (cfg.n_experts,))
    _check(bias, "bias", torch.float32, (cfg.n_experts,))
    rc = lib().moe_bias_update(ctypes.byref(cfg), int(T), _ptr(counts), _ptr(bias),
                               ctypes.c_float(gamma), _stream(stream))
    if rc != 0:
        raise MoeError(rc, "moe_bias_update")
