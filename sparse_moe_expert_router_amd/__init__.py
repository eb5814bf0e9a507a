"""Python binding of libmoe.so, the gfx950 HIP library for one sparse MoE FFN layer forward.

Argument marshalling only: every step of the layer runs in the library's HIP kernels.  Tensors
are torch tensors on the GPU (torch supplies device memory and the current stream).  There is no
fallback: if libmoe.so is missing, or a call returns an error status, this module raises.

The C ABI is declared and documented in include/moe.h; names here match it.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_SANITIZE=1 loads the build whose host code carries AddressSanitizer / UBSan checks
LIB_PATH = os.path.join(_PKG, "libmoe_san.so" if os.environ.get("MOE_SANITIZE") == "1" else "libmoe.so")

X_F32, X_BF16 = 0, 1
W_Q8_0, W_I8_ROW, W_E2M1_G16, W_Q8_0_TILED, W_I8_ROW_TILED = 0, 1, 2, 3, 4
W_FP8_ROW, W_FP8_ROW_TILED = 5, 6
ACT_SWIGLU, ACT_RELU2 = 0, 1
F_ZERO_SKIP, F_PREFILL_I8, F_PREFILL_FP8 = 1, 4, 8
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5
STATIC_WORKSPACE_BYTES = 64 << 20       # MOE_STATIC_WORKSPACE_BYTES: the buffer of layer_forward_static

EXPORTED = ("moe_workspace_bytes", "moe_route_workspace_bytes", "moe_route", "moe_permute",
            "moe_layer_forward", "moe_layer_forward_static", "moe_experts_forward", "moe_quantize_rows_i8", "moe_quantize_rows_fp8",
            "moe_repack_experts", "moe_read_intermediates",
            "moe_status_str", "moe_abi_version", "moe_profile_enable", "moe_profile_collect",
            "moe_profile_reset", "moe_profile_kinds", "moe_profile_get")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("gate_up", ctypes.c_void_p),
                ("gate_up_scales", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("down_scales", ctypes.c_void_p), ("n_shared", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python sparse_moe_expert_router_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        pex = ctypes.POINTER(Experts)
        L.moe_workspace_bytes.argtypes = [i32, i32, pex, i32, u32]
        L.moe_workspace_bytes.restype = sz
        L.moe_route_workspace_bytes.argtypes = [i32, i32]
        L.moe_route_workspace_bytes.restype = sz
        L.moe_route.argtypes = [vp, i32, i32, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.moe_route.restype = i32
        L.moe_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.moe_permute.restype = i32
        L.moe_layer_forward.argtypes = [vp, i32, i32, vp, vp, pex, i32, i32, u32, vp, vp, vp, vp,
                                        sz, vp]
        L.moe_layer_forward.restype = i32
        L.moe_layer_forward_static.argtypes = [vp, i32, i32, vp, vp, pex, i32, i32, u32, vp, vp, vp, vp]
        L.moe_layer_forward_static.restype = i32
        L.moe_experts_forward.argtypes = [vp, i32, i32, vp, vp, pex, i32, i32, u32, vp, vp, sz, vp]
        L.moe_experts_forward.restype = i32
        L.moe_repack_experts.argtypes = [pex, i32, pex, vp]
        L.moe_repack_experts.restype = i32
        L.moe_quantize_rows_i8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.moe_quantize_rows_i8.restype = i32
        L.moe_quantize_rows_fp8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.moe_quantize_rows_fp8.restype = i32
        L.moe_read_intermediates.argtypes = [i32, i32, pex, i32, u32, i32, vp, sz, vp, vp, vp, vp]
        L.moe_read_intermediates.restype = i32
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_abi_version.restype = i32
        L.moe_profile_enable.argtypes = [i32]
        L.moe_profile_enable.restype = i32
        L.moe_profile_collect.restype = i32
        L.moe_profile_reset.restype = None
        L.moe_profile_kinds.restype = i32
        L.moe_profile_get.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p),
                                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
        L.moe_profile_get.restype = i32
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != OK:
        raise MoeError(fn, status, lib().moe_status_str(status).decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _xtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return X_BF16
    if x.dtype == torch.float32:
        return X_F32
    raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")


def experts_struct(ex: dict) -> Experts:
    """The C struct for an experts dict (fmt, E, d_model, d_ff, four device tensors, n_shared)."""
    return Experts(int(ex["fmt"]), int(ex["E"]), int(ex["d_model"]), int(ex["d_ff"]),
                   ex["gate_up"].data_ptr(), ex["gate_up_scales"].data_ptr(),
                   ex["down"].data_ptr(), ex["down_scales"].data_ptr(), int(ex.get("n_shared", 0)))


def workspace_bytes(T: int, k: int, experts: dict, act: int, flags: int = 0) -> int:
    s = Experts(int(experts["fmt"]), int(experts["E"]), int(experts["d_model"]),
                int(experts["d_ff"]), None, None, None, None, int(experts.get("n_shared", 0)))
    return int(lib().moe_workspace_bytes(T, k, ctypes.byref(s), act, flags))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def route(x, w_router, bias, k: int, ws=None):
    """moe_route: (topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    T, d = x.shape
    E = w_router.shape[0]
    need = int(lib().moe_route_workspace_bytes(T, E))
    ws = alloc_workspace(need, x.device) if ws is None else ws
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check("moe_route", lib().moe_route(_p(x), _xtype(x), T, d, _p(w_router), _p(bias), E, k,
                                        _p(idx), _p(w), _p(ws), ws.numel(), _stream()))
    return idx, w


def permute(topk_idx, E: int):
    """moe_permute: (counts [E], offsets [E+1], perm [P], inv [P]), all int32."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    _check("moe_permute", lib().moe_permute(_p(topk_idx), T, k, E, _p(counts), _p(offsets),
                                            _p(perm), _p(inv), _stream()))
    return counts, offsets, perm, inv


def layer_forward(x, w_router, bias, experts: dict, k: int, act: int, flags: int = 0, out=None,
                  ws=None, want_routing: bool = False):
    """moe_layer_forward: out fp32 [T, d_model] (and the routing if want_routing)."""
    T = x.shape[0]
    s = experts_struct(experts)
    if ws is None:
        ws = alloc_workspace(workspace_bytes(T, k, experts, act, flags), x.device)
    out = torch.empty((T, int(experts["d_model"])), dtype=torch.float32, device=x.device) \
        if out is None else out
    idx = w = None
    if want_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check("moe_layer_forward",
           lib().moe_layer_forward(_p(x), _xtype(x), T, _p(w_router), _p(bias), ctypes.byref(s), k,
                                   act, flags, _p(out), _p(idx), _p(w), _p(ws), ws.numel(),
                                   _stream()))
    return (out, idx, w) if want_routing else out


def layer_forward_static(x, w_router, bias, experts: dict, k: int, act: int, flags: int = 0, out=None,
                         want_routing: bool = False):
    """moe_layer_forward_static: moe_layer_forward on the library's static device buffer (no
    workspace argument; the library allocates nothing).  Calls on one GPU must not overlap."""
    T = x.shape[0]
    s = experts_struct(experts)
    out = torch.empty((T, int(experts["d_model"])), dtype=torch.float32, device=x.device) \
        if out is None else out
    idx = w = None
    if want_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check("moe_layer_forward_static",
           lib().moe_layer_forward_static(_p(x), _xtype(x), T, _p(w_router), _p(bias), ctypes.byref(s), k,
                                          act, flags, _p(out), _p(idx), _p(w), _stream()))
    return (out, idx, w) if want_routing else out


def experts_forward(x, topk_idx, topk_w, experts: dict, act: int, flags: int = 0, out=None,
                    ws=None):
    """moe_experts_forward: out fp32 [T, d_model] for a given routing."""
    T, k = topk_idx.shape
    s = experts_struct(experts)
    if ws is None:
        ws = alloc_workspace(workspace_bytes(T, k, experts, act, flags), x.device)
    out = torch.empty((T, int(experts["d_model"])), dtype=torch.float32, device=x.device) \
        if out is None else out
    _check("moe_experts_forward",
           lib().moe_experts_forward(_p(x), _xtype(x), T, _p(topk_idx), _p(topk_w),
                                     ctypes.byref(s), k, act, flags, _p(out), _p(ws), ws.numel(),
                                     _stream()))
    return out


def repack_experts(experts: dict, act: int) -> dict:
    """moe_repack_experts: a tiled copy (new device tensors) of plain Q8_0 / I8_ROW / FP8_ROW experts."""
    fmt = int(experts["fmt"])
    tiled = {W_Q8_0: W_Q8_0_TILED, W_I8_ROW: W_I8_ROW_TILED, W_FP8_ROW: W_FP8_ROW_TILED}[fmt]
    out = dict(experts)
    out["fmt"] = tiled
    for key in ("gate_up", "gate_up_scales", "down", "down_scales"):
        out[key] = torch.empty_like(experts[key])
    src, dst = experts_struct(experts), experts_struct(out)
    _check("moe_repack_experts", lib().moe_repack_experts(ctypes.byref(src), act, ctypes.byref(dst),
                                                          _stream()))
    return out


def quantize_rows_i8(v):
    """moe_quantize_rows_i8: (q int8 [rows, cols], scale fp32 [rows])."""
    rows, cols = v.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=v.device)
    scale = torch.empty(rows, dtype=torch.float32, device=v.device)
    _check("moe_quantize_rows_i8", lib().moe_quantize_rows_i8(_p(v), _xtype(v), rows, cols, _p(q),
                                                              _p(scale), _stream()))
    return q, scale


def quantize_rows_fp8(v):
    """moe_quantize_rows_fp8: (q uint8 E4M3 codes [rows, cols], scale fp32 [rows])."""
    rows, cols = v.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=v.device)
    scale = torch.empty(rows, dtype=torch.float32, device=v.device)
    _check("moe_quantize_rows_fp8", lib().moe_quantize_rows_fp8(_p(v), _xtype(v), rows, cols, _p(q),
                                                                _p(scale), _stream()))
    return q, scale


def read_intermediates(T: int, k: int, experts: dict, act: int, flags: int, ws, with_router: bool = True):
    """moe_read_intermediates: the h (fp32 [T k + S T, d_ff], pair order) the last layer call on
    `ws` left there; with a prefill flag also (codes uint8 [rows, d_ff], row scales fp32 [rows])."""
    S = int(experts.get("n_shared", 0))
    rows, d_ff = T * k + S * T, int(experts["d_ff"])
    dev = ws.device
    h = torch.empty((rows, d_ff), dtype=torch.float32, device=dev)
    prefill = bool(flags & (F_PREFILL_I8 | F_PREFILL_FP8))
    hq = torch.empty((rows, d_ff), dtype=torch.uint8, device=dev) if prefill else None
    sh = torch.empty(rows, dtype=torch.float32, device=dev) if prefill else None
    s = experts_struct(experts)
    _check("moe_read_intermediates",
           lib().moe_read_intermediates(T, k, ctypes.byref(s), act, flags, 1 if with_router else 0, _p(ws),
                                        ws.numel(), _p(h), _p(hq), _p(sh), _stream()))
    return (h, hq, sh) if prefill else h


def profile_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events (see include/moe.h)."""
    _check("moe_profile_enable", lib().moe_profile_enable(1 if on else 0))


def profile_reset() -> None:
    lib().moe_profile_reset()


def profile_collect() -> dict:
    """Wait for the recorded events; {kernel name: (launches, total ms)} since the last reset."""
    L = lib()
    _check("moe_profile_collect", L.moe_profile_collect())
    res = {}
    for kind in range(L.moe_profile_kinds()):
        name = ctypes.c_char_p()
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check("moe_profile_get", L.moe_profile_get(kind, ctypes.byref(name), ctypes.byref(n),
                                                    ctypes.byref(ms)))
        if n.value:
            res[name.value.decode()] = (int(n.value), float(ms.value))
    return res
