"""CPU fp64 oracle for the sparse MoE FFN layer forward - TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product library (``sparse_moe_expert_router_amd``) never imports it, and it
shares no code with the HIP path: the arithmetic lives in ``moe_oracle.c`` (plain C, fp64 loops,
its own decoders), this file only marshals numpy arrays into it.

Every function states the passage it follows in ``moe_oracle.c``'s header.  Pins that check the
oracle against things other than itself live in ``tests/test_oracle_pins.py``.  Functions still
"parity unpinned": none (each is checked by a brute-force, closed-form, textbook or invariant pin).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_SANITIZE=1: a separate build with AddressSanitizer and UndefinedBehaviorSanitizer (run the
# process with gcc's libasan preloaded; see the command in the package's design notes)
_SANITIZE = os.environ.get("MOE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]

X_F32, X_BF16 = 0, 1
W_Q8_0, W_I8_ROW, W_E2M1_G16, W_FP8_ROW = 0, 1, 2, 5
ACT_SWIGLU, ACT_RELU2 = 0, 1


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas", *(_SAN_FLAGS if _SANITIZE else []),
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("gate_up", ctypes.c_void_p),
                ("gate_up_scales", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("down_scales", ctypes.c_void_p), ("n_shared", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.oracle_route.argtypes = [vp, i32, i32, i32, vp, vp, i32, i32, vp, vp, vp, vp]
        lib.oracle_route.restype = i32
        lib.oracle_permute.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        lib.oracle_permute.restype = i32
        lib.oracle_experts_forward.argtypes = [vp, i32, i32, vp, vp, i32, ctypes.POINTER(_Experts),
                                               i32, vp, i32, vp, vp]
        lib.oracle_experts_forward.restype = i32
        lib.oracle_zero_skip_down.argtypes = [vp, i32, vp, vp, i32, ctypes.POINTER(_Experts), vp, vp]
        lib.oracle_zero_skip_down.restype = i32
        lib.oracle_experts_forward_i8act.argtypes = [vp, i32, i32, vp, vp, i32,
                                                     ctypes.POINTER(_Experts), vp, i32, vp, vp, vp, vp]
        lib.oracle_experts_forward_i8act.restype = i32
        lib.oracle_rule_q.argtypes = [vp, i32, vp, vp]
        lib.oracle_rule_q.restype = None
        lib.oracle_rule_q8.argtypes = [vp, i32, vp, vp]
        lib.oracle_rule_q8.restype = None
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint
        lib.oracle_experts_forward_f8act.argtypes = [vp, i32, i32, vp, vp, i32,
                                                     ctypes.POINTER(_Experts), vp, i32, vp, vp, vp, vp]
        lib.oracle_experts_forward_f8act.restype = i32
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_e2m1_value.argtypes = [ctypes.c_uint]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_get_threads.restype = i32
        _lib = lib
    return _lib


def _np(a, dtype=None):
    """A C-contiguous numpy array from a numpy array or a CPU torch tensor (bf16 as uint16)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            elif a.dtype == torch.float16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        a = np.ascontiguousarray(a.astype(dtype))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _experts_struct(ex: dict):
    arrays = [_np(ex[k]) for k in ("gate_up", "gate_up_scales", "down", "down_scales")]
    s = _Experts(int(ex["fmt"]), int(ex["E"]), int(ex["d_model"]), int(ex["d_ff"]),
                 *[a.ctypes.data_as(ctypes.c_void_p) for a in arrays], int(ex.get("n_shared", 0)))
    return s, arrays  # keep the arrays alive with the struct


def _x(x):
    xa = _np(x)
    xtype = X_BF16 if xa.dtype == np.uint16 else X_F32
    if xtype == X_F32:
        xa = _np(xa, np.float32)
    return xa, xtype


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def half_to_double(bits: int) -> float:
    return float(_load().oracle_half_to_double(int(bits)))


def bf16_to_double(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(int(bits)))


def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code)))


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code (NaN for 0x7F / 0xFF)."""
    return float(_load().oracle_e4m3_value(int(code)))


def e4m3_encode(v: float) -> int:
    """E4M3 code of an fp32 value: nearest, ties to even; NaN code past the 464 midpoint."""
    return int(_load().oracle_e4m3_encode(float(v)))


def route(x, w_router, bias, k: int):
    """Router: logits, softmax over all E, top-k by (logit desc, index asc), renormalised weights.

    Returns (idx int32 [T,k], w float64 [T,k], logits float64 [T,E], min_gap float64 [T]).
    """
    xa, xtype = _x(x)
    T, d = xa.shape
    wr = _np(w_router, np.float32)
    E = wr.shape[0]
    b = None if bias is None else _np(bias, np.float32)
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    logits = np.zeros((T, E), np.float64)
    gap = np.zeros((T,), np.float64)
    rc = _load().oracle_route(_ptr(xa), xtype, T, d, _ptr(wr), _ptr(b), E, k, _ptr(idx), _ptr(w),
                              _ptr(logits), _ptr(gap))
    if rc != 0:
        raise ValueError(f"oracle_route failed: {rc}")
    return idx, w, logits, gap


def permute(idx, E: int):
    """Expert histogram, exclusive prefix sum, and the stable (expert, pair id) order."""
    ia = _np(idx, np.int32).reshape(-1)
    P = ia.size
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(P, np.int32)
    inv = np.zeros(P, np.int32)
    rc = _load().oracle_permute(_ptr(ia), P, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv))
    if rc != 0:
        raise ValueError(f"oracle_permute failed: {rc}")
    return counts, offsets, perm, inv


def experts_forward(x, idx, w, experts: dict, act: int, o_list=None, want_h: bool = False):
    """fp64 layer output [T, d_model] (or [T, len(o_list)]) for given routing (idx, w).

    With ``experts["n_shared"] = S`` the arrays hold E + S experts and every token also goes
    through experts E .. E+S-1 with weight 1, after its k routed slots (h then has T*(k+S) rows).
    """
    xa, xtype = _x(x)
    T = xa.shape[0]
    ia = _np(idx, np.int32)
    k = ia.shape[1]
    wa = _np(w, np.float64)
    s, keep = _experts_struct(experts)
    ol = None if o_list is None else _np(o_list, np.int32)
    no = int(experts["d_model"]) if ol is None else ol.size
    out = np.zeros((T, no), np.float64)
    S = int(experts.get("n_shared", 0))
    h = np.zeros((T * (k + S), int(experts["d_ff"])), np.float64) if want_h else None
    rc = _load().oracle_experts_forward(_ptr(xa), xtype, T, _ptr(ia), _ptr(wa), k, ctypes.byref(s),
                                        act, _ptr(ol), 0 if ol is None else ol.size, _ptr(out), _ptr(h))
    if rc != 0:
        raise ValueError(f"oracle_experts_forward failed: {rc}")
    return (out, h) if want_h else out


def zero_skip_down(h, idx, w, experts: dict):
    """Zero-skip down of E2M1 neuron-major experts; returns (out [T,d], active groups per pair)."""
    ia = _np(idx, np.int32)
    T, k = ia.shape
    ha = _np(h, np.float64)
    wa = _np(w, np.float64)
    s, keep = _experts_struct(experts)
    out = np.zeros((T, int(experts["d_model"])), np.float64)
    act = np.zeros(T * (k + int(experts.get("n_shared", 0))), np.int32)
    rc = _load().oracle_zero_skip_down(_ptr(ha), T, _ptr(ia), _ptr(wa), k, ctypes.byref(s),
                                       _ptr(out), _ptr(act))
    if rc != 0:
        raise ValueError(f"oracle_zero_skip_down failed: {rc}")
    return out, act


def experts_forward_i8act(x, idx, w, experts: dict, o_list=None, want_h: bool = False):
    """Batched-prefill variant: int8 activations by rule Q, exact integer sums, rescale."""
    xa, xtype = _x(x)
    T, d = xa.shape
    ia = _np(idx, np.int32)
    k = ia.shape[1]
    wa = _np(w, np.float64)
    s, keep = _experts_struct(experts)
    ol = None if o_list is None else _np(o_list, np.int32)
    no = d if ol is None else ol.size
    out = np.zeros((T, no), np.float64)
    h = np.zeros((T * (k + int(experts.get("n_shared", 0))), int(experts["d_ff"])), np.float64) if want_h else None
    xq = np.zeros((T, d), np.int8)
    sx = np.zeros((T,), np.float32)
    rc = _load().oracle_experts_forward_i8act(_ptr(xa), xtype, T, _ptr(ia), _ptr(wa), k,
                                              ctypes.byref(s), _ptr(ol), 0 if ol is None else ol.size,
                                              _ptr(out), _ptr(h), _ptr(xq), _ptr(sx))
    if rc != 0:
        raise ValueError(f"oracle_experts_forward_i8act failed: {rc}")
    res = {"out": out, "xq": xq, "sx": sx}
    if want_h:
        res["h"] = h
    return res


def experts_forward_f8act(x, idx, w, experts: dict, o_list=None, want_h: bool = False):
    """fp8 batched-prefill variant (FP8_ROW experts, SwiGLU): E4M3 activations by rule Q8."""
    xa, xtype = _x(x)
    T, d = xa.shape
    ia = _np(idx, np.int32)
    k = ia.shape[1]
    wa = _np(w, np.float64)
    s, keep = _experts_struct(experts)
    ol = None if o_list is None else _np(o_list, np.int32)
    no = d if ol is None else ol.size
    out = np.zeros((T, no), np.float64)
    h = np.zeros((T * (k + int(experts.get("n_shared", 0))), int(experts["d_ff"])), np.float64) if want_h else None
    xq = np.zeros((T, d), np.uint8)
    sx = np.zeros((T,), np.float32)
    rc = _load().oracle_experts_forward_f8act(_ptr(xa), xtype, T, _ptr(ia), _ptr(wa), k,
                                              ctypes.byref(s), _ptr(ol), 0 if ol is None else ol.size,
                                              _ptr(out), _ptr(h), _ptr(xq), _ptr(sx))
    if rc != 0:
        raise ValueError(f"oracle_experts_forward_f8act failed: {rc}")
    res = {"out": out, "xq": xq, "sx": sx}
    if want_h:
        res["h"] = h
    return res


def rule_q8(v):
    """Rule Q8 on one fp32 vector: (E4M3 codes uint8, fp32 scale)."""
    va = _np(v, np.float32).reshape(-1)
    q = np.zeros(va.size, np.uint8)
    s = np.zeros(1, np.float32)
    _load().oracle_rule_q8(_ptr(va), va.size, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def rule_q(v):
    """Rule Q on one fp32 vector: (int8 codes, fp32 scale)."""
    va = _np(v, np.float32).reshape(-1)
    q = np.zeros(va.size, np.int8)
    s = np.zeros(1, np.float32)
    _load().oracle_rule_q(_ptr(va), va.size, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def layer_forward(x, w_router, bias, experts: dict, k: int, act: int, o_list=None):
    """Route, then the expert FFN and combine: the whole layer in fp64."""
    idx, w, logits, gap = route(x, w_router, bias, k)
    out = experts_forward(x, idx, w, experts, act, o_list=o_list)
    return {"out": out, "idx": idx, "w": w, "logits": logits, "min_gap": gap}
