"""Seeded synthetic inputs for one sparse Mixture-of-Experts FFN layer.

This module only draws random numbers and packs them into the byte formats the layer reads
(Q8_0, per-row int8, E2M1 with an fp16 scale per 16 values, neuron-major down, per-row E4M3).  It holds none
of the layer's arithmetic: no dequantisation, no matmul, no routing.  Both the HIP path and the
CPU oracle consume the exact bytes produced here (the oracle gets a host copy).

Workloads are named for the model whose MoE layer they are shaped like:

* ``tiny``            - T=4, d_model=256, E=8, top-2, d_ff=512, SwiGLU, Q8_0, fp32 x, seed 0.
* ``gemma_decode``    - Gemma-4 26B-A4B shape: d_model=2816, E=128, top-8, d_ff=704, SwiGLU,
                        Q8_0 or per-row int8, bf16 x; T=1 or 8 (Squeezing a 26B MoE onto the
                        cheapest Inferentia instance, "Memory math"; Gemma 4 26B on a 13-year-old
                        Xeon, "Broken op path in non-AVX2 builds").
* ``m3_decode``       - MiniMax-M3 shape: d_model=6144, E=128, top-4, d_ff=3072, SwiGLU, Q8_0,
                        Zipf(1.1) router prior; T=1 or 32 (Why very large MoEs can be served
                        scattered, section 1 table).
* ``nemotron_latent`` - Nemotron latent MoE: d=1024, E=512, top-22, ungated ReLU^2, up 2688x1024,
                        down 1024x2688 stored neuron-major, E2M1 + fp16 scale per 16 values; T=1
                        (Running Nemotron-3.5-Super on an 8 GB GPU, "bytes per token" and "How the
                        engine works" step 4).
* ``gemma_prefill``   - T=2048 prompt tokens on the gemma_decode shape, per-row int8 weights,
                        Zipf(1.1) router prior.

Seeds: ``tiny`` uses seed 0; the others use ``1000 * workload_number + instance``.  Every tensor
gets its own stream: ``seed * 16 + tensor_number``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch

# Format / activation / x-type codes.  They mirror the enum values of the C ABI so the binding
# can pass them through unchanged.
FMT_Q8_0, FMT_I8_ROW, FMT_E2M1, FMT_FP8_ROW = 0, 1, 2, 5
ACT_SWIGLU, ACT_RELU2 = 0, 1
X_F32, X_BF16 = 0, 1

FMT_NAMES = {"q8_0": FMT_Q8_0, "i8_row": FMT_I8_ROW, "e2m1": FMT_E2M1, "fp8_row": FMT_FP8_ROW}
ACT_NAMES = {"swiglu": ACT_SWIGLU, "relu2": ACT_RELU2}

# Per-tensor stream numbers.
_TX, _TROUTER, _TGU, _TDOWN = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    number: int          # used in the seed
    T: int
    d_model: int
    E: int
    k: int
    d_ff: int
    act: int
    fmt: int
    xtype: int
    w_std: float
    router_std: float = 0.05
    zipf_s: Optional[float] = None
    instances: int = 1
    latent_bias_column: bool = False   # nemotron construction: x[-1] = 1, up[:, -1] large negative
    n_shared: int = 0                  # shared experts E .. E+n_shared-1 beside the routed ones

    @property
    def gate_up_rows(self) -> int:
        return (2 if self.act == ACT_SWIGLU else 1) * self.d_ff

    @property
    def pairs(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "tiny": Workload("tiny", 0, T=4, d_model=256, E=8, k=2, d_ff=512, act=ACT_SWIGLU,
                     fmt=FMT_Q8_0, xtype=X_F32, w_std=0.02),
    "gemma_decode": Workload("gemma_decode", 1, T=1, d_model=2816, E=128, k=8, d_ff=704,
                             act=ACT_SWIGLU, fmt=FMT_Q8_0, xtype=X_BF16, w_std=0.02, instances=30),
    "m3_decode": Workload("m3_decode", 2, T=1, d_model=6144, E=128, k=4, d_ff=3072,
                          act=ACT_SWIGLU, fmt=FMT_Q8_0, xtype=X_BF16, w_std=0.015, zipf_s=1.1,
                          instances=8),
    "nemotron_latent": Workload("nemotron_latent", 3, T=1, d_model=1024, E=512, k=22, d_ff=2688,
                                act=ACT_RELU2, fmt=FMT_E2M1, xtype=X_BF16, w_std=0.02,
                                instances=30, latent_bias_column=True),
    "gemma_prefill": Workload("gemma_prefill", 4, T=2048, d_model=2816, E=128, k=8, d_ff=704,
                              act=ACT_SWIGLU, fmt=FMT_I8_ROW, xtype=X_BF16, w_std=0.02,
                              zipf_s=1.1, instances=4),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. T=8, fmt=FMT_I8_ROW, E=16)."""
    return replace(WORKLOADS[name], **overrides)


def base_seed(w: Workload, instance: int) -> int:
    return 0 if w.number == 0 and instance == 0 else 1000 * w.number + instance


def _gen(device, seed: int, tensor: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + tensor)
    return g


# ---------------------------------------------------------------------------------------------
# Weight packers (generator side: fp32 draws -> bytes).  These choose the bytes; they are not part
# of what the layer computes, which only ever reads the bytes back.
# ---------------------------------------------------------------------------------------------

def pack_q8_0(w: torch.Tensor):
    """fp32 [..., N, K] -> (int8 [..., N, K], fp16 [..., N, K/32]).

    Block of 32 along K; scale d = fp16(max|w| / 127) rounded to nearest even; q = clamp(
    round_half_even(w / d), -127, 127); an all-zero block gets d = 0, q = 0.
    """
    *lead, N, K = w.shape
    assert K % 32 == 0
    b = w.reshape(*lead, N, K // 32, 32)
    amax = b.abs().amax(dim=-1)
    d16 = (amax / 127.0).to(torch.float16)
    d = d16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(d > 0, d, torch.ones_like(d))
    q = torch.where(d > 0, torch.round(b / safe), torch.zeros_like(b)).clamp_(-127, 127)
    return q.to(torch.int8).reshape(*lead, N, K), d16


def pack_i8_row(w: torch.Tensor):
    """fp32 [..., N, K] -> (int8 [..., N, K], fp32 [..., N]); s = max|row| / 127 (fp32)."""
    amax = w.abs().amax(dim=-1)
    s = amax / 127.0
    safe = torch.where(s > 0, s, torch.ones_like(s)).unsqueeze(-1)
    q = torch.where(s.unsqueeze(-1) > 0, torch.round(w / safe), torch.zeros_like(w)).clamp_(-127, 127)
    return q.to(torch.int8), s.to(torch.float32)


def pack_fp8_row(w: torch.Tensor):
    """fp32 [..., N, K] -> (uint8 E4M3 codes [..., N, K], fp32 [..., N]); s = max|row| / 448.

    Codes are torch's float8_e4m3fn conversion of w / s (nearest, ties to even); an all-zero row
    gets s = 0 and codes 0.
    """
    amax = w.abs().amax(dim=-1)
    s = amax / 448.0
    safe = torch.where(s > 0, s, torch.ones_like(s)).unsqueeze(-1)
    r = torch.where(s.unsqueeze(-1) > 0, w / safe, torch.zeros_like(w))
    return r.to(torch.float8_e4m3fn).view(torch.uint8), s.to(torch.float32)


# Representable E2M1 magnitudes in code order 0..7 (OCP Microscaling Formats v1.0, FP4 E2M1).
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _e2m1_codes(r: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code (4-bit, sign in bit 3) for each value of r; ties go to the even code."""
    a = r.abs()
    mag = torch.zeros_like(a, dtype=torch.int32)
    # Thresholds between consecutive magnitudes; at an exact midpoint pick the even code.
    mids = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for i, (m, even_code) in enumerate(mids):
        upper = i + 1
        above = a > m
        at = a == m
        mag = torch.where(above, torch.full_like(mag, upper), mag)
        mag = torch.where(at, torch.full_like(mag, even_code), mag)
    sign = (r < 0) & (mag > 0)
    return (mag | (sign.to(torch.int32) << 3)).to(torch.uint8)


def pack_e2m1_g16(w: torch.Tensor):
    """fp32 [..., N, K] -> (uint8 [..., N, K/2], fp16 [..., N, K/16], codes uint8 [..., N, K]).

    One fp16 scale per 16 contiguous values along K: s = fp16(max|w| / 6); code = nearest E2M1
    value of w / s.  Two codes per byte, element 2i in the low nibble and 2i+1 in the high nibble.
    """
    *lead, N, K = w.shape
    assert K % 16 == 0
    g = w.reshape(*lead, N, K // 16, 16)
    amax = g.abs().amax(dim=-1)
    s16 = (amax / 6.0).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    r = torch.where(s > 0, g / safe, torch.zeros_like(g))
    codes = _e2m1_codes(r).reshape(*lead, N, K)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.contiguous(), s16, codes


def neuron_major_down(codes: torch.Tensor, s16: torch.Tensor):
    """Re-lay an E2M1 down matrix out neuron-major (a pure byte permutation).

    codes [E, d_model, d_ff] (one 4-bit code per byte, scale group of 16 along d_ff) and
    s16 [E, d_model, d_ff/16] become
      V [E, d_ff, d_model/2]  - neuron f's d_model codes contiguous, output 2i in the low nibble;
      S [E, d_ff/16, d_model] - the scale of (output o, neurons 16g..16g+15) at S[g][o].
    """
    cT = codes.transpose(-1, -2).contiguous()           # [E, d_ff, d_model]
    V = (cT[..., 0::2] | (cT[..., 1::2] << 4)).contiguous()
    S = s16.transpose(-1, -2).contiguous()              # [E, d_ff/16, d_model]
    return V, S


def zipf_bias(E: int, s: float) -> torch.Tensor:
    """Log of a Zipf(s) prior over experts, up to its normaliser: b[e] = -s * ln(e + 1)."""
    return torch.tensor([-s * math.log(e + 1) for e in range(E)], dtype=torch.float64).to(torch.float32)


# ---------------------------------------------------------------------------------------------

def _chunks(E: int, per_expert_elems: int, budget_elems: int = 1 << 27):
    step = max(1, budget_elems // max(1, per_expert_elems))
    for e0 in range(0, E, step):
        yield e0, min(E, e0 + step)


def make_router(w: Workload, instance: int = 0, device="cpu"):
    """The router of one layer instance: (w_router fp32 [E, d], bias fp32 [E] or None), the same
    bytes make_layer gives (the router has a generator stream of its own)."""
    device = torch.device(device)
    g_r = _gen(device, base_seed(w, instance), _TROUTER)
    w_router = torch.randn((w.E, w.d_model), generator=g_r, device=device, dtype=torch.float32) * w.router_std
    bias = zipf_bias(w.E, w.zipf_s).to(device) if w.zipf_s else None
    return w_router, bias


def make_layer(w: Workload, instance: int = 0, device="cpu", keep_codes: bool = False) -> dict:
    """Generate one layer instance (router + all experts) on ``device``.

    Returns a dict with the workload, ``w_router`` fp32 [E, d], ``bias`` fp32 [E] or None and an
    ``experts`` dict holding the four expert arrays in the format named by ``w.fmt``.
    """
    device = torch.device(device)
    seed = base_seed(w, instance)
    E, d, dff = w.E, w.d_model, w.d_ff
    NE = E + w.n_shared                       # expert arrays: the routed experts, then the shared
    rows = w.gate_up_rows

    w_router, bias = make_router(w, instance, device)

    g_gu = _gen(device, seed, _TGU)
    g_dn = _gen(device, seed, _TDOWN)
    if w.fmt == FMT_Q8_0:
        gu = torch.empty((NE, rows, d), dtype=torch.int8, device=device)
        gus = torch.empty((NE, rows, d // 32), dtype=torch.float16, device=device)
        dn = torch.empty((NE, d, dff), dtype=torch.int8, device=device)
        dns = torch.empty((NE, d, dff // 32), dtype=torch.float16, device=device)
    elif w.fmt in (FMT_I8_ROW, FMT_FP8_ROW):
        cdt = torch.int8 if w.fmt == FMT_I8_ROW else torch.uint8
        gu = torch.empty((NE, rows, d), dtype=cdt, device=device)
        gus = torch.empty((NE, rows), dtype=torch.float32, device=device)
        dn = torch.empty((NE, d, dff), dtype=cdt, device=device)
        dns = torch.empty((NE, d), dtype=torch.float32, device=device)
    elif w.fmt == FMT_E2M1:
        gu = torch.empty((NE, rows, d // 2), dtype=torch.uint8, device=device)
        gus = torch.empty((NE, rows, d // 16), dtype=torch.float16, device=device)
        dn = torch.empty((NE, dff, d // 2), dtype=torch.uint8, device=device)
        dns = torch.empty((NE, dff // 16, d), dtype=torch.float16, device=device)
    else:
        raise ValueError(w.fmt)

    bias_val = -1.44 * w.w_std * math.sqrt(d - 1)
    for e0, e1 in _chunks(NE, rows * d):
        wgu = torch.randn((e1 - e0, rows, d), generator=g_gu, device=device, dtype=torch.float32) * w.w_std
        if w.latent_bias_column:
            wgu[:, :, d - 1] = bias_val
        if w.fmt == FMT_Q8_0:
            gu[e0:e1], gus[e0:e1] = pack_q8_0(wgu)
        elif w.fmt == FMT_I8_ROW:
            gu[e0:e1], gus[e0:e1] = pack_i8_row(wgu)
        elif w.fmt == FMT_FP8_ROW:
            gu[e0:e1], gus[e0:e1] = pack_fp8_row(wgu)
        else:
            gu[e0:e1], gus[e0:e1], _ = pack_e2m1_g16(wgu)
        del wgu
    for e0, e1 in _chunks(NE, d * dff):
        wdn = torch.randn((e1 - e0, d, dff), generator=g_dn, device=device, dtype=torch.float32) * w.w_std
        if w.fmt == FMT_Q8_0:
            dn[e0:e1], dns[e0:e1] = pack_q8_0(wdn)
        elif w.fmt == FMT_I8_ROW:
            dn[e0:e1], dns[e0:e1] = pack_i8_row(wdn)
        elif w.fmt == FMT_FP8_ROW:
            dn[e0:e1], dns[e0:e1] = pack_fp8_row(wdn)
        else:
            _, s16, codes = pack_e2m1_g16(wdn)
            dn[e0:e1], dns[e0:e1] = neuron_major_down(codes, s16)
        del wdn

    return {
        "workload": w, "instance": instance, "seed": seed,
        "w_router": w_router, "bias": bias,
        "experts": {"fmt": w.fmt, "E": E, "d_model": d, "d_ff": dff, "n_shared": w.n_shared,
                    "gate_up": gu, "gate_up_scales": gus, "down": dn, "down_scales": dns},
    }


def make_x(w: Workload, instance: int = 0, T: Optional[int] = None, device="cpu") -> torch.Tensor:
    """Activations [T, d_model]: N(0, 1), fp32 or bf16 (rounded to nearest even from fp32)."""
    T = w.T if T is None else T
    g = _gen(torch.device(device), base_seed(w, instance), _TX)
    x = torch.randn((T, w.d_model), generator=g, device=device, dtype=torch.float32)
    if w.latent_bias_column:
        x[:, w.d_model - 1] = 1.0
    return x.to(torch.bfloat16) if w.xtype == X_BF16 else x


def expert_bytes(w: Workload) -> int:
    """Bytes of one expert's four arrays in the workload's format."""
    rows, d, dff = w.gate_up_rows, w.d_model, w.d_ff
    if w.fmt == FMT_Q8_0:
        return rows * d + rows * (d // 32) * 2 + d * dff + d * (dff // 32) * 2
    if w.fmt in (FMT_I8_ROW, FMT_FP8_ROW):
        return rows * d + rows * 4 + d * dff + d * 4
    return rows * d // 2 + rows * (d // 16) * 2 + dff * d // 2 + (dff // 16) * d * 2


def to_host(layer: dict) -> dict:
    """A host (CPU) copy of a layer dict, for the oracle."""
    out = dict(layer)
    out["w_router"] = layer["w_router"].cpu()
    out["bias"] = None if layer["bias"] is None else layer["bias"].cpu()
    ex = dict(layer["experts"])
    for key in ("gate_up", "gate_up_scales", "down", "down_scales"):
        ex[key] = ex[key].cpu()
    out["experts"] = ex
    return out


def subset_experts(experts: dict, ids) -> dict:
    """Experts ``ids`` (a list) of a host expert dict, renumbered 0..len(ids)-1 (shared experts
    are kept, after them)."""
    S = int(experts.get("n_shared", 0))
    idx = torch.as_tensor(list(ids) + [int(experts["E"]) + s for s in range(S)], dtype=torch.long)
    ex = dict(experts)
    for key in ("gate_up", "gate_up_scales", "down", "down_scales"):
        ex[key] = experts[key].index_select(0, idx.to(experts[key].device)).contiguous()
    ex["E"] = len(ids)
    return ex
