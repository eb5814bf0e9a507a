"""Independent numpy fp64 brute-force evaluator of the MoE layer, for pinning the oracle.

It takes a different route from the oracle on purpose: whole matrices are dequantised with
numpy's own fp16 decoding and a table of E2M1 values read from the OCP spec fixture, every expert
is evaluated for every token with np.matmul, and the combine uses a dense [T, E] weight matrix
that is zero outside each token's top-k.  Routing uses math.fsum (correctly rounded sums of exact
products) and np.lexsort.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))


def e2m1_table() -> np.ndarray:
    vals = {}
    with open(os.path.join(_HERE, "golden", "e2m1_ocp_mx_v1.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)], np.float64)


def _f16(t) -> np.ndarray:
    return t.cpu().contiguous().numpy().astype(np.float64)  # torch fp16 -> numpy via float16


def x64(x) -> np.ndarray:
    return x.cpu().float().double().numpy()


def _unpack_nibbles(b: np.ndarray) -> np.ndarray:
    lo = b & 15
    hi = b >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant(experts: dict, act: int):
    """Dense fp64 (gate_up [E, rows, d], down [E, d, d_ff]) from the packed bytes."""
    fmt, E, d, dff = experts["fmt"], experts["E"], experts["d_model"], experts["d_ff"]
    gu, gus = experts["gate_up"].cpu(), experts["gate_up_scales"].cpu()
    dn, dns = experts["down"].cpu(), experts["down_scales"].cpu()
    if fmt == 0:  # Q8_0
        q = gu.numpy().astype(np.float64)
        s = np.repeat(_f16(gus), 32, axis=-1)
        wgu = q * s
        qd = dn.numpy().astype(np.float64)
        sd = np.repeat(_f16(dns), 32, axis=-1)
        wdn = qd * sd
    elif fmt == 1:  # per-row int8
        wgu = gu.numpy().astype(np.float64) * gus.numpy().astype(np.float64)[..., None]
        wdn = dn.numpy().astype(np.float64) * dns.numpy().astype(np.float64)[..., None]
    else:  # E2M1, up [E, rows, d/2] + fp16 [E, rows, d/16]; down neuron-major
        tab = e2m1_table()
        codes = _unpack_nibbles(gu.numpy())
        wgu = tab[codes] * np.repeat(_f16(gus), 16, axis=-1)
        v = tab[_unpack_nibbles(dn.numpy())]            # [E, d_ff, d]  (neuron f, output o)
        s = np.repeat(_f16(dns), 16, axis=1)            # [E, d_ff, d]  (S[f/16][o])
        wdn = np.transpose(v * s, (0, 2, 1))            # [E, d, d_ff]
    return wgu, wdn


def route(x, w_router, bias, k):
    """Exact logits (fsum of exact fp64 products), lexsort ranking, fp64 softmax weights."""
    X = x64(x)
    W = w_router.cpu().double().numpy()
    b = None if bias is None else bias.cpu().double().numpy()
    T, E = X.shape[0], W.shape[0]
    logits = np.empty((T, E))
    for t in range(T):
        for e in range(E):
            logits[t, e] = math.fsum((X[t] * W[e]).tolist()) + (0.0 if b is None else b[e])
    idx = np.empty((T, k), np.int64)
    wts = np.empty((T, k))
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))
        sel = order[:k]
        z = np.exp(logits[t] - logits[t].max())
        p = z / z.sum()
        idx[t] = sel
        wts[t] = p[sel] / p[sel].sum()
    return idx, wts, logits


def dense_layer(x, idx, wts, experts: dict, act: int):
    """Every expert on every token; combine with a dense [T, E] matrix zero outside the top-k."""
    wgu, wdn = dequant(experts, act)
    X = x64(x)
    E, dff = experts["E"], experts["d_ff"]
    T = X.shape[0]
    dense_w = np.zeros((T, E))
    for t in range(T):
        for j in range(idx.shape[1]):
            dense_w[t, idx[t, j]] += wts[t, j]
    pre = np.einsum("erd,td->ter", wgu, X)              # [T, E, rows]
    if act == 0:
        g, u = pre[..., :dff], pre[..., dff:]
        h = g / (1.0 + np.exp(-g)) * u
    else:
        u = pre
        h = np.where(u > 0, u * u, 0.0)
    y = np.einsum("eof,tef->teo", wdn, h)               # [T, E, d]
    return np.einsum("te,teo->to", dense_w, y), h


def rel_err(a, b) -> float:
    """Row-normwise relative error: max over rows of max|a-b| / max|b|."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.abs(a - b).max(axis=-1)
    den = np.abs(b).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if a.size else 0.0
