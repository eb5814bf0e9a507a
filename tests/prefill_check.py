"""Parity check of the batched-prefill paths (test infrastructure of the GPU tests).

Batched prefill re-quantises h (fp32) per pair row.  The GPU's h and the oracle's agree to fp32
accumulation order, not bit for bit, so an element whose scaled value lies within that
disagreement of a rounding midpoint has two correct codes one step apart.  This check marks
every such element of the oracle's h (window: H_REL * |v| + H_ABS * max|v| in scaled units) and bounds, per output,
what flipping all of them could change; the GPU output must match to the stated tolerance
beyond that bound.  Unique parts stay exact: the routing ids and the x codes.
"""
import numpy as np

import moe_inputs as mi
import oracle

# Measured on the Gemma-shaped prefill (d_ff = 704, 633,600 h values): the GPU's h differs from the
# oracle's by at most 2.6e-7 of the row maximum (int8 and E4M3 paths alike), an absolute-scale
# difference; the window keeps 7x that in scaled units, plus a small relative term.
H_REL, H_ABS = 2e-6, 2e-6
_E4M3_MAG = None


def _e4m3_mags():
    global _E4M3_MAG
    if _E4M3_MAG is None:
        _E4M3_MAG = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)  # increasing
    return _E4M3_MAG


def _ambiguous_codes(row, fp8):
    """(mask of elements near a midpoint, their code step in h units) for one fp32 h row."""
    a = np.float32(np.abs(row).max())
    if a == 0:
        return np.zeros(row.size, bool), np.zeros(row.size)
    top = np.float32(448.0 if fp8 else 127.0)
    inv = top / a
    v = (row * inv).astype(np.float64)                    # fp32 products, as the rule takes them
    mag = np.abs(v)
    window = H_REL * mag + H_ABS * float(top)
    if fp8:
        q, sc = oracle.rule_q8(row)
        tbl = _e4m3_mags()
        c = (q & 0x7F).astype(np.int64)
        v0, up, dn = tbl[c], tbl[np.minimum(c + 1, 0x7E)], tbl[np.maximum(c - 1, 0)]
        d_up = np.where(c < 0x7E, np.abs(mag - (v0 + up) / 2), np.inf)
        d_dn = np.where(c > 0, np.abs(mag - (v0 + dn) / 2), np.inf)
        step = np.maximum(up - v0, v0 - dn) * float(sc)
        return np.minimum(d_up, d_dn) <= window, step
    sc = a / top
    dist = np.abs(mag - (np.floor(mag) + 0.5))
    return dist <= window, np.full(row.size, float(sc))


def _down_column(ex, e, f):
    """|W_down[e][:, f]| of the experts dict (host), dequantised."""
    q = ex["down"][e][:, f].numpy()
    if ex["fmt"] == mi.FMT_FP8_ROW:
        return np.abs(_e4m3_mags()[q & 0x7F]) * ex["down_scales"][e].numpy().astype(np.float64)
    if ex["fmt"] == mi.FMT_Q8_0:
        return np.abs(q.astype(np.float64)) * ex["down_scales"][e][:, f // 32].float().numpy().astype(np.float64)
    return np.abs(q.astype(np.float64)) * ex["down_scales"][e].numpy().astype(np.float64)


def oracle_prefill(lay_host, x_host, idx, w, fp8):
    """The oracle's prefill output on the experts the routing touches, the bound on what h codes
    at rounding midpoints can move each output by, and how many such codes there are."""
    ids = sorted(set(np.asarray(idx).reshape(-1).tolist()))
    remap = np.zeros(max(ids) + 1, np.int32)
    remap[ids] = np.arange(len(ids), dtype=np.int32)
    idx2 = remap[np.asarray(idx)]
    ex = mi.subset_experts(lay_host["experts"], ids)
    fwd = oracle.experts_forward_f8act if fp8 else oracle.experts_forward_i8act
    res = fwd(x_host, idx2, w, ex, want_h=True)
    T, k = idx2.shape
    S = int(ex.get("n_shared", 0))
    e_all = np.concatenate([idx2, np.tile(np.arange(ex["E"], ex["E"] + S, dtype=np.int32), (T, 1))], 1)
    w_all = np.concatenate([np.asarray(w, np.float64), np.ones((T, S))], 1)
    h = res["h"].astype(np.float32)
    bound = np.zeros_like(res["out"])
    n_amb = 0
    for p in range(h.shape[0]):
        amb, step = _ambiguous_codes(h[p], fp8)
        t, j = divmod(p, k + S)
        for f in np.nonzero(amb)[0]:
            bound[t] += w_all[t, j] * step[f] * _down_column(ex, int(e_all[t, j]), int(f))
            n_amb += 1
    return res["out"], bound, n_amb


def prefill_err(got, ref, bound):
    """Row-normwise relative error left once the midpoint bound is taken off."""
    excess = np.maximum(np.abs(np.asarray(got, np.float64) - ref) - bound, 0.0)
    den = np.abs(ref).max(axis=-1)
    return float((excess.max(axis=-1) / np.where(den > 0, den, 1.0)).max())
