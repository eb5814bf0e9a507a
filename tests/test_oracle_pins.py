"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test names what it pins: library routines (numpy fp16, torch bf16, math.fsum, lexsort,
bincount, stable argsort, int64 matmul), a brute-force dense evaluation on tiny inputs, closed
forms, invariants of the method, and the figures the pages print for shapes and formats.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(name="tiny", **kw):
    """A shrunken workload that still has several Q8_0 blocks and E2M1 groups per row."""
    base = dict(T=5, d_model=96, E=6, k=3, d_ff=64)
    base.update(kw)
    return mi.workload(name, **base)


def layer_and_x(w, instance=0):
    lay = mi.make_layer(w, instance, "cpu")
    x = mi.make_x(w, instance, device="cpu")
    return lay, x


# ------------------------------------------------------------------------------------------
# Decoders vs library routines and the OCP table
# ------------------------------------------------------------------------------------------

def test_half_decoder_matches_numpy_for_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decoder_matches_torch():
    g = torch.Generator().manual_seed(5)
    bits = torch.randint(0, 1 << 16, (4096,), generator=g, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(int(b) & 0xFFFF) for b in bits.tolist()])
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e2m1_values_match_ocp_table():
    table = bf.e2m1_table()
    got = np.array([oracle.e2m1_value(c) for c in range(16)])
    assert np.array_equal(got, table)
    assert np.array_equal(np.signbit(got), np.signbit(table))


# ------------------------------------------------------------------------------------------
# Router
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("xdtype,bias", [("f32", False), ("bf16", True)])
def test_route_matches_exact_fsum_and_lexsort(xdtype, bias):
    w = small(xtype=mi.X_F32 if xdtype == "f32" else mi.X_BF16, zipf_s=1.1 if bias else None,
              E=16, k=5, T=12)
    lay, x = layer_and_x(w)
    idx, wts, logits, gap = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    ridx, rw, rlog = bf.route(x, lay["w_router"], lay["bias"], w.k)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(logits, rlog, rtol=0, atol=1e-13)
    np.testing.assert_allclose(wts, rw, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(wts.sum(1), 1.0, rtol=0, atol=1e-14)   # weights sum to 1
    assert np.all(gap >= 0)


def test_route_ties_go_to_lower_index():
    w = small(E=8, k=4, T=3)
    lay, x = layer_and_x(w)
    wr = lay["w_router"].clone()
    wr[5] = wr[2]           # experts 2 and 5 tie exactly for every token
    wr[7] = wr[2]
    idx, wts, logits, gap = oracle.route(x, wr, None, 8)
    for t in range(3):
        order = list(idx[t])
        assert order.index(2) < order.index(5) < order.index(7)
        assert order.index(5) == order.index(2) + 1 and order.index(7) == order.index(5) + 1
    # all-zero router: uniform, ranks are 0..k-1 and weights 1/k
    idx, wts, _, _ = oracle.route(x, torch.zeros_like(wr), None, 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (3, 1)))
    np.testing.assert_allclose(wts, 0.25, rtol=0, atol=1e-15)


def test_route_weights_equal_softmax_over_selected_logits():
    w = small(E=32, k=6, T=7, zipf_s=1.1)
    lay, x = layer_and_x(w)
    idx, wts, logits, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    for t in range(w.T):
        sel = logits[t, idx[t]]
        z = np.exp(sel - sel.max())
        np.testing.assert_allclose(wts[t], z / z.sum(), rtol=1e-13)
        assert np.all(np.diff(sel) <= 0)


# ------------------------------------------------------------------------------------------
# Permute
# ------------------------------------------------------------------------------------------

def test_permute_matches_bincount_and_stable_argsort():
    rng = np.random.default_rng(3)
    for E, P in [(8, 1), (8, 37), (128, 1000), (512, 22), (5, 0)]:
        idx = rng.integers(0, E, size=P).astype(np.int32)
        counts, offsets, perm, inv = oracle.permute(idx, E)
        assert np.array_equal(counts, np.bincount(idx, minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(idx, minlength=E))]))
        assert np.array_equal(perm, np.argsort(idx, kind="stable"))
        assert np.array_equal(inv[perm], np.arange(P))


# ------------------------------------------------------------------------------------------
# Expert FFN vs brute-force dense evaluation
# ------------------------------------------------------------------------------------------

CASES = [
    ("q8_0 swiglu", dict(fmt=mi.FMT_Q8_0, act=mi.ACT_SWIGLU)),
    ("i8_row swiglu", dict(fmt=mi.FMT_I8_ROW, act=mi.ACT_SWIGLU)),
    ("q8_0 relu2", dict(fmt=mi.FMT_Q8_0, act=mi.ACT_RELU2)),
    ("e2m1 relu2", dict(fmt=mi.FMT_E2M1, act=mi.ACT_RELU2, latent_bias_column=True)),
    ("e2m1 swiglu", dict(fmt=mi.FMT_E2M1, act=mi.ACT_SWIGLU)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("xtype", [mi.X_F32, mi.X_BF16])
def test_layer_matches_dense_bruteforce(name, kw, xtype):
    w = small(xtype=xtype, **kw)
    lay, x = layer_and_x(w)
    res = oracle.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act)
    ridx, rw, _ = bf.route(x, lay["w_router"], lay["bias"], w.k)
    assert np.array_equal(res["idx"], ridx)
    ref, _ = bf.dense_layer(x, ridx, rw, lay["experts"], w.act)
    assert bf.rel_err(res["out"], ref) < 1e-12


def test_single_expert_is_a_dense_swiglu_ffn():
    """E = 1, k = 1 reduces to out = W_down (silu(W_gate x) * (W_up x)) with numpy matmuls."""
    w = small(E=1, k=1, T=3)
    lay, x = layer_and_x(w)
    res = oracle.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], 1, w.act)
    ex = lay["experts"]
    q = ex["gate_up"][0].numpy().astype(np.float64)
    s = ex["gate_up_scales"][0].numpy().astype(np.float64)
    Wgu = q * np.kron(s, np.ones((1, 32)))
    qd = ex["down"][0].numpy().astype(np.float64)
    sd = ex["down_scales"][0].numpy().astype(np.float64)
    Wd = qd * np.kron(sd, np.ones((1, 32)))
    X = x.double().numpy()
    G, U = X @ Wgu[: w.d_ff].T, X @ Wgu[w.d_ff:].T
    ref = (G / (1 + np.exp(-G)) * U) @ Wd.T
    np.testing.assert_array_equal(res["w"], 1.0)
    assert bf.rel_err(res["out"], ref) < 1e-12


def test_one_hot_input_selects_one_column():
    """Closed form: x = e_j gives g_f = Wg[f, j], u_f = Wu[f, j] (catches a transposed operand)."""
    w = small(E=2, k=1, T=1)
    lay, _ = layer_and_x(w)
    ex = lay["experts"]
    j = 45
    x = torch.zeros((1, w.d_model))
    x[0, j] = 1.0
    idx = np.array([[1]], np.int32)
    out, h = oracle.experts_forward(x, idx, np.ones((1, 1)), ex, w.act, want_h=True)
    q = ex["gate_up"][1].numpy().astype(np.float64)
    s = ex["gate_up_scales"][1].numpy().astype(np.float64)
    g = q[: w.d_ff, j] * s[: w.d_ff, j // 32]
    u = q[w.d_ff:, j] * s[w.d_ff:, j // 32]
    np.testing.assert_allclose(h[0], g / (1 + np.exp(-g)) * u, rtol=1e-14, atol=1e-300)


def test_zero_gate_rows_give_zero_output():
    w = small(T=3)
    lay, x = layer_and_x(w)
    ex = dict(lay["experts"])
    gu = ex["gate_up"].clone()
    gu[:, : w.d_ff] = 0                                   # silu(0) = 0
    ex["gate_up"] = gu
    res = oracle.layer_forward(x, lay["w_router"], None, ex, w.k, w.act)
    assert np.all(res["out"] == 0.0)


# ------------------------------------------------------------------------------------------
# Invariants
# ------------------------------------------------------------------------------------------

def test_k_equals_E_with_uniform_router_is_the_dense_average():
    w = small(E=4, k=4, T=3)
    lay, x = layer_and_x(w)
    res = oracle.layer_forward(x, torch.zeros_like(lay["w_router"]), None, lay["experts"], 4, w.act)
    outs = []
    for e in range(4):
        idx = np.full((w.T, 1), e, np.int32)
        outs.append(oracle.experts_forward(x, idx, np.ones((w.T, 1)), lay["experts"], w.act))
    assert bf.rel_err(res["out"], np.mean(outs, axis=0)) < 1e-13


def test_token_permutation_equivariance():
    w = small(T=7, zipf_s=1.1)
    lay, x = layer_and_x(w)
    res = oracle.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act)
    pi = np.array([3, 0, 6, 1, 5, 2, 4])
    res2 = oracle.layer_forward(x[pi], lay["w_router"], lay["bias"], lay["experts"], w.k, w.act)
    assert np.array_equal(res2["out"], res["out"][pi])
    assert np.array_equal(res2["idx"], res["idx"][pi])


def test_expert_relabeling_invariance():
    w = small(T=5, E=6, zipf_s=1.1)
    lay, x = layer_and_x(w)
    res = oracle.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act)
    sigma = [4, 2, 5, 0, 3, 1]                            # new expert i is old expert sigma[i]
    ex2 = mi.subset_experts(lay["experts"], sigma)
    wr2 = lay["w_router"][sigma]
    b2 = lay["bias"][sigma]
    res2 = oracle.layer_forward(x, wr2, b2, ex2, w.k, w.act)
    assert np.array_equal(np.array(sigma)[res2["idx"]], res["idx"])
    assert bf.rel_err(res2["out"], res["out"]) < 1e-15


@pytest.mark.parametrize("fmt", [mi.FMT_Q8_0, mi.FMT_I8_ROW])
def test_doubling_down_scales_doubles_output(fmt):
    w = small(fmt=fmt)
    lay, x = layer_and_x(w)
    res = oracle.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act)
    ex = dict(lay["experts"])
    ex["down_scales"] = ex["down_scales"] * 2                 # exact in fp16 and fp32
    res2 = oracle.layer_forward(x, lay["w_router"], None, ex, w.k, w.act)
    assert np.array_equal(res2["out"], 2 * res["out"])


def test_thread_count_does_not_change_bits():
    w = small(T=6, d_ff=128)
    lay, x = layer_and_x(w)
    n = oracle.get_threads()
    try:
        oracle.set_threads(1)
        a = oracle.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act)["out"]
        oracle.set_threads(max(2, n))
        b = oracle.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act)["out"]
    finally:
        oracle.set_threads(n)
    assert np.array_equal(a, b)


def test_output_column_subset_equals_full():
    w = small(T=4)
    lay, x = layer_and_x(w)
    idx, wts, _, _ = oracle.route(x, lay["w_router"], None, w.k)
    full = oracle.experts_forward(x, idx, wts, lay["experts"], w.act)
    cols = np.array([0, 7, 95, 31], np.int32)
    part = oracle.experts_forward(x, idx, wts, lay["experts"], w.act, o_list=cols)
    assert np.array_equal(part, full[:, cols])


# ------------------------------------------------------------------------------------------
# Zero-skip down (E2M1, neuron-major)
# ------------------------------------------------------------------------------------------

def test_zero_skip_down_equals_full_down():
    w = small(fmt=mi.FMT_E2M1, act=mi.ACT_RELU2, latent_bias_column=True, d_model=64, d_ff=256,
              E=8, k=3, T=4)
    lay, x = layer_and_x(w)
    idx, wts, _, _ = oracle.route(x, lay["w_router"], None, w.k)
    full, h = oracle.experts_forward(x, idx, wts, lay["experts"], w.act, want_h=True)
    zs, active = oracle.zero_skip_down(h, idx, wts, lay["experts"])
    assert bf.rel_err(zs, full) < 1e-15
    assert active.max() <= w.d_ff // 16
    # A group counts as active exactly when one of its 16 h is nonzero.
    ref_active = (h.reshape(w.T * w.k, -1, 16) != 0).any(-1).sum(-1)
    assert np.array_equal(active, ref_active)


def test_all_negative_bias_column_gives_zero_output_and_no_active_group():
    w = small(fmt=mi.FMT_E2M1, act=mi.ACT_RELU2, latent_bias_column=True, d_model=64, d_ff=64,
              E=4, k=2, T=2)
    lay, _ = layer_and_x(w)
    x = torch.zeros((2, 64), dtype=torch.bfloat16)
    x[:, 63] = 1.0                                        # only the bias column contributes (< 0)
    idx, wts, _, _ = oracle.route(x, lay["w_router"], None, w.k)
    out, h = oracle.experts_forward(x, idx, wts, lay["experts"], w.act, want_h=True)
    zs, active = oracle.zero_skip_down(h, idx, wts, lay["experts"])
    assert np.all(out == 0) and np.all(zs == 0) and np.all(active == 0)


def test_swapped_nibbles_change_the_output():
    """The pages' must-fail check: swapping the two 4-bit halves of every byte breaks the result."""
    w = small(fmt=mi.FMT_E2M1, act=mi.ACT_RELU2, latent_bias_column=True, d_model=64, d_ff=64,
              E=4, k=2, T=3)
    lay, x = layer_and_x(w)
    idx, wts, _, _ = oracle.route(x, lay["w_router"], None, w.k)
    ok = oracle.experts_forward(x, idx, wts, lay["experts"], w.act)
    ex = dict(lay["experts"])
    for key in ("gate_up", "down"):
        b = ex[key]
        ex[key] = ((b & 15) << 4) | (b >> 4)
    bad = oracle.experts_forward(x, idx, wts, ex, w.act)
    assert bf.rel_err(bad, ok) > 0.1


# ------------------------------------------------------------------------------------------
# int8-activation (prefill) variant and rule Q
# ------------------------------------------------------------------------------------------

def test_rule_q_closed_forms():
    v = np.array([127.0, -0.5, 0.5, 1.5, 2.5, -2.5, 126.5, -127.0, 3.49], np.float32)
    q, s = oracle.rule_q(v)                        # a = 127 -> inv = 1: round half to even
    assert list(q) == [127, 0, 0, 2, 2, -2, 126, -127, 3]
    assert s == np.float32(1.0)
    q, s = oracle.rule_q(np.zeros(7, np.float32))
    assert np.all(q == 0) and s == 0.0
    v = np.array([1.0, -0.25, 0.004], np.float32)  # a = 1: inv = 127, codes 127, -32 (31.75), 1 (0.508)
    q, s = oracle.rule_q(v)
    assert list(q) == [127, -32, 1] and s == np.float32(1.0) / np.float32(127.0)


def test_rule_q_matches_numpy_float32_rounding():
    rng = np.random.default_rng(11)
    for n in (1, 17, 704, 2816):
        v = rng.standard_normal(n).astype(np.float32) * np.float32(rng.uniform(0.01, 10))
        q, s = oracle.rule_q(v)
        a = np.abs(v).max()
        inv = np.float32(127.0) / a
        ref = np.clip(np.rint(v * inv), -127, 127).astype(np.int8)      # numpy: IEEE fp32 ops
        assert np.array_equal(q, ref)
        assert s == a / np.float32(127.0)
        assert np.abs(q).max() == 127


def test_i8act_variant_matches_int64_bruteforce():
    w = small(fmt=mi.FMT_I8_ROW, T=6, d_model=128, d_ff=96, E=5, k=2, zipf_s=1.1)
    lay, x = layer_and_x(w)
    idx, wts, _, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    res = oracle.experts_forward_i8act(x, idx, wts, lay["experts"], want_h=True)
    ex = lay["experts"]
    xq = np.stack([oracle.rule_q(x[t].float().numpy())[0] for t in range(w.T)])
    sx = np.array([oracle.rule_q(x[t].float().numpy())[1] for t in range(w.T)])
    assert np.array_equal(res["xq"], xq) and np.array_equal(res["sx"], sx)
    qgu = ex["gate_up"].numpy().astype(np.int64)
    sgu = ex["gate_up_scales"].numpy().astype(np.float64)
    qdn = ex["down"].numpy().astype(np.int64)
    sdn = ex["down_scales"].numpy().astype(np.float64)
    out = np.zeros((w.T, w.d_model))
    for t in range(w.T):
        for j in range(w.k):
            e = idx[t, j]
            acc = qgu[e] @ xq[t].astype(np.int64)                   # exact int64 matmul
            gu = sx[t].astype(np.float64) * sgu[e] * acc
            g, u = gu[: w.d_ff], gu[w.d_ff:]
            h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
            np.testing.assert_allclose(res["h"][t * w.k + j], h, rtol=1e-6, atol=1e-30)
            hq, sh = oracle.rule_q(res["h"][t * w.k + j].astype(np.float32))
            y = np.float64(sh) * sdn[e] * (qdn[e] @ hq.astype(np.int64))
            out[t] += wts[t, j] * y
    assert bf.rel_err(res["out"], out) < 1e-13


def test_i8act_q8_0_with_one_scale_per_row_is_the_per_row_variant():
    """Special case: Q8_0 weights whose blocks in a row all share one scale s are per-row int8
    weights with scale s, so the two int8-activation layers agree exactly (each block's scaled
    integer sum is exact in fp64 and so are the partial sums)."""
    w = small(fmt=mi.FMT_Q8_0, T=5, d_model=128, d_ff=96, E=4, k=2)
    lay, x = layer_and_x(w)
    ex = dict(lay["experts"])
    for key in ("gate_up_scales", "down_scales"):
        sc = ex[key].clone()
        sc[...] = sc[..., :1]                  # every block of a row takes the row's first scale
        ex[key] = sc
    row = dict(ex, fmt=mi.FMT_I8_ROW,
               gate_up_scales=ex["gate_up_scales"][..., 0].float().contiguous(),
               down_scales=ex["down_scales"][..., 0].float().contiguous())
    idx, wts, _, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    a = oracle.experts_forward_i8act(x, idx, wts, ex, want_h=True)
    b = oracle.experts_forward_i8act(x, idx, wts, row, want_h=True)
    assert np.array_equal(a["h"], b["h"])
    assert np.array_equal(a["out"], b["out"])


def test_i8act_q8_0_matches_dequantised_bruteforce():
    """Q8_0 blocks with their own scales: against a plain fp64 loop over dequantised weights
    (q * s of each element's block) and the rule-Q codes; fp64 rounding only."""
    w = small(fmt=mi.FMT_Q8_0, T=4, d_model=128, d_ff=64, E=3, k=2)
    lay, x = layer_and_x(w)
    ex = lay["experts"]
    idx, wts, _, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    res = oracle.experts_forward_i8act(x, idx, wts, ex, want_h=True)
    qgu = ex["gate_up"].numpy().astype(np.float64)
    sgu = np.repeat(ex["gate_up_scales"].numpy().astype(np.float64), 32, axis=-1)
    qdn = ex["down"].numpy().astype(np.float64)
    sdn = np.repeat(ex["down_scales"].numpy().astype(np.float64), 32, axis=-1)
    out = np.zeros((w.T, w.d_model))
    for t in range(w.T):
        xq, sx = oracle.rule_q(x[t].float().numpy())
        for j in range(w.k):
            e = idx[t, j]
            gu = np.zeros(2 * w.d_ff)
            for f in range(2 * w.d_ff):
                for i in range(w.d_model):
                    gu[f] += float(xq[i]) * qgu[e, f, i] * sgu[e, f, i]
            gu *= np.float64(sx)
            g, u = gu[: w.d_ff], gu[w.d_ff:]
            h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
            np.testing.assert_allclose(res["h"][t * w.k + j], h, rtol=1e-6, atol=1e-30)
            hq, sh = oracle.rule_q(res["h"][t * w.k + j].astype(np.float32))
            y = np.zeros(w.d_model)
            for o in range(w.d_model):
                for f in range(w.d_ff):
                    y[o] += float(hq[f]) * qdn[e, o, f] * sdn[e, o, f]
            out[t] += wts[t, j] * np.float64(sh) * y
    assert bf.rel_err(res["out"], out) < 1e-12


def _dequant_q8_0(q, s16):
    return q.astype(np.float64) * np.repeat(s16.astype(np.float64), 32, axis=-1)


def test_shared_expert_adds_its_dense_ffn():
    """The shared expert (expert E) is a dense SwiGLU FFN every token goes through, added with
    weight 1: the layer with it minus the layer without it is that FFN, computed here by plain
    fp64 matrix products of the dequantised weights."""
    w = small(fmt=mi.FMT_Q8_0, T=5, d_model=128, d_ff=64, E=4, k=2, n_shared=1)
    lay, x = layer_and_x(w)
    ex = lay["experts"]
    assert ex["gate_up"].shape[0] == w.E + 1
    idx, wts, _, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    with_s = oracle.experts_forward(x, idx, wts, ex, w.act)
    without = oracle.experts_forward(x, idx, wts, dict(ex, n_shared=0), w.act)
    gu = _dequant_q8_0(ex["gate_up"][w.E].numpy(), ex["gate_up_scales"][w.E].numpy())
    dn = _dequant_q8_0(ex["down"][w.E].numpy(), ex["down_scales"][w.E].numpy())
    xv = x.double().numpy()
    g, u = xv @ gu[: w.d_ff].T, xv @ gu[w.d_ff:].T
    dense = (g / (1 + np.exp(-g)) * u) @ dn.T
    assert bf.rel_err(with_s - without, dense) < 1e-12
    # and the int8-activation variant: the same extra slot, now through rule Q
    w8 = small(fmt=mi.FMT_I8_ROW, T=5, d_model=128, d_ff=64, E=4, k=2, n_shared=1)
    lay8, x8 = layer_and_x(w8)
    ex8 = lay8["experts"]
    a = oracle.experts_forward_i8act(x8, idx, wts, ex8, want_h=True)
    b = oracle.experts_forward_i8act(x8, np.concatenate([idx, np.full((w8.T, 1), w8.E, np.int32)], 1),
                                     np.concatenate([wts, np.ones((w8.T, 1))], 1), dict(ex8, n_shared=0, E=w8.E + 1))
    assert np.array_equal(a["out"], b["out"]) and a["h"].shape[0] == w8.T * (w8.k + 1)


def test_i8act_integer_inputs_are_quantised_exactly():
    """Closed form: an x row of integers whose max |x| is 127 quantises to itself with s_x = 1."""
    w = small(fmt=mi.FMT_I8_ROW, T=2, d_model=64, d_ff=32, E=2, k=1)
    lay, _ = layer_and_x(w)
    rng = np.random.default_rng(2)
    xi = rng.integers(-126, 127, size=(2, 64)).astype(np.float32)
    xi[:, 5] = 127.0
    idx = np.zeros((2, 1), np.int32)
    res = oracle.experts_forward_i8act(torch.from_numpy(xi), idx, np.ones((2, 1)), lay["experts"])
    assert np.array_equal(res["xq"], xi.astype(np.int8)) and np.all(res["sx"] == 1.0)


# ------------------------------------------------------------------------------------------
# E4M3 (OCP 8-bit floating point) and the fp8 batched-prefill variant
# ------------------------------------------------------------------------------------------

def _torch_e4m3_decode(codes):
    return torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()


def test_e4m3_values_match_torch_and_closed_forms():
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    ref = _torch_e4m3_decode(list(range(256)))          # torch's float8_e4m3fn decoder
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2
    fin = ~np.isnan(got)
    assert np.array_equal(got[fin], ref[fin]) and np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    # closed forms of the spec: bias 7, subnormals m/8 * 2^-6, largest finite 448
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x07] == 7 * 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x80] == 0.0 and np.signbit(got[0x80])


def test_e4m3_encode_matches_torch_round_to_nearest_even():
    finite = np.array(sorted({oracle.e4m3_value(c) for c in range(128)} - {float("nan")}))
    finite = finite[~np.isnan(finite)]
    mids = (finite[1:] + finite[:-1]) / 2                     # exact ties: both neighbours
    vals = np.concatenate([finite, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                           np.random.default_rng(5).uniform(0, 470, 2000),
                           np.random.default_rng(6).uniform(0, 2.0 ** -6, 500), [2.0 ** -10, 464.0, 463.9]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    vals = vals[np.abs(vals) <= 464.0]                        # torch maps larger values to NaN too
    got = np.array([oracle.e4m3_encode(v) for v in vals], np.uint8)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # ties go to the even code: 1 + 1/16 lies between codes 0x38 (1.0) and 0x39 (1.125)
    assert oracle.e4m3_encode(1.0625) == 0x38 and oracle.e4m3_encode(1.1875) == 0x3A
    assert oracle.e4m3_encode(464.0) == 0x7E and oracle.e4m3_encode(464.5) == 0x7F
    assert oracle.e4m3_encode(-465.0) == 0xFF and oracle.e4m3_encode(2.0 ** -10) == 0x00


def test_rule_q8_invariants_and_closed_forms():
    rng = np.random.default_rng(12)
    for n in (1, 17, 704, 2816):
        v = rng.standard_normal(n).astype(np.float32) * np.float32(rng.uniform(0.01, 10))
        q, s = oracle.rule_q8(v)
        a = np.abs(v).max()
        assert s == a / np.float32(448.0)
        dec = np.array([oracle.e4m3_value(c) for c in q])
        assert np.abs(dec).max() == 448.0                     # the row's max maps to 448
        inv = np.float64(np.float32(448.0) / a)
        scaled = v.astype(np.float64) * inv
        # nearest code: at most half a code step from the scaled value (step 2^(e-3), subnormal 2^-9)
        step = np.where(np.abs(scaled) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(scaled), 1e-300))) - 3), 2.0 ** -9)
        assert np.all(np.abs(dec - scaled) <= step / 2 * (1 + 1e-6))
        q2, s2 = oracle.rule_q8(-v)                           # odd symmetry: sign bits flip
        assert s2 == s and np.array_equal(q2, q ^ 0x80)
    # codes of a vector whose max is 448: inv = 1, values exact in E4M3 keep their codes
    v = np.array([448.0, -1.0, 0.5, 3.5, -2.0 ** -9, 240.0], np.float32)
    q, s = oracle.rule_q8(v)
    assert list(q) == [0x7E, 0xB8, 0x30, 0x46, 0x81, 0x77] and s == np.float32(1.0)
    q, s = oracle.rule_q8(np.zeros(9, np.float32))
    assert np.all(q == 0) and s == 0.0


def test_f8act_variant_matches_dequantised_bruteforce():
    """Per-row E4M3 weights: against a plain fp64 loop over decoded codes times the row scales,
    with the rule-Q8 codes of x and of the oracle's own fp32 h (h checked against the brute
    force first); fp64 rounding only."""
    w = small(fmt=mi.FMT_FP8_ROW, T=4, d_model=128, d_ff=64, E=3, k=2)
    lay, x = layer_and_x(w)
    ex = lay["experts"]
    idx, wts, _, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    res = oracle.experts_forward_f8act(x, idx, wts, ex, want_h=True)
    dec = _torch_e4m3_decode(list(range(256)))
    qgu = dec[ex["gate_up"].numpy()]
    sgu = ex["gate_up_scales"].numpy().astype(np.float64)
    qdn = dec[ex["down"].numpy()]
    sdn = ex["down_scales"].numpy().astype(np.float64)
    out = np.zeros((w.T, w.d_model))
    for t in range(w.T):
        xq, sx = oracle.rule_q8(x[t].float().numpy())
        assert np.array_equal(res["xq"][t], xq) and res["sx"][t] == sx
        for j in range(w.k):
            e = idx[t, j]
            gu = np.zeros(2 * w.d_ff)
            for f in range(2 * w.d_ff):
                for i in range(w.d_model):
                    gu[f] += dec[xq[i]] * qgu[e, f, i]
            gu *= np.float64(sx) * sgu[e]
            g, u = gu[: w.d_ff], gu[w.d_ff:]
            h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
            np.testing.assert_allclose(res["h"][t * w.k + j], h, rtol=1e-6, atol=1e-30)
            hq, sh = oracle.rule_q8(res["h"][t * w.k + j].astype(np.float32))
            y = np.zeros(w.d_model)
            for o in range(w.d_model):
                for f in range(w.d_ff):
                    y[o] += dec[hq[f]] * qdn[e, o, f]
            out[t] += wts[t, j] * np.float64(sh) * sdn[e] * y
    assert bf.rel_err(res["out"], out) < 1e-12


def test_f8act_codes_exact_in_e4m3_are_kept():
    """Closed form: an x row of E4M3 values whose max is 448 quantises to its own codes, s_x = 1;
    with one expert whose gate/up rows are unit vectors the gate/up sums are single products."""
    w = small(fmt=mi.FMT_FP8_ROW, T=2, d_model=64, d_ff=64, E=1, k=1)
    lay, _ = layer_and_x(w)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, size=(2, 64)).astype(np.uint8) | (rng.integers(0, 2, size=(2, 64)).astype(np.uint8) << 7)
    codes[:, 9] = 0x7E
    codes[codes == 0x80] = 0                                  # -0 and +0 decode alike; keep +0
    xv = _torch_e4m3_decode(codes.reshape(-1)).reshape(2, 64).astype(np.float32)
    res = oracle.experts_forward_f8act(torch.from_numpy(xv), np.zeros((2, 1), np.int32), np.ones((2, 1)),
                                       lay["experts"])
    assert np.array_equal(res["xq"], codes) and np.all(res["sx"] == 1.0)


def test_fp8_shared_expert_is_an_extra_slot():
    w = small(fmt=mi.FMT_FP8_ROW, T=5, d_model=128, d_ff=64, E=4, k=2, n_shared=1)
    lay, x = layer_and_x(w)
    ex = lay["experts"]
    idx, wts, _, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    a = oracle.experts_forward_f8act(x, idx, wts, ex, want_h=True)
    b = oracle.experts_forward_f8act(x, np.concatenate([idx, np.full((w.T, 1), w.E, np.int32)], 1),
                                     np.concatenate([wts, np.ones((w.T, 1))], 1), dict(ex, n_shared=0, E=w.E + 1))
    assert np.array_equal(a["out"], b["out"]) and a["h"].shape[0] == w.T * (w.k + 1)


# ------------------------------------------------------------------------------------------
# The pages' own figures (shapes and formats)
# ------------------------------------------------------------------------------------------

def _figs():
    with open(os.path.join(GOLDEN, "pages_figures.json")) as fh:
        return json.load(fh)


def test_page_expert_block_bytes_fix_two_codes_per_byte_and_one_scale_per_16():
    figs = _figs()
    sh = figs["nemotron_expert_shape"]
    d, dff = sh["d_latent"], sh["d_ff"]
    values = 2 * d * dff                       # up + down
    block = values // 2 + values // 16 * 1     # 4-bit codes, one 1-byte scale per 16 values
    assert block == figs["nemotron_expert_block_bytes"]["value"] == 756 * 4096
    # the library stores the same codes with fp16 scales: one extra byte per 16 values
    w = mi.workload("nemotron_latent")
    assert mi.expert_bytes(w) == values // 2 + values // 16 * 2
    assert abs(block / 1e6 - sh["expert_mb"]) < 0.01


def test_page_gemma_expert_bytes_fix_d_ff():
    figs = _figs()["gemma_bf16_expert_gb"]
    w = mi.workload("gemma_decode")
    total = figs["gemma_layers"] * figs["experts"] * 3 * w.d_ff * w.d_model * 2
    assert abs(total / 1e9 - figs["value"]) / figs["value"] < 0.01


def test_page_m3_shape():
    f = _figs()["m3_shape"]
    w = mi.workload("m3_decode")
    assert (w.E, w.k, w.d_model, w.d_ff) == (f["experts"], f["top_k"], f["n_embd"], f["expert_ffn"])
    assert (f["layers"] - f["dense_layers"]) * f["top_k"] == f["active_experts_per_token"]


@pytest.mark.slow
def test_nemotron_construction_gives_about_92_5_percent_zeros():
    """The latent construction (x[-1] = 1, up[:, -1] = -1.44 sigma sqrt(d-1)) leaves roughly the
    pages' fraction of zero neurons after ReLU^2 (checked at the full 2688 x 1024 expert shape,
    on 24 of the 512 experts)."""
    w = mi.workload("nemotron_latent", E=24, k=8, T=3)
    lay, x = layer_and_x(w)
    idx, wts, _, _ = oracle.route(x, lay["w_router"], None, w.k)
    _, h = oracle.experts_forward(x, idx, wts, lay["experts"], w.act, o_list=[0], want_h=True)
    zero = float((h == 0).mean())
    assert abs(zero - _figs()["nemotron_zero_fraction"]["value"]) < 0.02, zero


# ------------------------------------------------------------------------------------------
# The prefill parity check's midpoint bound (test infrastructure of the GPU tests), on the CPU
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_midpoint_bound_explains_one_flipped_code_and_nothing_else(fp8):
    """Plant an h element exactly on a rounding midpoint: the oracle's two correct outputs (code
    below, code above) both pass the check, while an unrelated 1% error on one output fails it."""
    from tests import prefill_check as gp
    fmt = mi.FMT_FP8_ROW if fp8 else mi.FMT_I8_ROW
    w = small(fmt=fmt, T=3, d_model=128, d_ff=64, E=3, k=2)
    lay, x = layer_and_x(w)
    idx, wts, _, _ = oracle.route(x, lay["w_router"], lay["bias"], w.k)
    ex = lay["experts"]
    fwd = oracle.experts_forward_f8act if fp8 else oracle.experts_forward_i8act
    res = fwd(x, idx, wts, ex, want_h=True)
    row = res["h"][0].astype(np.float32)
    amb, step = gp._ambiguous_codes(row, fp8)
    # an element exactly on a midpoint (in scaled units) is flagged; recompute that output by hand
    top = np.float32(448.0 if fp8 else 127.0)
    inv = top / np.float32(np.abs(row).max())
    f = int(np.argsort(np.abs(row))[len(row) // 2])
    v = float(row[f] * inv)
    if fp8:
        tbl = gp._e4m3_mags()
        c = int(np.searchsorted(tbl, abs(v)))
        mid = (tbl[c - 1] + tbl[c]) / 2 * np.sign(v)
    else:
        mid = np.floor(v) + 0.5
    row2 = row.copy()
    row2[f] = np.float32(mid / inv)
    amb2, _ = gp._ambiguous_codes(row2, fp8)
    assert amb2[f]
    assert amb.sum() <= max(2, row.size // 20)           # few elements sit near midpoints
    ref, bound, n_amb = gp.oracle_prefill({"experts": ex}, x, idx, wts, fp8)
    e = int(idx[0, 0])
    col = gp._down_column(ex, e, f)
    flipped = ref.copy()
    flipped[0] += wts[0, 0] * step[f] * col                 # one code step on element f
    b2 = bound.copy()
    b2[0] += wts[0, 0] * step[f] * col                      # what the bound adds when f is flagged
    assert gp.prefill_err(flipped, ref, b2) < 1e-12
    assert gp.prefill_err(ref, ref, bound) == 0.0
    bad = ref.copy()
    bad[1, 7] += 0.01 * np.abs(ref[1]).max()
    assert gp.prefill_err(bad, ref, bound) > 5e-3
