"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Bars: top-k ids equal the oracle's exactly; routing weights within 1e-6; permutation arrays and
int8 codes bit-exact; layer outputs within a row-normwise relative error of 2e-3 (the stated
tolerance), and within 1e-4 on the paths whose products are exact (decode: int8 / E2M1 weights
and bf16 activations are exact in bf16, fp32 h is split into two bf16 terms, all sums are fp32
over at most 6144 terms, so the error is a few 1e-6 at most).
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_expert_router_amd as moe
from tests import bruteforce as bf
from tests.prefill_check import oracle_prefill, prefill_err

pytestmark = pytest.mark.gpu

TOL = 2e-3
EXACT_PRODUCT_TOL = 1e-4
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def oracle_experts(lay_host, x_host, idx, w, act, o_list=None, i8act=False, f8act=False):
    """Oracle on only the experts the routing touches (renumbered), so big layers stay cheap."""
    ids = sorted(set(np.asarray(idx).reshape(-1).tolist()))
    remap = np.zeros(max(ids) + 1, np.int32)
    remap[ids] = np.arange(len(ids), dtype=np.int32)
    idx2 = remap[np.asarray(idx)]
    ex = mi.subset_experts(lay_host["experts"], ids)
    if i8act:
        return oracle.experts_forward_i8act(x_host, idx2, w, ex, o_list=o_list)["out"]
    if f8act:
        return oracle.experts_forward_f8act(x_host, idx2, w, ex, o_list=o_list)["out"]
    return oracle.experts_forward(x_host, idx2, w, ex, act, o_list=o_list)


def check_prefill(got, host, x_host, idx, w, fp8):
    """Prefill output against the oracle, to TOL beyond the midpoint bound (tests/prefill_check)."""
    ref, bound, n_amb = oracle_prefill(host, x_host, idx, w, fp8)
    raw = bf.rel_err(got, ref)
    err = prefill_err(got, ref, bound)
    rel_bound = float((bound.max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-300)).max())
    say(f"  rel err {raw:.3g}; {n_amb} midpoint h codes, bound up to {rel_bound:.3g} of a row; "
        f"beyond it {err:.3g}")
    assert err < TOL
    return raw


def gen(w, instance=0, T=None):
    lay = mi.make_layer(w, instance, DEV)
    x = mi.make_x(w, instance, T=T, device=DEV)
    return lay, x


# ------------------------------------------------------------------------------------------
# Router: bit-exact ids
# ------------------------------------------------------------------------------------------

ROUTE_CASES = [("tiny", 4), ("gemma_decode", 1), ("gemma_decode", 8), ("gemma_decode", 64),
               ("gemma_decode", 65), ("m3_decode", 1), ("m3_decode", 32), ("m3_decode", 100),
               ("nemotron_latent", 1), ("nemotron_latent", 7), ("nemotron_latent", 300),
               ("gemma_prefill", 2048)]


@pytest.mark.parametrize("name,T", ROUTE_CASES, ids=[f"{n}-T{t}" for n, t in ROUTE_CASES])
def test_route_ids_bit_exact(name, T):
    w = mi.workload(name)
    say("route", name, T)
    g = torch.Generator(device=DEV).manual_seed(77)
    wr = torch.randn((w.E, w.d_model), generator=g, device=DEV) * w.router_std
    bias = mi.zipf_bias(w.E, w.zipf_s).to(DEV) if w.zipf_s else None
    x = mi.make_x(w, 0, T=T, device=DEV)
    idx, wts = moe.route(x, wr, bias, w.k)
    torch.cuda.synchronize()
    ridx, rw, _, gap = oracle.route(x.cpu(), wr.cpu(), None if bias is None else bias.cpu(), w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx), "top-k ids differ from the oracle"
    np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=0, atol=1e-6)
    say("  min adjacent gap among ranks 1..k+1:", float(gap.min()))


@pytest.mark.parametrize("xt", ["bf16", "f32"])
@pytest.mark.parametrize("T", [5, 100], ids=["decode-router", "batched-router"])
def test_route_ties_and_degenerate_routers(T, xt):
    """Equal router rows (exact ties: the lower index first) and an all-zero router, on the
    decode router and on the batched (fp64 matrix-core) one, with bf16 and fp32 tokens."""
    w = mi.workload("gemma_decode")
    x = mi.make_x(w, 0, T=T, device=DEV)
    if xt == "f32":
        x = x.float()
    g = torch.Generator(device=DEV).manual_seed(3)
    wr = torch.randn((w.E, w.d_model), generator=g, device=DEV) * 0.05
    wr[9] = wr[3]
    wr[100] = wr[3]
    wr[64] = wr[3]
    for W in (wr, torch.zeros_like(wr)):
        idx, wts = moe.route(x, W, None, w.k)
        ridx, rw, _, _ = oracle.route(x.cpu(), W.cpu(), None, w.k)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        np.testing.assert_allclose(wts.cpu().numpy(), rw, atol=1e-6)
    z = torch.zeros((64, w.d_model), device=DEV)
    idx, wts = moe.route(x, z, None, 64)             # k = E = 64: every expert, weight 1/E
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(64), (T, 1)))
    np.testing.assert_allclose(wts.cpu().numpy(), 1 / 64, atol=1e-9)


@pytest.mark.parametrize("E,k", [(128, 8), (512, 22), (40, 40), (200, 5)])
def test_batched_router_near_ties(E, k):
    """The batched router (T > 64) on near ties: router rows that differ by 1e-6 relative, exact
    duplicates, a zero token, tokens of 1e15 and of 1e-20 magnitude, with and without a bias: the
    ids are the oracle's and the weights agree to 1e-6."""
    T, d = 96, 512
    g = torch.Generator(device=DEV).manual_seed(E + k)
    base = torch.randn((1, d), generator=g, device=DEV) * 0.05
    wr = base + base.abs() * 1e-6 * torch.randn((E, d), generator=g, device=DEV)
    wr[E // 2] = wr[1]
    wr[E - 1] = wr[0]
    x = torch.randn((T, d), generator=g, device=DEV)
    x[3] = 0
    x[4] *= 1e15
    x[5] *= 1e-20
    x = x.to(torch.bfloat16)
    bias = torch.randn(E, generator=g, device=DEV) * 1e-3
    for b in (None, bias):
        idx, wts = moe.route(x, wr, b, k)
        torch.cuda.synchronize()
        ridx, rw, _, _ = oracle.route(x.cpu(), wr.cpu(), None if b is None else b.cpu(), k)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=0, atol=1e-6)


@pytest.mark.parametrize("E,T,k", [(129, 1, 22), (200, 7, 5), (256, 3, 64), (512, 1, 22),
                                   (512, 64, 8), (512, 2, 64), (300, 5, 1), (256, 4, 16),
                                   (512, 2, 32), (300, 2, 3)])
def test_layer_selection_many_experts(E, T, k):
    """The layer's own selection (more than 128 experts: per-wave sorted lists merged by rank)
    against the oracle's, on random, tied and all-zero routers."""
    say("selection", E, T, k)
    w = mi.workload("tiny", E=E, k=k, T=T, d_model=64, d_ff=64)
    lay, x = gen(w)
    wr = lay["w_router"].clone()
    tied = wr.clone()
    for e in (3, 64, 65, 127, 128, 191, E - 1):      # equal rows in different 64-expert lists
        if e < E:
            tied[e] = wr[1]
    for W in (wr, tied, torch.zeros_like(wr)):
        out, idx, wts = moe.layer_forward(x, W, None, lay["experts"], k, w.act, want_routing=True)
        torch.cuda.synchronize()
        ridx, rw, _, _ = oracle.route(x.cpu(), W.cpu(), None, k)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=0, atol=1e-6)


# ------------------------------------------------------------------------------------------
# Permute: bit-exact
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("E,T,k", [(8, 4, 2), (128, 1, 8), (128, 8, 8), (512, 1, 22),
                                   (128, 2048, 8), (1, 3, 1), (512, 300, 7), (37, 1000, 5)])
def test_permute_bit_exact(E, T, k):
    say("permute", E, T, k)
    rng = np.random.default_rng(E * 1000 + T)
    # skewed draws, so some experts get many pairs and some none
    idx = np.minimum(rng.zipf(1.3, size=(T, k)) - 1, E - 1).astype(np.int32)
    counts, offsets, perm, inv = moe.permute(torch.from_numpy(idx).to(DEV), E)
    rc, ro, rp, ri = oracle.permute(idx, E)
    for a, b in ((counts, rc), (offsets, ro), (perm, rp), (inv, ri)):
        assert np.array_equal(a.cpu().numpy(), b)


# ------------------------------------------------------------------------------------------
# Activation quantiser (rule Q): bit-exact
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("cols", [64, 704, 2816, 4096, 4160, 16384])
def test_quantize_rows_bit_exact(dtype, cols):
    g = torch.Generator(device=DEV).manual_seed(9)
    v = (torch.randn((70, cols), generator=g, device=DEV) * 3).to(dtype)
    v[5] = 0                                  # an all-zero row: q = 0, scale = 0
    v[6, :] = 0.5
    v[6, 7] = 127.0                           # inv = 1: exact half-way cases round to even
    v[6, 8] = 2.5
    q, s = moe.quantize_rows_i8(v)
    vh = v.float().cpu().numpy()
    for r in range(v.shape[0]):
        rq, rs = oracle.rule_q(vh[r])
        assert np.array_equal(q[r].cpu().numpy(), rq), r
        assert s[r].item() == rs, r


def _e4m3_grid():
    """Every finite E4M3 magnitude, the midpoints between neighbours (ties) and the fp32 values
    just either side of each midpoint, both signs: with a row maximum of 448 (inv = 1 exactly)
    these are converted as they stand."""
    mags = np.array(sorted(oracle.e4m3_value(c) for c in range(0x7F)), np.float64)
    mids = (mags[1:] + mags[:-1]) / 2
    m32 = mids.astype(np.float32)
    v = np.concatenate([mags, mids, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                        [2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11]]).astype(np.float32)
    v = np.concatenate([v, -v])
    return np.resize(v, ((v.size + 63) // 64) * 64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("cols", [64, 704, 2816, 4160, 16384])
def test_quantize_rows_fp8_bit_exact(dtype, cols):
    """Rule Q8 (E4M3 codes, round to nearest even) on the GPU's v_cvt_pk_fp8_f32 against the
    oracle's encoder, code for code, including ties, subnormals, signed zeros and zero rows."""
    g = torch.Generator(device=DEV).manual_seed(19)
    v = (torch.randn((70, cols), generator=g, device=DEV) * 3).to(dtype)
    v[5] = 0                                  # an all-zero row: codes 0, scale 0
    v[6] = -0.0                               # negative zeros only: still codes 0
    v[7, :] = 1e-30                           # values far below the smallest subnormal
    v[7, 3] = -1.0
    grid = torch.from_numpy(_e4m3_grid()).to(DEV)
    n = min(cols, grid.numel())
    v[8, :n] = grid[:n].to(dtype)
    v[8, 0] = 448.0                           # inv = 1
    v[9] = v[8].flip(0)
    q, s = moe.quantize_rows_fp8(v)
    vh = v.float().cpu().numpy()
    for r in range(v.shape[0]):
        rq, rs = oracle.rule_q8(vh[r])
        assert np.array_equal(q[r].cpu().numpy(), rq), r
        assert s[r].item() == rs, r


# ------------------------------------------------------------------------------------------
# Expert FFN with the routing fixed (moe_experts_forward), every format, small shapes that still
# span several tiles and ragged token groups
# ------------------------------------------------------------------------------------------

FFN_CASES = [
    ("q8_0-swiglu", dict(fmt=mi.FMT_Q8_0, act=mi.ACT_SWIGLU)),
    ("i8row-swiglu", dict(fmt=mi.FMT_I8_ROW, act=mi.ACT_SWIGLU)),
    ("q8_0-relu2", dict(fmt=mi.FMT_Q8_0, act=mi.ACT_RELU2)),
    ("i8row-relu2", dict(fmt=mi.FMT_I8_ROW, act=mi.ACT_RELU2)),
    ("e2m1-relu2", dict(fmt=mi.FMT_E2M1, act=mi.ACT_RELU2, latent_bias_column=True)),
    ("e2m1-swiglu", dict(fmt=mi.FMT_E2M1, act=mi.ACT_SWIGLU)),
]


@pytest.mark.parametrize("name,kw", FFN_CASES, ids=[c[0] for c in FFN_CASES])
@pytest.mark.parametrize("xtype", [mi.X_BF16, mi.X_F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 5, 37])
def test_experts_forward_small(name, kw, xtype, T):
    w = mi.workload("tiny", T=T, d_model=192, E=6, k=3, d_ff=192, xtype=xtype, **kw)
    say("experts_forward", name, xtype, T)
    lay, x = gen(w)
    idx, wts, _, _ = oracle.route(x.cpu(), lay["w_router"].cpu(), None, w.k)
    runs = [(lay["experts"], 0)]
    if w.fmt == mi.FMT_E2M1:
        runs.append((lay["experts"], moe.F_ZERO_SKIP))
    else:
        runs.append((moe.repack_experts(lay["experts"], w.act), 0))
    ref = oracle_experts(mi.to_host(lay), x.cpu(), idx, wts, w.act)
    for ex, flags in runs:
        out = moe.experts_forward(x, torch.from_numpy(idx).to(DEV),
                                  torch.from_numpy(wts.astype(np.float32)).to(DEV), ex, w.act, flags)
        err = bf.rel_err(out.cpu().numpy(), ref)
        say("  fmt", ex["fmt"], "flags", flags, "rel err", err)
        assert err < EXACT_PRODUCT_TOL


@pytest.mark.parametrize("fmt", [mi.FMT_Q8_0, mi.FMT_I8_ROW], ids=["q8_0", "i8row"])
@pytest.mark.parametrize("xtype", [mi.X_BF16, mi.X_F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 2])
def test_small_batch_wide_grid(fmt, xtype, T):
    """T <= 2 on a gate/up grid of at least 512 blocks (8 or 16 slots x 64 feature tiles), where the
    gate/up takes two super-blocks per load batch and loads activations only in the lanes of valid
    rows: through the whole layer (the gate/up blocks route in-block) and with the routing fixed,
    plain and tiled weights, bf16 and fp32 activations, against the oracle."""
    w = mi.workload("tiny", T=T, d_model=512, E=64, k=8, d_ff=1024, fmt=fmt, xtype=xtype)
    say("small batch, wide grid", T, fmt, xtype)
    lay, x = gen(w)
    host = mi.to_host(lay)
    ref = oracle.layer_forward(x.cpu(), host["w_router"], None, host["experts"], w.k, w.act)
    for ex in (lay["experts"], moe.repack_experts(lay["experts"], w.act)):
        out, idx, wts = moe.layer_forward(x, lay["w_router"], None, ex, w.k, w.act, want_routing=True)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref["idx"])
        np.testing.assert_allclose(wts.cpu().numpy(), ref["w"], atol=1e-6)
        err = bf.rel_err(out.cpu().numpy(), ref["out"])
        out2 = moe.experts_forward(x, idx, wts, ex, w.act)
        err2 = bf.rel_err(out2.cpu().numpy(), ref["out"])
        say("  fmt", ex["fmt"], "rel err layer / fixed routing", err, err2)
        assert err < EXACT_PRODUCT_TOL and err2 < EXACT_PRODUCT_TOL


@pytest.mark.parametrize("d_model", [512, 1024, 1536, 2048, 2816, 6144, 8256])
@pytest.mark.parametrize("act", [mi.ACT_RELU2, mi.ACT_SWIGLU], ids=["relu2", "swiglu"])
@pytest.mark.parametrize("xtype", [mi.X_BF16, mi.X_F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 5])
def test_e2m1_row_widths(d_model, act, xtype, T):
    """E2M1 rows of 512 - 8256 codes: the lane-group up kernel (512 / 1024 / 2048), the general
    one (1536), the wide-row one with 2, 4 and 8 chunks per lane (2816 / 6144 / 8256), and one to
    nine 1024-output parts in the down kernel; dense and zero-skip, against the oracle."""
    w = mi.workload("tiny", T=T, d_model=d_model, E=6, k=3, d_ff=192, fmt=mi.FMT_E2M1, act=act,
                    xtype=xtype, latent_bias_column=act == mi.ACT_RELU2)
    say("e2m1 row widths", d_model, act, xtype, T)
    lay, x = gen(w)
    idx, wts, _, _ = oracle.route(x.cpu(), lay["w_router"].cpu(), None, w.k)
    ref = oracle_experts(mi.to_host(lay), x.cpu(), idx, wts, w.act)
    outs = []
    for flags in (0, moe.F_ZERO_SKIP):
        out = moe.experts_forward(x, torch.from_numpy(idx).to(DEV),
                                  torch.from_numpy(wts.astype(np.float32)).to(DEV), lay["experts"],
                                  w.act, flags)
        err = bf.rel_err(out.cpu().numpy(), ref)
        say("  flags", flags, "rel err", err)
        assert err < EXACT_PRODUCT_TOL
        outs.append(out)
    assert torch.equal(outs[0], outs[1])


# ------------------------------------------------------------------------------------------
# Whole layer (moe_layer_forward)
# ------------------------------------------------------------------------------------------

def test_tiny_layer_exactly_as_specified():
    """T=4, d=256, E=8, top-2, d_ff=512, SwiGLU, Q8_0, fp32 x, seed 0."""
    w = mi.workload("tiny")
    lay, x = gen(w)
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act,
                                      want_routing=True)
    ref = oracle.layer_forward(x.cpu(), lay["w_router"].cpu(), None,
                               mi.to_host(lay)["experts"], w.k, w.act)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    np.testing.assert_allclose(wts.cpu().numpy(), ref["w"], atol=1e-6)
    err = bf.rel_err(out.cpu().numpy(), ref["out"])
    say("tiny rel err", err)
    assert err < EXACT_PRODUCT_TOL


FULL_CASES = [("gemma_decode", 1, mi.FMT_Q8_0, 0), ("gemma_decode", 8, mi.FMT_Q8_0, 0),
              ("gemma_decode", 8, "q8_0_tiled", 0), ("gemma_decode", 1, "i8_row_tiled", 0),
              ("m3_decode", 32, "q8_0_tiled", 0),
              ("gemma_decode", 1, mi.FMT_I8_ROW, 0), ("gemma_decode", 8, mi.FMT_I8_ROW, 0),
              ("m3_decode", 1, mi.FMT_Q8_0, 0), ("m3_decode", 32, mi.FMT_Q8_0, 0),
              ("nemotron_latent", 1, mi.FMT_E2M1, 1), ("nemotron_latent", 1, mi.FMT_E2M1, 0),
              ("nemotron_latent", 8, mi.FMT_E2M1, 1), ("nemotron_latent", 32, mi.FMT_E2M1, 1),
              ("gemma_decode", 8, mi.FMT_E2M1, 0), ("m3_decode", 1, mi.FMT_E2M1, 0),
              ("m3_decode", 32, mi.FMT_E2M1, 0)]


@pytest.mark.parametrize("name,T,fmt,flags", FULL_CASES,
                         ids=[f"{n}-T{t}-f{f}-z{z}" for n, t, f, z in FULL_CASES])
def test_full_size_layer_sampled(name, T, fmt, flags):
    """Full-size layer on the GPU; the oracle computes every token on 96 sampled output columns
    (first, last and random ones), using only the experts the routing touches."""
    tiled = isinstance(fmt, str)
    if tiled:
        fmt = mi.FMT_Q8_0 if fmt == "q8_0_tiled" else mi.FMT_I8_ROW
    w = mi.workload(name, T=T, fmt=fmt)
    say("full layer", name, T, fmt, "tiled" if tiled else "plain", flags)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act,
                                      flags, want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(wts.cpu().numpy(), rw, atol=1e-6)
    rng = np.random.default_rng(5)
    cols = np.unique(np.concatenate([[0, w.d_model - 1], rng.choice(w.d_model, 94, replace=False)]))
    ref = oracle_experts(host, x.cpu(), ridx, rw, w.act, o_list=cols.astype(np.int32))
    got = out.cpu().numpy()[:, cols]
    err = bf.rel_err(got, ref)
    say("  rel err on sampled columns", err, "distinct experts", len(set(ridx.reshape(-1).tolist())))
    assert err < EXACT_PRODUCT_TOL


# The widest rows the library accepts (d_model = d_ff = 16384), every kernel family, a few tokens
# and two or three experts; the oracle computes 64 sampled output columns (first, last, random).
MAX_WIDTH_CASES = [("q8_0-tiled", mi.FMT_Q8_0, mi.ACT_SWIGLU, 0, True, 3, 2, 3),
                   ("i8row-relu2", mi.FMT_I8_ROW, mi.ACT_RELU2, 0, False, 2, 1, 2),
                   ("e2m1-relu2-zero-skip", mi.FMT_E2M1, mi.ACT_RELU2, 1, False, 2, 2, 2),
                   ("e2m1-swiglu", mi.FMT_E2M1, mi.ACT_SWIGLU, 0, False, 2, 1, 2),
                   ("prefill-i8row", mi.FMT_I8_ROW, mi.ACT_SWIGLU, 4, True, 5, 2, 2),
                   ("prefill-fp8", mi.FMT_FP8_ROW, mi.ACT_SWIGLU, 8, True, 3, 1, 2)]


@pytest.mark.parametrize("name,fmt,act,flags,tiled,T,k,E", MAX_WIDTH_CASES, ids=[c[0] for c in MAX_WIDTH_CASES])
def test_maximum_row_widths(name, fmt, act, flags, tiled, T, k, E):
    w = mi.workload("tiny", T=T, k=k, E=E, d_model=16384, d_ff=16384, fmt=fmt, act=act)
    say("maximum widths", name)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act, flags,
                                      want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    if flags & (moe.F_PREFILL_I8 | moe.F_PREFILL_FP8):
        check_prefill(out.cpu().numpy(), host, x.cpu(), ridx, rw, fp8=bool(flags & moe.F_PREFILL_FP8))
        return
    rng = np.random.default_rng(6)
    cols = np.unique(np.concatenate([[0, w.d_model - 1], rng.choice(w.d_model, 62, replace=False)]))
    ref = oracle_experts(host, x.cpu(), ridx, rw, w.act, o_list=cols.astype(np.int32))
    err = bf.rel_err(out.cpu().numpy()[:, cols], ref)
    say("  rel err on sampled columns", err)
    assert err < EXACT_PRODUCT_TOL


def test_route_and_permute_at_maximum_T():
    """T = 32768 tokens (the largest accepted) on the Gemma shape: 262,144 pairs through the
    multi-workgroup permute.  Ids of 16 sampled tokens against the oracle; the permutation arrays
    of every pair against the oracle's."""
    w = mi.workload("gemma_decode", T=32768)
    lay, x = gen(w)
    idx, wts = moe.route(x, lay["w_router"], lay["bias"], w.k)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    toks = np.array([0, 1, 4095, 4096, 8191, 12345, 16383, 16384, 20000, 24575, 30000, 32000,
                     32765, 32766, 32767, 777])
    ridx, rw, _, _ = oracle.route(x[toks].cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy()[toks], ridx)
    np.testing.assert_allclose(wts.cpu().numpy()[toks], rw, atol=1e-6)
    counts, offsets, perm, inv = moe.permute(idx, w.E)
    rc, ro, rp, ri = oracle.permute(idx.cpu().numpy(), w.E)
    for a, b in ((counts, rc), (offsets, ro), (perm, rp), (inv, ri)):
        assert np.array_equal(a.cpu().numpy(), b)


def test_prefill_at_maximum_T():
    """T = 32768 through the whole int8 prefill layer (262,144 pairs, ~2,100 M-tiles) on a narrow
    shape; 12 sampled tokens against the oracle."""
    w = mi.workload("gemma_prefill", T=32768, d_model=256, E=16, k=8, d_ff=256)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act)
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act,
                                      moe.F_PREFILL_I8, want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    toks = np.array([0, 1, 2, 8191, 8192, 16383, 16384, 24576, 32000, 32765, 32766, 32767])
    ridx, rw, _, _ = oracle.route(x[toks].cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy()[toks], ridx)
    check_prefill(out.cpu().numpy()[toks], host, x[toks].cpu(), ridx, rw, fp8=False)


def test_zero_skip_equals_dense_down_bitwise():
    w = mi.workload("nemotron_latent")
    lay, x = gen(w)
    a = moe.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act, moe.F_ZERO_SKIP)
    b = moe.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act, 0)
    assert torch.equal(a, b)


def test_three_runs_are_bitwise_identical():
    w = mi.workload("gemma_decode", T=8)
    lay, x = gen(w)
    outs = [moe.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act) for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


GRAPH_CASES = [("gemma_decode", 8, mi.FMT_Q8_0, 0), ("gemma_decode", 1, mi.FMT_Q8_0, 0),
               ("gemma_decode", 3, mi.FMT_I8_ROW, 0), ("m3_decode", 1, mi.FMT_Q8_0, 0),
               ("gemma_prefill", 512, mi.FMT_I8_ROW, 4), ("gemma_prefill", 512, mi.FMT_FP8_ROW, 8)]


@pytest.mark.parametrize("name,T,fmt,flags", GRAPH_CASES, ids=[f"{c[0]}-T{c[1]}-f{c[3]}" for c in GRAPH_CASES])
def test_graph_replay_matches_eager(name, T, fmt, flags):
    """The layer captured in a HIP graph and replayed several times, with eager work and
    synchronisations in between, gives the eager output bit for bit on every replay: decode with
    the separate and the fused combine (MiniMax-M3-shaped T = 1: a gate/up grid of 768 blocks,
    two super-blocks per load batch), and the int8 and E4M3 prefill paths (4,096 pairs: the
    multi-workgroup permute; the E4M3 GEMMs' direct-to-LDS ring)."""
    w = mi.workload(name, T=T, fmt=fmt)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act)
    b = lay["bias"]
    ws = moe.alloc_workspace(moe.workspace_bytes(w.T, w.k, ex, w.act, flags))
    out = torch.empty((w.T, w.d_model), device=DEV)
    ref = moe.layer_forward(x, lay["w_router"], b, ex, w.k, w.act, flags).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.layer_forward(x, lay["w_router"], b, ex, w.k, w.act, flags, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.layer_forward(x, lay["w_router"], b, ex, w.k, w.act, flags, out=out, ws=ws)
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        other = moe.layer_forward(x * 0.5, lay["w_router"], b, ex, w.k, w.act, flags)   # eager work
        torch.cuda.synchronize()
        assert not torch.equal(other, ref)


GRAPH_SMALL = [("gemma_decode", dict(T=2, n_shared=2)),                          # in-block routing
               ("tiny", dict(T=2, E=300, k=32, d_model=64, d_ff=64, n_shared=1))]  # sorted small select


@pytest.mark.parametrize("name,kw", GRAPH_SMALL, ids=["inblock-shared", "sorted-select-shared"])
def test_graph_replay_small_batch_paths(name, kw):
    """The small-batch routing paths with shared experts, captured in a HIP graph and replayed
    with eager calls on other inputs in between: every replay equals the eager output bit for bit
    (the records and permutation are rebuilt by the replayed kernels, not left over)."""
    w = mi.workload(name, **kw)
    lay, x = gen(w, T=w.T)
    ex = moe.repack_experts(lay["experts"], w.act)
    b = lay["bias"]
    ws = moe.alloc_workspace(moe.workspace_bytes(w.T, w.k, ex, w.act, 0))
    out = torch.empty((w.T, w.d_model), device=DEV)
    ref = moe.layer_forward(x, lay["w_router"], b, ex, w.k, w.act).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.layer_forward(x, lay["w_router"], b, ex, w.k, w.act, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.layer_forward(x, lay["w_router"], b, ex, w.k, w.act, out=out, ws=ws)
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        # eager work on the same workspace with another routing in between
        moe.layer_forward(-x, lay["w_router"], b, ex, w.k, w.act, ws=ws)
        torch.cuda.synchronize()


def test_workspace_reuse_across_batch_sizes():
    """One workspace, sized for T = 8, reused by calls with T = 8, 1, 3, 2 and 8 again (the small
    select kernel, the in-block routing, the fused down + combine, in turn): every call equals a
    call with a fresh workspace bit for bit, so nothing an earlier, larger call left is read."""
    w = mi.workload("gemma_decode", T=8, n_shared=1)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act)
    ws = moe.alloc_workspace(moe.workspace_bytes(8, w.k, ex, w.act, 0))
    for T in (8, 1, 3, 2, 8):
        xs = x[:T].contiguous()
        got = moe.layer_forward(xs, lay["w_router"], lay["bias"], ex, w.k, w.act, ws=ws).clone()
        fresh = moe.layer_forward(xs, lay["w_router"], lay["bias"], ex, w.k, w.act)
        torch.cuda.synchronize()
        assert torch.equal(got, fresh), T


@pytest.mark.parametrize("name,fmt,flags,T", [("gemma_decode", mi.FMT_Q8_0, 0, 3),
                                              ("gemma_decode", mi.FMT_Q8_0, 0, 2),
                                              ("nemotron_latent", mi.FMT_E2M1, 1, 3),
                                              ("gemma_prefill", mi.FMT_I8_ROW, 4, 3),
                                              ("gemma_prefill", mi.FMT_FP8_ROW, 8, 3)])
def test_no_uncomputed_output_survives_poison(name, fmt, flags, T):
    """Output and workspace are NaN-filled before the call; every output must be overwritten
    (T = 2 takes the fused down + combine kernel)."""
    w = mi.workload(name, T=T, fmt=fmt)
    lay, x = gen(w, T=T)
    nbytes = moe.workspace_bytes(T, w.k, lay["experts"], w.act, flags)
    ws = torch.full((nbytes // 4 + 64,), float("nan"), device=DEV).view(torch.uint8)
    out = torch.full((T, w.d_model), float("nan"), device=DEV)
    moe.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act, flags, out=out, ws=ws)
    assert not torch.isnan(out).any()


def test_k_equals_E_uniform_router_is_the_dense_average():
    w = mi.workload("tiny", E=8, k=8, T=3)
    lay, x = gen(w)
    zero_r = torch.zeros_like(lay["w_router"])
    out = moe.layer_forward(x, zero_r, None, lay["experts"], 8, w.act)
    idx = torch.arange(8, dtype=torch.int32, device=DEV).repeat(3, 1)
    per = []
    for e in range(8):
        one = torch.full((3, 1), e, dtype=torch.int32, device=DEV)
        per.append(moe.experts_forward(x, one, torch.ones((3, 1), device=DEV), lay["experts"], w.act))
    dense = torch.stack(per).mean(0)
    assert bf.rel_err(out.cpu().numpy(), dense.double().cpu().numpy()) < EXACT_PRODUCT_TOL
    ref = oracle.experts_forward(x.cpu(), idx.cpu().numpy(), np.full((3, 8), 1 / 8),
                                 mi.to_host(lay)["experts"], w.act)
    assert bf.rel_err(out.cpu().numpy(), ref) < EXACT_PRODUCT_TOL


def test_single_expert_single_token():
    w = mi.workload("tiny", E=1, k=1, T=1)
    lay, x = gen(w)
    out = moe.layer_forward(x, lay["w_router"], None, lay["experts"], 1, w.act)
    ref = oracle.layer_forward(x.cpu(), lay["w_router"].cpu(), None, mi.to_host(lay)["experts"], 1, w.act)
    assert bf.rel_err(out.cpu().numpy(), ref["out"]) < EXACT_PRODUCT_TOL


def test_large_batch_without_int8_activations():
    """T = 2048 on the Gemma shape through the bf16 matrix-core path (more than 1024 pairs: the
    down outputs go through the per-pair buffer and the separate fixed-order combine)."""
    w = mi.workload("gemma_prefill", fmt=mi.FMT_Q8_0)
    lay, x = gen(w)
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act,
                                      want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    toks = np.array([0, 1, 777, 2047])
    ridx, rw, _, _ = oracle.route(x[toks].cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy()[toks], ridx)
    ref = oracle_experts(host, x[toks].cpu(), ridx, rw, w.act)
    err = bf.rel_err(out.cpu().numpy()[toks], ref)
    say("T=2048 bf16-path rel err", err)
    assert err < EXACT_PRODUCT_TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["plain", "tiled"])
@pytest.mark.parametrize("n_shared", [0, 1])
def test_token_rows_do_not_depend_on_the_batch(tiled, n_shared):
    """Each token's output depends on that token alone.  Batches of 1 and 2 tokens take the fused
    down + combine kernel, 3 and 8 the down kernel and the separate combine; the same tokens'
    rows agree across them to fp32 summation order, and match the oracle."""
    w = mi.workload("gemma_decode", T=8, n_shared=n_shared)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    outs = {T: moe.layer_forward(x[:T].contiguous(), lay["w_router"], lay["bias"], ex, w.k, w.act)
            for T in (1, 2, 3, 8)}
    torch.cuda.synchronize()
    full = outs[8].cpu().numpy()
    for T in (1, 2, 3):
        err = bf.rel_err(outs[T].cpu().numpy(), full[:T])
        say(f"  T={T} vs T=8 rows", err)
        assert err < 1e-5
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x[:2].cpu(), host["w_router"], host["bias"], w.k)
    cols = np.arange(0, w.d_model, 37, dtype=np.int32)
    ref = oracle_experts(host, x[:2].cpu(), ridx, rw, w.act, o_list=cols)
    assert bf.rel_err(outs[2].cpu().numpy()[:, cols], ref) < EXACT_PRODUCT_TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["plain", "tiled"])
@pytest.mark.parametrize("n_shared", [0, 2])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_in_block_routing_matches_the_permute_path(tiled, n_shared, T):
    """Small batches (T k <= 64, E <= 128): at T <= 2 the layer's gate/up blocks select the experts
    themselves and write the records the later kernels read, at T = 3, 4 the small select kernel
    does; moe_route + moe_experts_forward take the separate top-k and the general permute.  Same ids and weights, and the same output, bit for bit
    (the same expert kernels on the same records); the ids equal the oracle's."""
    w = mi.workload("gemma_decode", T=T, n_shared=n_shared)
    lay, x = gen(w, T=T)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    say("in-block routing", T, n_shared, tiled)
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act, want_routing=True)
    ridx, rw = moe.route(x, lay["w_router"], lay["bias"], w.k)
    ref = moe.experts_forward(x, ridx, rw, ex, w.act)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx) and torch.equal(wts, rw)
    assert torch.equal(out, ref)
    host = mi.to_host(lay)
    oidx, ow, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.abs(wts.cpu().numpy() - ow).max() < 1e-6


E2M1_ROUTE_CASES = [(512, 22, 1, 0), (512, 22, 2, 2), (200, 8, 1, 1), (64, 8, 2, 0), (512, 32, 2, 0),
                    (256, 64, 1, 0), (129, 1, 1, 0)]


@pytest.mark.parametrize("flags", [0, 1], ids=["dense", "zero-skip"])
@pytest.mark.parametrize("E,k,T,S", E2M1_ROUTE_CASES, ids=[f"E{e}-k{k}-T{t}-S{s}" for e, k, t, s in E2M1_ROUTE_CASES])
def test_e2m1_in_block_routing_matches_the_permute_path(E, k, T, S, flags):
    """E2M1 experts at d_model 1024 (the lane-group up kernel) with T <= 2: the up blocks select the
    experts themselves (up to 512), while moe_route + moe_experts_forward take the separate top-k
    and permute.  Same ids and weights and the same output bit for bit; ids equal the oracle's and
    the output matches it on sampled columns."""
    w = mi.workload("nemotron_latent", T=T, E=E, k=k, n_shared=S)
    lay, x = gen(w, T=T)
    say("e2m1 in-block routing", E, k, T, S, flags)
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act, flags,
                                      want_routing=True)
    ridx, rw = moe.route(x, lay["w_router"], lay["bias"], w.k)
    ref = moe.experts_forward(x, ridx, rw, lay["experts"], w.act, flags)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx) and torch.equal(wts, rw)
    assert torch.equal(out, ref)
    host = mi.to_host(lay)
    oidx, ow, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.abs(wts.cpu().numpy() - ow).max() < 1e-6
    cols = np.unique(np.concatenate([[0, w.d_model - 1], np.arange(5, w.d_model, 97)])).astype(np.int32)
    oref = oracle_experts(host, x.cpu(), oidx, ow, w.act, o_list=cols)
    err = bf.rel_err(out.cpu().numpy()[:, cols], oref)
    say("  rel err on sampled columns", err)
    assert err < EXACT_PRODUCT_TOL


ROUTE_EDGE = [("gemma_decode", dict(T=2, k=32)),        # in-block routing at T k = 64
              ("gemma_decode", dict(T=4, k=16)),        # small select kernel at T k = 64
              ("gemma_decode", dict(T=2, k=1)),
              ("gemma_decode", dict(T=1, E=64, k=6)),   # E <= 64: every lane's second key empty
              ("gemma_decode", dict(T=3, E=64, k=6)),
              ("gemma_decode", dict(T=2, act=mi.ACT_RELU2, n_shared=1)),
              ("gemma_decode", dict(T=8, n_shared=4)),
              ("tiny", dict(T=2)),                      # E = 8, fp32 x
              ("tiny", dict(T=4)),
              ("tiny", dict(T=2, k=8)),                 # k = E: every expert selected (in-block)
              ("tiny", dict(T=8, k=8)),                 # k = E, T k = 64 (small select)
              ("tiny", dict(T=1, E=1, k=1)),            # a single expert
              ("tiny", dict(T=5, E=1, k=1, n_shared=1)),
              ("m3_decode", dict(T=1)),                 # Zipf-skewed router
              ("m3_decode", dict(T=3, fmt=mi.FMT_I8_ROW)),
              # more than 128 experts: the small sorted select kernel (T <= 16 / keys per lane)
              ("tiny", dict(T=1, E=512, k=22, d_model=64, d_ff=64)),
              ("tiny", dict(T=4, E=256, k=16, d_model=64, d_ff=64)),
              ("tiny", dict(T=2, E=300, k=32, d_model=64, d_ff=64, n_shared=2)),
              ("nemotron_latent", dict(T=2))]

@pytest.mark.parametrize("name,kw", ROUTE_EDGE, ids=[f"{n}-{'-'.join(f'{a}{b}' for a, b in kw.items())}"
                                                      for n, kw in ROUTE_EDGE])
def test_in_block_routing_edge_shapes(name, kw):
    """The in-block routing and the small select kernels at their limits (T k = 64, k = 1, E <= 64,
    more than 128 experts, ReLU^2 with a shared expert, four shared experts, Zipf-skewed routers,
    E2M1 experts): ids, weights and output equal the separate top-k + general permute path's."""
    w = mi.workload(name, **kw)
    lay, x = gen(w, T=w.T)
    say("in-block routing edge", name, kw)
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act,
                                      want_routing=True)
    ridx, rw = moe.route(x, lay["w_router"], lay["bias"], w.k)
    ref = moe.experts_forward(x, ridx, rw, lay["experts"], w.act)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx) and torch.equal(wts, rw)
    assert torch.equal(out, ref)
    host = mi.to_host(lay)
    oidx, _, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), oidx)


def test_in_block_routing_ties():
    """All logits equal (zero router, no bias): every token takes experts 0 .. k-1, weight 1/k,
    on the in-block routing path (T = 3) as on the separate top-k."""
    w = mi.workload("gemma_decode", T=3)
    lay, x = gen(w, T=3)
    zr = torch.zeros_like(lay["w_router"])
    out, idx, wts = moe.layer_forward(x, zr, None, lay["experts"], w.k, w.act, want_routing=True)
    ref = moe.experts_forward(x, idx, wts, lay["experts"], w.act)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(w.k, dtype=np.int32), (3, 1)))
    assert np.all(wts.cpu().numpy() == np.float32(1.0 / w.k))
    assert torch.equal(out, ref)


def test_out_of_range_ids_are_clamped_not_faulted():
    w = mi.workload("tiny", T=2)
    lay, x = gen(w, T=2)
    bad = torch.tensor([[9, -3], [1, 100]], dtype=torch.int32, device=DEV)
    good = torch.tensor([[7, 0], [1, 7]], dtype=torch.int32, device=DEV)
    wts = torch.tensor([[0.6, 0.4], [0.5, 0.5]], device=DEV)
    a = moe.experts_forward(x, bad, wts, lay["experts"], w.act)
    b = moe.experts_forward(x, good, wts, lay["experts"], w.act)
    assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------
# Batched prefill with int8 activations (MOE_F_PREFILL_I8)
# ------------------------------------------------------------------------------------------
# The oracle applies the same rule Q (fp32, round half to even) to x and to its fp32-rounded h.
# x codes are bit-exact (test_quantize_rows_bit_exact); h differs from the oracle's by fp32
# accumulation order (~1e-6 relative), which can move a code by one step where h * (127 / max|h|)
# sits on a rounding midpoint: outputs are held to the stated 2e-3 beyond what those codes can
# move them by (check_prefill).

@pytest.mark.parametrize("fmt", [mi.FMT_I8_ROW, mi.FMT_Q8_0], ids=["i8row", "q8_0"])
@pytest.mark.parametrize("tiled", [False, True], ids=["plain", "tiled"])
@pytest.mark.parametrize("T,d_ff", [(1, 192), (37, 192), (300, 192), (37, 1088), (300, 4160)])
def test_prefill_i8_small(tiled, T, d_ff, fmt):
    w = mi.workload("gemma_prefill", T=T, d_model=192, E=6, k=3, d_ff=d_ff, fmt=fmt)
    say("prefill small", T, d_ff, fmt, "tiled" if tiled else "plain")
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act,
                                      moe.F_PREFILL_I8, want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    check_prefill(out.cpu().numpy(), host, x.cpu(), ridx, rw, fp8=False)


@pytest.mark.parametrize("tiled,fmt", [(False, mi.FMT_I8_ROW), (True, mi.FMT_I8_ROW), (True, mi.FMT_Q8_0)],
                         ids=["i8row-plain", "i8row-tiled", "q8_0-tiled"])
def test_prefill_i8_full_size_sampled_tokens(tiled, fmt):
    """T = 2048 on the Gemma shape with the Zipf router prior (ragged groups); the oracle checks 12
    sampled tokens in full."""
    w = mi.workload("gemma_prefill", fmt=fmt)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act,
                                      moe.F_PREFILL_I8, want_routing=True)
    torch.cuda.synchronize()
    counts = torch.bincount(idx.reshape(-1).long(), minlength=w.E)
    say("  group sizes min/max", int(counts.min()), int(counts.max()))
    host = mi.to_host(lay)
    toks = np.array([0, 1, 2, 511, 1000, 1023, 1024, 1500, 2000, 2045, 2046, 2047])
    ridx, rw, _, _ = oracle.route(x[toks].cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy()[toks], ridx)
    check_prefill(out.cpu().numpy()[toks], host, x[toks].cpu(), ridx, rw, fp8=False)


# ------------------------------------------------------------------------------------------
# Batched prefill with E4M3 activations and weights (MOE_F_PREFILL_FP8)
# ------------------------------------------------------------------------------------------
# The oracle applies rule Q8 to x and to its fp32-rounded h.  E4M3 x E4M3 products are exact in
# fp32 and the matrix cores add them in fp32, so h differs from the oracle's by accumulation
# order only (~1e-6 relative).  An E4M3 step is 1/16 to 1/8 of the value, so one h code taken on
# the other side of a midpoint moves a pair's output by up to ~1e-2 at d_ff = 192: outputs are
# held to the stated 2e-3 beyond what such codes can move them by (check_prefill).

@pytest.mark.parametrize("tiled", [False, True], ids=["plain", "tiled"])
@pytest.mark.parametrize("T,d_ff", [(1, 192), (37, 192), (300, 704), (37, 1088), (300, 4160)])
def test_prefill_fp8_small(tiled, T, d_ff):
    w = mi.workload("gemma_prefill", T=T, d_model=192, E=6, k=3, d_ff=d_ff, fmt=mi.FMT_FP8_ROW)
    say("prefill fp8 small", T, d_ff, "tiled" if tiled else "plain")
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act,
                                      moe.F_PREFILL_FP8, want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    check_prefill(out.cpu().numpy(), host, x.cpu(), ridx, rw, fp8=True)


@pytest.mark.parametrize("tiled", [False, True], ids=["plain", "tiled"])
def test_prefill_fp8_full_size_sampled_tokens(tiled):
    """T = 2048 on the Gemma shape, E4M3 weights, Zipf router prior; 12 sampled tokens in full."""
    w = mi.workload("gemma_prefill", fmt=mi.FMT_FP8_ROW)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act,
                                      moe.F_PREFILL_FP8, want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    toks = np.array([0, 1, 2, 511, 1000, 1023, 1024, 1500, 2000, 2045, 2046, 2047])
    ridx, rw, _, _ = oracle.route(x[toks].cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy()[toks], ridx)
    check_prefill(out.cpu().numpy()[toks], host, x[toks].cpu(), ridx, rw, fp8=True)
    assert torch.isfinite(out).all()


def test_prefill_fp8_is_deterministic():
    w = mi.workload("gemma_prefill", T=512, fmt=mi.FMT_FP8_ROW)
    lay, x = gen(w)
    a = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act, moe.F_PREFILL_FP8)
    b = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act, moe.F_PREFILL_FP8)
    assert torch.equal(a, b)


SHARED_CASES = [("q8_0", "tiny", dict(E=8, k=2, d_model=256, d_ff=512), 1, 0, False),
                ("q8_0-tiled", "tiny", dict(E=8, k=2, d_model=256, d_ff=512), 5, 0, True),
                ("i8row", "tiny", dict(E=8, k=2, d_model=256, d_ff=512, fmt=mi.FMT_I8_ROW), 37, 0, False),
                ("e2m1-zs", "nemotron_latent", dict(E=32, k=8), 3, 1, False),
                ("prefill-i8row", "gemma_prefill", dict(T=300, d_model=192, E=6, k=3, d_ff=192), 300, 4, True),
                ("prefill-q8_0", "gemma_prefill", dict(d_model=192, E=6, k=3, d_ff=704, fmt=mi.FMT_Q8_0),
                 1000, 4, False),
                ("prefill-fp8", "gemma_prefill", dict(d_model=192, E=6, k=3, d_ff=704, fmt=mi.FMT_FP8_ROW),
                 1000, 8, True)]


@pytest.mark.parametrize("name,wl,kw,T,flags,tiled", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
@pytest.mark.parametrize("S", [1, 2])
def test_layer_with_shared_experts(name, wl, kw, T, flags, tiled, S):
    """Shared experts beside the routed ones (every token, weight 1, after the routed slots):
    decode kernels, zero-skip E2M1, and the int8 / fp8 prefill GEMMs with their extra tiles
    (3000 pairs take the multi-workgroup permute), against the oracle."""
    kw = dict(kw)
    kw["T"] = T
    w = mi.workload(wl, n_shared=S, **kw)
    say("shared experts", name, S, T)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act, flags,
                                      want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    if flags & (moe.F_PREFILL_I8 | moe.F_PREFILL_FP8):
        check_prefill(out.cpu().numpy(), host, x.cpu(), ridx, rw, fp8=bool(flags & moe.F_PREFILL_FP8))
        ref = oracle_experts(host, x.cpu(), ridx, rw, w.act, i8act=bool(flags & moe.F_PREFILL_I8),
                             f8act=bool(flags & moe.F_PREFILL_FP8))
    else:
        ref = oracle_experts(host, x.cpu(), ridx, rw, w.act)
        err = bf.rel_err(out.cpu().numpy(), ref)
        say("  rel err", err)
        assert err < EXACT_PRODUCT_TOL
    # the shared experts change the output: the same layer without them differs
    plain = moe.layer_forward(x, lay["w_router"], lay["bias"], dict(ex, n_shared=0), w.k, w.act, flags)
    assert bf.rel_err(plain.cpu().numpy(), ref) > 1e-2


DEGENERATE_PREFILL = [("one-expert", dict(E=1, k=1, T=300)), ("k-equals-E", dict(E=4, k=4, T=150)),
                      ("fp32-x", dict(E=6, k=3, T=200, xtype=mi.X_F32))]


@pytest.mark.parametrize("fp8", [False, True], ids=["i8row", "fp8"])
@pytest.mark.parametrize("name,kw", DEGENERATE_PREFILL, ids=[c[0] for c in DEGENERATE_PREFILL])
def test_prefill_degenerate_cases(name, kw, fp8):
    """Prefill with one expert taking every pair (several M-tiles of one expert), with k = E (every
    expert on every token), and with fp32 activations; every case also carries zero rows of x
    (rule a = 0: codes 0, scale 0, so those tokens' outputs are exactly 0)."""
    w = mi.workload("gemma_prefill", d_model=192, d_ff=256, fmt=mi.FMT_FP8_ROW if fp8 else mi.FMT_I8_ROW,
                    zipf_s=None, **kw)
    lay, x = gen(w)
    x[3] = 0
    x[w.T - 1] = 0
    ex = moe.repack_experts(lay["experts"], w.act)
    flags = moe.F_PREFILL_FP8 if fp8 else moe.F_PREFILL_I8
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act, flags, want_routing=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[3] == 0) and np.all(got[w.T - 1] == 0)
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    check_prefill(got, host, x.cpu(), ridx, rw, fp8=fp8)


def test_prefill_is_deterministic():
    w = mi.workload("gemma_prefill", T=512)
    lay, x = gen(w)
    a = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act, moe.F_PREFILL_I8)
    b = moe.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act, moe.F_PREFILL_I8)
    assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------
# Tiled layout: the repack is a pure byte permutation (checked against a numpy tiling)
# ------------------------------------------------------------------------------------------

def np_tile(W, M):
    """[E, R, K] -> flat tiled bytes: tile ((e*NT + t)*S + s)*M + m, lane n + 16g, then j, i."""
    E, R, K = W.shape
    NT, S = R // M // 16, K // 64
    return W.reshape(E, M, NT, 16, S, 2, 4, 8).transpose(0, 2, 4, 1, 6, 3, 5, 7).reshape(-1)


def np_tile_scales(Sc, M):
    E, R, KB = Sc.shape
    NT, S = R // M // 16, KB // 2
    return Sc.reshape(E, M, NT, 16, S, 2).transpose(0, 2, 4, 1, 3, 5).reshape(-1)


@pytest.mark.parametrize("fmt,act", [(mi.FMT_Q8_0, mi.ACT_SWIGLU), (mi.FMT_Q8_0, mi.ACT_RELU2),
                                     (mi.FMT_I8_ROW, mi.ACT_SWIGLU), (mi.FMT_FP8_ROW, mi.ACT_SWIGLU)])
def test_repack_is_the_documented_byte_permutation(fmt, act):
    w = mi.workload("tiny", fmt=fmt, act=act, E=3, d_model=192, d_ff=128)
    lay = mi.make_layer(w, 0, DEV)
    t = moe.repack_experts(lay["experts"], act)
    torch.cuda.synchronize()
    M = 2 if act == mi.ACT_SWIGLU else 1
    src = {k: v.cpu().numpy() for k, v in lay["experts"].items() if isinstance(v, torch.Tensor)}
    got = {k: v.cpu().numpy() for k, v in t.items() if isinstance(v, torch.Tensor)}
    assert np.array_equal(got["gate_up"].reshape(-1), np_tile(src["gate_up"], M))
    assert np.array_equal(got["down"].reshape(-1), np_tile(src["down"], 1))
    if fmt == mi.FMT_Q8_0:
        assert np.array_equal(got["gate_up_scales"].view(np.uint16).reshape(-1),
                              np_tile_scales(src["gate_up_scales"].view(np.uint16), M))
        assert np.array_equal(got["down_scales"].view(np.uint16).reshape(-1),
                              np_tile_scales(src["down_scales"].view(np.uint16), 1))
    else:
        assert np.array_equal(got["gate_up_scales"], src["gate_up_scales"])
        assert np.array_equal(got["down_scales"], src["down_scales"])
    # and the multiset of bytes is unchanged
    assert np.array_equal(np.sort(got["gate_up"].reshape(-1)), np.sort(src["gate_up"].reshape(-1)))


# ------------------------------------------------------------------------------------------
# Must-fail checks: each corrupts one convention and parity must break
# ------------------------------------------------------------------------------------------

def test_swapped_nibbles_break_parity():
    w = mi.workload("nemotron_latent", E=32, k=8)
    lay, x = gen(w)
    ref_out = moe.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act)
    ex = dict(lay["experts"])
    for key in ("gate_up", "down"):
        b = ex[key]
        ex[key] = ((b & 15) << 4) | (b >> 4)
    bad = moe.layer_forward(x, lay["w_router"], None, ex, w.k, w.act)
    assert bf.rel_err(bad.cpu().numpy(), ref_out.double().cpu().numpy()) > 0.1


def test_swapped_gate_up_halves_break_parity():
    w = mi.workload("gemma_decode", E=16)
    lay, x = gen(w)
    ok = moe.layer_forward(x, lay["w_router"], None, lay["experts"], w.k, w.act)
    ex = dict(lay["experts"])
    d_ff = w.d_ff
    ex["gate_up"] = torch.cat([ex["gate_up"][:, d_ff:], ex["gate_up"][:, :d_ff]], 1).contiguous()
    ex["gate_up_scales"] = torch.cat([ex["gate_up_scales"][:, d_ff:], ex["gate_up_scales"][:, :d_ff]], 1).contiguous()
    bad = moe.layer_forward(x, lay["w_router"], None, ex, w.k, w.act)
    assert bf.rel_err(bad.cpu().numpy(), ok.double().cpu().numpy()) > 0.1


# ------------------------------------------------------------------------------------------
# Routing of every timed layer instance, through the layer call's own selection path
# ------------------------------------------------------------------------------------------

INSTANCE_ROUTE_CASES = [("gemma_decode", 1), ("gemma_decode", 8), ("nemotron_latent", 1),
                        ("nemotron_latent", 8), ("m3_decode", 1), ("m3_decode", 32)]


@pytest.mark.parametrize("name,T", INSTANCE_ROUTE_CASES, ids=[f"{n}-T{t}" for n, t in INSTANCE_ROUTE_CASES])
def test_every_timed_instance_routes_like_the_oracle(name, T):
    """The ids and weights of moe_layer_forward (the selection path the timed calls take at this
    batch size) for the router of every layer instance the benchmark times, with instance 0's
    experts, against the oracle's."""
    w = mi.workload(name, T=T)
    say("every instance", name, T, w.instances)
    lay = mi.make_layer(w, 0, DEV)
    ws = moe.alloc_workspace(moe.workspace_bytes(T, w.k, lay["experts"], w.act, 0))
    for i in range(w.instances):
        wr, bias = mi.make_router(w, i, DEV)
        x = mi.make_x(w, i, device=DEV)
        _, idx, wts = moe.layer_forward(x, wr, bias, lay["experts"], w.k, w.act, 0, ws=ws, want_routing=True)
        torch.cuda.synchronize()
        ridx, rw, _, gap = oracle.route(x.cpu(), wr.cpu(), None if bias is None else bias.cpu(), w.k)
        assert np.array_equal(idx.cpu().numpy(), ridx), f"instance {i}: top-k ids differ from the oracle"
        np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=0, atol=1e-6)
    say("  all", w.instances, "instances bit-exact")


# ------------------------------------------------------------------------------------------
# Batched prefill: h and its codes element by element
# ------------------------------------------------------------------------------------------

def _pair_order(h_oracle, T, k, S):
    """Oracle rows (t (k + S) + j) in the library's pair order (t k + j, then k T + s T + t)."""
    idx = [t * (k + S) + j for t in range(T) for j in range(k)]
    idx += [t * (k + S) + k + s for s in range(S) for t in range(T)]
    return h_oracle[np.array(idx)]


@pytest.mark.parametrize("S", [0, 1], ids=["routed", "shared"])
@pytest.mark.parametrize("fmt,tiled", [(mi.FMT_I8_ROW, True), (mi.FMT_Q8_0, True), (mi.FMT_I8_ROW, False),
                                       (mi.FMT_FP8_ROW, True)], ids=["i8row-tiled", "q8_0-tiled", "i8row-plain",
                                                                     "fp8-tiled"])
def test_prefill_h_and_codes_elementwise(fmt, tiled, S):
    """The prefill path's h (fp32) and its rule-Q / Q8 codes and row scales, read back from the
    workspace, against the oracle's own, element by element, at a shape with several 128-row
    tiles per expert and ragged last tiles.  h may differ from the oracle's only by fp32 summation
    order: within the window the output check (tests/prefill_check) assumes.  Codes must be equal
    except where that window straddles a rounding midpoint, and there at most one code step apart."""
    from tests.prefill_check import H_ABS, H_REL, _ambiguous_codes
    fp8 = fmt == mi.FMT_FP8_ROW
    flags = moe.F_PREFILL_FP8 if fp8 else moe.F_PREFILL_I8
    w = mi.workload("gemma_prefill", T=300, d_model=192, E=4, k=2, d_ff=192, fmt=fmt, n_shared=S)
    say("prefill h/codes", fmt, "tiled" if tiled else "plain", "shared", S)
    lay, x = gen(w)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    ws = moe.alloc_workspace(moe.workspace_bytes(w.T, w.k, ex, w.act, flags))
    out, idx, wts = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act, flags, ws=ws,
                                      want_routing=True)
    h, hq, sh = moe.read_intermediates(w.T, w.k, ex, w.act, flags, ws)
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.E)
    say("  group sizes", counts.tolist())
    assert counts.max() > 2 * 128 and (counts % 128 != 0).all()
    host = mi.to_host(lay)
    ridx, rw, _, _ = oracle.route(x.cpu(), host["w_router"], host["bias"], w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    fwd = oracle.experts_forward_f8act if fp8 else oracle.experts_forward_i8act
    res = fwd(x.cpu(), ridx, rw, host["experts"], want_h=True)
    href = _pair_order(res["h"], w.T, w.k, S).astype(np.float32)
    hg, qg, sg = h.cpu().numpy(), hq.cpu().numpy(), sh.cpu().numpy()
    n_flag = n_moved = 0
    for r in range(href.shape[0]):
        a = float(np.abs(href[r]).max())
        diff = np.abs(hg[r].astype(np.float64) - href[r])
        assert (diff <= H_REL * np.abs(href[r]) + H_ABS * a).all(), f"h row {r}: max diff {diff.max():.3g}"
        qref, sref = (oracle.rule_q8 if fp8 else oracle.rule_q)(href[r])
        assert abs(float(sg[r]) - float(sref)) <= 2e-6 * float(sref), f"row {r} scale"
        amb, _ = _ambiguous_codes(href[r], fp8)
        n_flag += int(amb.sum())
        got = qg[r] if fp8 else qg[r].view(np.int8)
        assert np.array_equal(got[~amb], qref[~amb]), f"h codes of row {r} differ away from a midpoint"
        if fp8:
            g8, r8 = got[amb].astype(np.int32), qref[amb].astype(np.int32)
            same_sign = (g8 & 0x80) == (r8 & 0x80)
            assert ((np.abs((g8 & 0x7F) - (r8 & 0x7F)) <= 1) & (same_sign | ((g8 & 0x7F) == 0))).all()
        else:
            assert (np.abs(got[amb].astype(np.int32) - qref[amb].astype(np.int32)) <= 1).all()
        n_moved += int((got[amb] != qref[amb]).sum())
    say(f"  {href.size} h values; {n_flag} near a midpoint, {n_moved} of them one step apart")
    check_prefill(out.cpu().numpy(), host, x.cpu(), ridx, rw, fp8=fp8)
