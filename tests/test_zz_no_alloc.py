"""moe_layer_forward_static (the entry point that allocates nothing, for callers that cannot
allocate device memory) against moe_layer_forward with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so outputs and routing must be equal bit for bit.
Two calls in a row share the static buffer, the second with a smaller batch; a third call on a
size beyond the buffer must be rejected before anything runs.  This file is collected last, so
that it passes both alone in a fresh process and after every other test.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_expert_router_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _case(name, T, fmt=None, tiled=False, flags=0, **kw):
    w = mi.workload(name, T=T, **({} if fmt is None else {"fmt": fmt}), **kw)
    lay = mi.make_layer(w, 0, DEV)
    ex = moe.repack_experts(lay["experts"], w.act) if tiled else lay["experts"]
    return w, lay, ex, flags


CASES = [("gemma-q8_0-tiled", dict(name="gemma_decode", T=8, fmt=mi.FMT_Q8_0, tiled=True), 1),
         ("nemotron-zero-skip", dict(name="nemotron_latent", T=8, flags=moe.F_ZERO_SKIP), 1),
         ("tiny-shared", dict(name="tiny", T=37, n_shared=1), 5),
         ("prefill-i8row", dict(name="gemma_prefill", T=300, d_model=192, E=6, k=3, d_ff=192,
                                fmt=mi.FMT_I8_ROW, flags=moe.F_PREFILL_I8), 77)]


@pytest.mark.parametrize("label,kw,T2", CASES, ids=[c[0] for c in CASES])
def test_static_entry_matches_the_workspace_entry(label, kw, T2):
    """Two calls in a row (the second with fewer tokens) equal moe_layer_forward bit for bit."""
    kw = dict(kw)
    name, T = kw.pop("name"), kw.pop("T")
    w, lay, ex, flags = _case(name, T, **kw)
    say("static entry", label, "T", T, "then", T2)
    for t in (T, T2):
        x = mi.make_x(w, 0, T=t, device=DEV)
        ref, ridx, rw = moe.layer_forward(x, lay["w_router"], lay["bias"], ex, w.k, w.act, flags, want_routing=True)
        got, gidx, gw = moe.layer_forward_static(x, lay["w_router"], lay["bias"], ex, w.k, w.act, flags,
                                                 want_routing=True)
        torch.cuda.synchronize()
        assert torch.equal(gidx, ridx)
        assert torch.equal(gw, rw)
        assert torch.equal(got, ref), f"T={t}: max diff {(got - ref).abs().max().item()}"
        assert torch.isfinite(got).all()
    say("  bitwise equal at both sizes")


def test_static_entry_matches_the_oracle():
    """The tiny layer as specified, through the static entry, against the CPU oracle."""
    w = mi.workload("tiny")
    lay = mi.make_layer(w, 0, DEV)
    x = mi.make_x(w, 0, device=DEV)
    out, idx, wts = moe.layer_forward_static(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act,
                                             want_routing=True)
    torch.cuda.synchronize()
    host = mi.to_host(lay)
    ref = oracle.layer_forward(x.cpu(), host["w_router"], host["bias"], host["experts"], w.k, w.act)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    o = out.cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(o - ref["out"]).max(1) / np.abs(ref["out"]).max(1)))
    say("static entry vs oracle, rel err", err)
    assert err < 1e-4


def test_static_entry_rejects_sizes_beyond_its_buffer():
    """A call needing more than the static buffer returns MOE_ESCRATCH and writes nothing."""
    w = mi.workload("gemma_prefill", T=2048, fmt=mi.FMT_I8_ROW)
    assert moe.workspace_bytes(w.T, w.k, {"fmt": w.fmt, "E": w.E, "d_model": w.d_model, "d_ff": w.d_ff},
                               w.act, moe.F_PREFILL_I8) > moe.STATIC_WORKSPACE_BYTES
    small = mi.workload("tiny", E=8, d_model=2816, d_ff=704, fmt=mi.FMT_I8_ROW, k=8, T=2048)
    lay = mi.make_layer(small, 0, DEV)
    x = mi.make_x(small, 0, device=DEV)
    out = torch.full((small.T, small.d_model), 7.0, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_forward_static(x, lay["w_router"], lay["bias"], lay["experts"], small.k, small.act,
                                 moe.F_PREFILL_I8, out=out)
    assert e.value.status == moe.ESCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
