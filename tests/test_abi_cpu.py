"""The C ABI without a GPU: the library loads, exports what include/moe.h declares, sizes its
workspace, and rejects bad arguments before launching anything (every call here fails a check,
so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

import sparse_moe_expert_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced by these calls


def declared_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = moe.lib()
    names = declared_functions()
    assert set(names) == set(moe.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = moe.lib()
    assert L.moe_abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert L.moe_status_str(st).startswith(b"MOE_")
    assert b"unknown" in L.moe_status_str(7)


def ex(fmt=0, E=8, d=256, dff=512, ptr=FAKE, S=0):
    return moe.Experts(fmt, E, d, dff, ptr, ptr, ptr, ptr, S)


def test_workspace_bytes():
    L = moe.lib()
    s = ex()
    a = L.moe_workspace_bytes(4, 2, ctypes.byref(s), 0, 0)
    b = L.moe_workspace_bytes(8, 2, ctypes.byref(s), 0, 0)
    assert 0 < a < b
    # h alone needs P * d_ff floats
    assert a >= 4 * 2 * 512 * 4
    assert L.moe_workspace_bytes(4, 9, ctypes.byref(s), 0, 0) == 0          # k > E
    assert L.moe_workspace_bytes(0, 2, ctypes.byref(s), 0, 0) == 0          # T < 1
    assert L.moe_workspace_bytes(4, 2, None, 0, 0) == 0
    bad = ex(d=200)
    assert L.moe_workspace_bytes(4, 2, ctypes.byref(bad), 0, 0) == 0
    s1 = ex(S=1)                                       # a shared expert adds T rows of h and y
    assert L.moe_workspace_bytes(4, 2, ctypes.byref(s1), 0, 0) >= a + 4 * (512 + 256) * 4
    e2 = ex(fmt=2, E=512, d=1024, dff=2688)
    assert L.moe_workspace_bytes(1, 22, ctypes.byref(e2), 1, 1) > 22 * 2688 * 4
    assert L.moe_route_workspace_bytes(4, 8) >= 4 * 8 * 8


def fwd(L, *, x=FAKE, xt=1, T=4, wr=FAKE, bias=None, s=None, k=2, act=0, flags=0, out=FAKE,
        ws=FAKE, ws_bytes=1 << 40):
    s = ex() if s is None else s
    return L.moe_layer_forward(x, xt, T, wr, bias, ctypes.byref(s), k, act, flags, out, None, None,
                               ws, ws_bytes, None)


def test_layer_forward_argument_checks():
    L = moe.lib()
    assert fwd(L, k=9) == moe.EINVAL                      # k > E
    assert fwd(L, k=0) == moe.EINVAL
    assert fwd(L, T=0) == moe.EINVAL
    assert fwd(L, T=40000) == moe.EINVAL
    assert fwd(L, xt=3) == moe.EINVAL
    assert fwd(L, x=FAKE + 4) == moe.EINVAL               # misaligned
    assert fwd(L, x=None) == moe.EINVAL
    assert fwd(L, out=None) == moe.EINVAL
    assert fwd(L, bias=FAKE + 8) == moe.EINVAL
    assert fwd(L, act=5) == moe.EINVAL
    assert fwd(L, flags=2) == moe.EINVAL                  # unknown flag bit
    assert fwd(L, s=ex(fmt=7)) == moe.EINVAL
    assert fwd(L, s=ex(fmt=-1)) == moe.EINVAL
    assert fwd(L, s=ex(E=513), k=2) == moe.EINVAL
    assert fwd(L, s=ex(d=96)) == moe.EINVAL               # d_model not a multiple of 64
    assert fwd(L, s=ex(dff=48)) == moe.EINVAL             # d_ff not a multiple of 32
    assert fwd(L, s=ex(dff=96)) == moe.EINVAL             # int8 formats need d_ff % 64 == 0
    assert fwd(L, s=ex(fmt=5, dff=96), flags=moe.F_PREFILL_FP8) == moe.EINVAL   # fp8 too
    assert fwd(L, s=ex(fmt=3, dff=96)) == moe.EINVAL
    assert fwd(L, s=ex(fmt=3), ws_bytes=1024) == moe.EWORKSPACE       # tiled format accepted
    assert fwd(L, s=ex(ptr=FAKE + 2)) == moe.EINVAL
    assert fwd(L, flags=moe.F_ZERO_SKIP) == moe.EUNSUPPORTED          # zero-skip needs E2M1
    assert fwd(L, flags=moe.F_PREFILL_I8, s=ex(fmt=2)) == moe.EUNSUPPORTED   # prefill: int8 weights
    assert fwd(L, flags=moe.F_PREFILL_I8, s=ex(fmt=1), act=1) == moe.EUNSUPPORTED   # and SwiGLU
    assert fwd(L, flags=moe.F_PREFILL_I8, ws_bytes=1024) == moe.EWORKSPACE  # Q8_0 prefill accepted
    assert fwd(L, s=ex(fmt=2, d=4096, dff=64), ws_bytes=1024) == moe.EWORKSPACE   # wide E2M1 rows
    assert fwd(L, s=ex(fmt=5)) == moe.EUNSUPPORTED                    # E4M3 experts: fp8 prefill only
    assert fwd(L, s=ex(fmt=6)) == moe.EUNSUPPORTED
    assert fwd(L, s=ex(fmt=5), flags=moe.F_PREFILL_I8) == moe.EUNSUPPORTED
    assert fwd(L, s=ex(fmt=1), flags=moe.F_PREFILL_FP8) == moe.EUNSUPPORTED   # and it on them only
    assert fwd(L, s=ex(fmt=5), flags=moe.F_PREFILL_FP8, act=1) == moe.EUNSUPPORTED   # SwiGLU
    assert fwd(L, s=ex(fmt=5), flags=moe.F_PREFILL_FP8 | moe.F_PREFILL_I8) == moe.EINVAL
    assert fwd(L, s=ex(fmt=5), flags=moe.F_PREFILL_FP8, ws_bytes=1024) == moe.EWORKSPACE
    assert fwd(L, s=ex(fmt=6, S=2), flags=moe.F_PREFILL_FP8, ws_bytes=1024) == moe.EWORKSPACE
    assert fwd(L, ws_bytes=1024) == moe.EWORKSPACE
    assert fwd(L, s=ex(S=5)) == moe.EINVAL                # at most 4 shared experts
    assert fwd(L, s=ex(S=-1)) == moe.EINVAL
    assert fwd(L, s=ex(S=1), ws_bytes=1024) == moe.EWORKSPACE           # one shared expert accepted


def test_other_entry_points_argument_checks():
    L = moe.lib()
    s = ex()
    assert L.moe_experts_forward(FAKE, 1, 4, FAKE, FAKE, ctypes.byref(s), 9, 0, 0, FAKE, FAKE,
                                 1 << 40, None) == moe.EINVAL
    assert L.moe_experts_forward(FAKE, 1, 4, FAKE + 4, FAKE, ctypes.byref(s), 2, 0, 0, FAKE, FAKE,
                                 1 << 40, None) == moe.EINVAL
    assert L.moe_experts_forward(FAKE, 1, 4, FAKE, FAKE, ctypes.byref(s), 2, 0, 0, FAKE, FAKE,
                                 16, None) == moe.EWORKSPACE
    assert L.moe_route(FAKE, 1, 4, 256, FAKE, None, 8, 9, FAKE, FAKE, FAKE, 1 << 30, None) == moe.EINVAL
    assert L.moe_route(FAKE, 1, 4, 250, FAKE, None, 8, 2, FAKE, FAKE, FAKE, 1 << 30, None) == moe.EINVAL
    assert L.moe_route(FAKE, 1, 4, 256, FAKE, None, 8, 2, FAKE, FAKE, FAKE, 8, None) == moe.EWORKSPACE
    assert L.moe_permute(FAKE, 4, 2, 513, FAKE, FAKE, FAKE, FAKE, None) == moe.EINVAL
    assert L.moe_permute(FAKE, 4, 2, 8, FAKE, FAKE + 1, FAKE, FAKE, None) == moe.EINVAL
    assert L.moe_quantize_rows_i8(FAKE, 1, 4, 100, FAKE, FAKE, None) == moe.EINVAL
    assert L.moe_quantize_rows_i8(FAKE, 1, 0, 128, FAKE, FAKE, None) == moe.EINVAL
    assert L.moe_quantize_rows_fp8(FAKE, 1, 4, 100, FAKE, FAKE, None) == moe.EINVAL
    assert L.moe_quantize_rows_fp8(FAKE, 2, 4, 128, FAKE, FAKE, None) == moe.EINVAL
    assert L.moe_quantize_rows_fp8(FAKE, 0, 4, 128, FAKE, FAKE + 4, None) == moe.EINVAL


def test_read_intermediates_argument_checks():
    L = moe.lib()
    s = ex()
    def rd(T=4, k=2, s=s, act=0, flags=0, ws=FAKE, ws_bytes=1 << 40, h=FAKE, hq=None, sh=None):
        return L.moe_read_intermediates(T, k, ctypes.byref(s), act, flags, 1, ws, ws_bytes, h, hq, sh, None)
    assert rd(k=9) == moe.EINVAL                          # k > E
    assert rd(h=None) == moe.EINVAL
    assert rd(h=FAKE + 4) == moe.EINVAL
    assert rd(ws=None) == moe.EINVAL
    assert rd(hq=FAKE, sh=FAKE) == moe.EINVAL             # codes only on the prefill paths
    assert rd(flags=moe.F_PREFILL_I8) == moe.EINVAL       # and there both are required
    assert rd(flags=moe.F_PREFILL_I8, hq=FAKE, sh=FAKE + 2) == moe.EINVAL
    assert rd(ws_bytes=1024) == moe.EWORKSPACE
    assert rd(flags=moe.F_PREFILL_I8, hq=FAKE, sh=FAKE, ws_bytes=1024) == moe.EWORKSPACE
    assert rd(s=ex(fmt=2), flags=moe.F_ZERO_SKIP, act=1, ws_bytes=1024) == moe.EWORKSPACE


def test_static_entry_argument_checks():
    """moe_layer_forward_static checks its arguments like moe_layer_forward and rejects a call
    whose workspace exceeds its static buffer before touching the device."""
    L = moe.lib()
    def st(T=4, k=2, s=None, act=0, flags=0, x=FAKE, out=FAKE):
        s = ex() if s is None else s
        return L.moe_layer_forward_static(x, 1, T, FAKE, None, ctypes.byref(s), k, act, flags, out, None, None, None)
    assert st(k=9) == moe.EINVAL
    assert st(T=0) == moe.EINVAL
    assert st(x=None) == moe.EINVAL
    assert st(out=FAKE + 4) == moe.EINVAL
    assert st(flags=moe.F_ZERO_SKIP) == moe.EUNSUPPORTED
    big = ex(fmt=1, E=128, d=2816, dff=704)                # the Gemma-shaped prefill at T = 2048
    need = L.moe_workspace_bytes(2048, 8, ctypes.byref(big), 0, moe.F_PREFILL_I8)
    assert need > moe.STATIC_WORKSPACE_BYTES
    assert st(T=2048, k=8, s=big, flags=moe.F_PREFILL_I8) == moe.ESCRATCH
    for T, k, e in ((64, 8, ex(fmt=3, E=128, d=2816, dff=704)), (64, 4, ex(fmt=0, E=128, d=6144, dff=3072)),
                    (1, 22, ex(fmt=2, E=512, d=1024, dff=2688))):
        assert 0 < L.moe_workspace_bytes(T, k, ctypes.byref(e), 0, 0) <= moe.STATIC_WORKSPACE_BYTES


def test_repack_argument_checks():
    L = moe.lib()
    src, dst = ex(fmt=0), ex(fmt=3, ptr=FAKE * 2)
    assert L.moe_repack_experts(ctypes.byref(src), 0, ctypes.byref(ex(fmt=4, ptr=FAKE * 2)), None) == moe.EINVAL
    assert L.moe_repack_experts(ctypes.byref(ex(fmt=2)), 0, ctypes.byref(dst), None) == moe.EINVAL
    assert L.moe_repack_experts(ctypes.byref(src), 0, ctypes.byref(ex(fmt=3)), None) == moe.EINVAL  # in place
    assert L.moe_repack_experts(ctypes.byref(src), 0, ctypes.byref(ex(fmt=3, E=4, ptr=FAKE * 2)), None) == moe.EINVAL
    assert L.moe_repack_experts(None, 0, ctypes.byref(dst), None) == moe.EINVAL
    f8 = ex(fmt=5)
    assert L.moe_repack_experts(ctypes.byref(f8), 0, ctypes.byref(ex(fmt=4, ptr=FAKE * 2)), None) == moe.EINVAL
    assert L.moe_repack_experts(ctypes.byref(f8), 1, ctypes.byref(ex(fmt=6, ptr=FAKE * 2)), None) == moe.EINVAL


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(ImportError):
        moe.lib()
