"""Numerics of the two gfx950 matrix-core instructions the E4M3 (fp8) prefill could use, measured
directly (tests/probes/mfma_sum_probe.hip): every output of one MFMA is the sum 256 + a, exact in
fp32.  The f16 instruction returns it exactly; the E4M3 instruction keeps 256 + 2^-5 but drops a
2^-6 addend next to 256 in the same 8-code group of a lane.  That truncation, which the products of
a real row carry too, is why the E4M3 grouped GEMM widens its codes to f16 (exact) and runs on the
f16 matrix cores instead."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libmfma_probe.so")
E4M3 = {2.0 ** -2: 0x28, 2.0 ** -5: 0x10, 2.0 ** -6: 0x08}     # sign 0, exponent bias 7, mantissa 0


def probe(kind, a):
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    out = np.zeros(1024, np.float32)
    rc = lib.mfma_sum_probe(kind, E4M3.get(a, 0), ctypes.c_float(a),
                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    assert rc == 0, f"HIP error {rc}"
    assert np.all(out == out[0]), "every output is the same row sum"
    return float(out[0])


@pytest.mark.parametrize("a", [2.0 ** -2, 2.0 ** -6, 2.0 ** -9])
def test_f16_matrix_core_sum_is_exact(a):
    import torch  # noqa: F401  (initialises the device the way the other tests do)
    assert probe(1, a) == 256.0 + a


def test_e4m3_matrix_core_truncates_small_addends():
    import torch  # noqa: F401
    assert probe(0, 2.0 ** -2) == 256.25                 # the probe is wired right
    assert probe(0, 2.0 ** -5) == 256.0 + 2.0 ** -5
    assert probe(0, 2.0 ** -6) != 256.0 + 2.0 ** -6      # exact in fp32, lost by the instruction
