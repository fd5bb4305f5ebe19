"""Accuracy of the TTT-MLP kernels' polynomial normal CDF (phi_poly in
csrc/gelu.h), read from the kernel source and evaluated in float32 the way
the kernel does (Horner with fused multiply-adds), against scipy's exact CDF.
The kernel takes this path only while every |x| in the wave is below sqrt 2;
elsewhere it uses the library erff."""
import os
import re

import numpy as np
import pytest

scipy_special = pytest.importorskip("scipy.special")

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "test_sequence_layer_amd", "csrc", "gelu.h")


def _coefficients():
    src = open(SRC).read()
    body = src[src.index("float phi_poly("):]
    body = body[:body.index("return")]
    return [float.fromhex(h) for h in re.findall(r"(-?0x[0-9a-fA-F.]+p-?\d+)f", body)]


def _fma32(a, b, c):
    # a*b + c rounded once to float32 (the product and sum exact in float64 for float32 inputs)
    return (a.astype(np.float64) * b + c).astype(np.float32)


def test_phi_poly_accuracy():
    c = _coefficients()
    assert len(c) == 6
    x = np.linspace(-np.sqrt(2.0), np.sqrt(2.0), 200001).astype(np.float32)
    x = x[x * x < 2.0]
    u = (x * x).astype(np.float32)
    q = np.full_like(u, np.float32(c[0]))
    for k in c[1:]:
        q = _fma32(q, u, np.float32(k))
    cdf = _fma32(x, q, np.float32(0.5))
    exact = scipy_special.ndtr(x.astype(np.float64))
    assert np.abs(cdf - exact).max() <= 1e-7
    gelu, gelu_exact = x.astype(np.float64) * cdf, x.astype(np.float64) * exact
    nz = np.abs(x) > 1e-3
    assert (np.abs(gelu - gelu_exact)[nz] / np.abs(gelu_exact[nz])).max() <= 1e-6
