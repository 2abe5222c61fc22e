"""Pins for the oracle's GeLU and its derivative.

Textbook values of the standard normal CDF, the odd-part identity
g(z) - g(-z) = z (from Phi(z) + Phi(-z) = 1), the limits, and the derivative
against central differences of g.
"""
import numpy as np

from oracle import stage as ost


def test_gelu_textbook_values():
    # Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208 (standard normal table)
    assert abs(ost.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(ost.gelu(-1.0) + (1 - 0.8413447460685429)) < 1e-15
    assert abs(ost.gelu(2.0) - 2 * 0.9772498680518208) < 1e-14
    assert ost.gelu(0.0) == 0.0


def test_gelu_odd_part_identity_and_limits():
    z = np.linspace(-9, 9, 181)
    assert np.allclose(ost.gelu(z) - ost.gelu(-z), z, rtol=0, atol=1e-14)
    assert abs(ost.gelu(12.0) - 12.0) < 1e-12
    assert abs(ost.gelu(-12.0)) < 1e-12


def test_gelu_grad_central_differences():
    z = np.linspace(-6, 6, 241)
    eps = 1e-6
    num = (ost.gelu(z + eps) - ost.gelu(z - eps)) / (2 * eps)
    assert np.max(np.abs(num - ost.gelu_grad(z))) < 1e-8
    assert ost.gelu_grad(0.0) == 0.5


# The tanh approximation (Hendrycks & Gimpel, "Gaussian Error Linear Units
# (GELUs)", section 2), used by no workload but offered by the kernels.

def test_gelu_tanh_stays_within_the_approximation_band_of_exact_gelu():
    """Against exact GeLU written with math.erf (independent of the oracle): the
    approximation is off by at most 4.73e-4 (near z = -2.70).  A dropped cubic
    term (3.4e-2) or a mistyped 0.044715 (e.g. 0.04715: 1.5e-3) leaves the band."""
    import math
    z = np.linspace(-10, 10, 40001)
    exact = np.array([0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in z])
    dev = np.abs(ost.gelu(z, "tanh") - exact)
    assert dev.max() < 5e-4
    assert dev.max() > 4e-4  # an approximation, not the exact form
    assert abs(z[np.argmax(dev)] + 2.70) < 0.05


def test_gelu_tanh_odd_part_identity_limits_and_origin():
    # tanh is odd, so g(z) - g(-z) = z exactly as for the exact form
    z = np.linspace(-9, 9, 181)
    assert np.allclose(ost.gelu(z, "tanh") - ost.gelu(-z, "tanh"), z, rtol=0, atol=1e-14)
    assert abs(ost.gelu(12.0, "tanh") - 12.0) < 1e-12
    assert abs(ost.gelu(-12.0, "tanh")) < 1e-12
    assert ost.gelu(0.0, "tanh") == 0.0
    assert ost.gelu_grad(0.0, "tanh") == 0.5


def test_gelu_tanh_grad_central_differences():
    z = np.linspace(-6, 6, 241)
    eps = 1e-6
    num = (ost.gelu(z + eps, "tanh") - ost.gelu(z - eps, "tanh")) / (2 * eps)
    assert np.max(np.abs(num - ost.gelu_grad(z, "tanh"))) < 1e-8


def test_gelu_rejects_unknown_forms():
    import pytest
    with pytest.raises(ValueError):
        ost.gelu(1.0, "sigmoid")
    with pytest.raises(ValueError):
        ost.gelu_grad(1.0, "sigmoid")
