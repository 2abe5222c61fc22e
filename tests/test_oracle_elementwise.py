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
