"""Constants typed into the HIP kernels, checked on the host against what they claim.

The nonlinear-refinement kernels evaluate the standard normal CDF with the erfc
approximation of Abramowitz and Stegun, formula 7.1.26 (absolute error below 1.5e-7 on
erf, so below 7.5e-8 on Phi = erfc / 2).  The coefficients are read out of the kernel
source and the formula is evaluated in float64 against scipy's normal CDF, so a mistyped
constant fails here on the CPU.
"""
import os
import re

import numpy as np
from scipy.special import ndtr

SRC = os.path.join(os.path.dirname(__file__), "..", "delta_rule_sequence_amd", "csrc", "prism_nl.h")


def _cdf_constants():
    text = open(SRC).read()
    body = text[text.index("float std_normal_cdf(float z)"):]
    body = body[:body.index("\n}\n")]
    p = float(re.search(r"1\.f \+ ([0-9.]+)f \* x", body).group(1))
    poly = re.search(r"t \* \((.*)\)\)\)\);", body.replace("\n", " ")).group(1)
    coef = [float(c) for c in re.findall(r"(-?[0-9]+\.[0-9]+)f", poly)]
    scale = float(re.search(r"fabsf\(z\) \* ([0-9.]+)f", body).group(1))
    return p, coef, scale


def test_cdf_coefficients_meet_the_published_bound():
    p, coef, scale = _cdf_constants()
    assert len(coef) == 5
    assert abs(scale - 1 / np.sqrt(2)) < 1e-15
    z = np.linspace(-9, 9, 200001)
    x = np.abs(z) * scale
    t = 1.0 / (1.0 + p * x)
    poly = t * (coef[0] + t * (coef[1] + t * (coef[2] + t * (coef[3] + t * coef[4]))))
    half_erfc = 0.5 * poly * np.exp(-x * x)
    phi = np.where(z >= 0, 1.0 - half_erfc, half_erfc)
    err = np.max(np.abs(phi - ndtr(z)))
    assert err < 7.5e-8, err
    # the approximation is not a no-op: perturbing any coefficient breaks the bound
    for i in range(5):
        c = list(coef)
        c[i] *= 1.001
        poly = t * (c[0] + t * (c[1] + t * (c[2] + t * (c[3] + t * c[4]))))
        phi = np.where(z >= 0, 1.0 - 0.5 * poly * np.exp(-x * x), 0.5 * poly * np.exp(-x * x))
        assert np.max(np.abs(phi - ndtr(z))) > 7.5e-8
