"""The triplet encoder's arctangent polynomial (atan01 in tq_octo.hip) is the
one fit_atan.py produces, and its fp32 evaluation stays within 1.6e-7 rad of
arctan on [0, 1] (the equal-area map's azimuth feeds the cell choice, whose
ties the GPU parity tests allow within 1e-5 of a cell edge)."""

import os
import re

import numpy as np

from kv_cache_vector_encode_amd import fit_atan

SRC = os.path.join(os.path.dirname(fit_atan.__file__), "csrc", "tq_octo.hip")


def _kernel_coefficients():
    with open(SRC) as f:
        text = f.read()
    body = text[text.index("float atan01(float a)"):]
    body = body[:body.index("return a * p;")]
    vals = [float(v) for v in re.findall(r"(-?\d\.\d+e[-+]\d+)f", body)]
    assert len(vals) == fit_atan.DEGREE + 1
    return np.array(vals[::-1], dtype=np.float32)      # c_0 .. c_7


def test_kernel_coefficients_are_the_scripts_fit():
    c_kernel = _kernel_coefficients()
    c_fit = fit_atan.fit().astype(np.float32)
    assert np.array_equal(c_kernel, c_fit)


def test_fp32_evaluation_error_bound():
    c = _kernel_coefficients()
    err = fit_atan.max_error_fp32(c)
    assert err <= 1.6e-7, err
    # atan(0) = 0 and atan(1) = pi/4 to the bound; the slope at 0 is 1
    assert fit_atan.horner_fp32(c, np.array([0.0]))[0] == 0.0
    assert abs(float(fit_atan.horner_fp32(c, np.array([1.0]))[0]) - np.pi / 4) <= 1.6e-7
    assert abs(float(c[0]) - 1.0) < 1e-6
