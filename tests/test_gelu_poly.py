"""The encoders' GELU polynomial (the constants compiled into csrc/encode_core.h), checked
in the kernel's own fp32 arithmetic against GELU from the normal CDF in float64."""
import numpy as np
from scipy.special import ndtr

from hash_top_kv_amd import gelu_fit


def test_constants_meet_the_stated_bound():
    # |GELU_kernel(a) - a Phi(a)| <= 4.6e-7 beyond the fp32 rounding of the result
    assert gelu_fit.check() <= 4.6e-7


def test_special_values():
    c = gelu_fit.constants()
    a = np.array([0.0, -0.0, 1e-30, -1e-30, 15.0, -15.0, 1e6, -1e6, 3e38, -3e38])
    g = gelu_fit.gelu_kernel(a, c)
    assert not np.isnan(g).any()
    assert g[0] == 0.0 and g[1] == 0.0
    # large |a|: max(a, 0) exactly (the exponential has underflowed to zero)
    assert np.array_equal(g[4::2], a.astype(np.float32)[4::2]) and np.all(g[5::2] == 0.0)
    # GELU(-1) = -Phi(-1), GELU(1) = Phi(1)
    assert abs(gelu_fit.gelu_kernel(np.array([-1.0]), c)[0] + ndtr(-1.0)) < 5e-7
    assert abs(gelu_fit.gelu_kernel(np.array([1.0]), c)[0] - ndtr(1.0)) < 5e-7


def test_polynomial_falls_without_bound():
    # R's leading coefficient is negative and R < -140 from x = 12 on: 2^R is zero there
    c = gelu_fit.constants().astype(np.float64)
    assert c[-1] < 0
    x = np.geomspace(12.0, 1e6, 10000)
    assert np.all(np.polyval(c[::-1], x) < -140)
