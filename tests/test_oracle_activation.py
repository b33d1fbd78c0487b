"""Pins of the GeLU oracle of the FP8-stored activation input against facts
that do not come from its own formula:

* Phi by numerical integration of the normal density (scipy quad), which also
  rejects the plausible slip erf(x) for erf(x / sqrt 2);
* the symmetry gelu(x) - gelu(-x) = x (Phi(x) + Phi(-x) = 1);
* textbook values: Phi(1.959963984540054) = 0.975, Phi(-10) = 7.619853024160527e-24,
  the minimum of gelu at x = -0.7517915 (gelu' = 0 there), about -0.16997;
* gelu' against central finite differences of gelu;
* the backward pass on hand-made FP8 bytes (E4M3 0x38 = 1.0 with scale_inv 2);
* the acceptance rule rejects a planted 1 % error.
"""

import numpy as np
from scipy import integrate
from scipy.special import erf

import oracle


def phi_density(t):
    return np.exp(-0.5 * t * t) / np.sqrt(2.0 * np.pi)


def test_gelu_against_integrated_normal_cdf():
    xs = [-6.0, -2.5, -1.0, -0.3, 0.0, 0.4, 1.0, 2.2, 5.0]
    for x in xs:
        cdf, _ = integrate.quad(phi_density, -np.inf, x, epsabs=1e-14, epsrel=1e-13)
        assert abs(oracle.gelu(x) - x * cdf) <= 1e-12 * max(1.0, abs(x * cdf)) + 1e-15
        slip = x * 0.5 * (1.0 + erf(x))  # erf without the 1/sqrt 2: a plausible mistake
        if x != 0.0:
            assert abs(slip - x * cdf) > 1e-8 * abs(x * cdf)  # far above the pin's 1e-12


def test_symmetry_and_textbook_values():
    x = np.linspace(-8, 8, 3201)
    assert np.max(np.abs(oracle.gelu(x) - oracle.gelu(-x) - x)) <= 1e-14 * 8
    assert abs(oracle.gelu(1.959963984540054) / 1.959963984540054 - 0.975) < 1e-15
    assert abs(oracle.gelu(-10.0) / -10.0 - 7.619853024160527e-24) < 1e-36
    assert abs(oracle.gelu_grad(-0.7517915)) < 1e-7
    assert abs(oracle.gelu(-0.7517915) - (-0.16997)) < 1e-5
    assert oracle.gelu_grad(0.0) == 0.5 and oracle.gelu(0.0) == 0.0


def test_gelu_grad_finite_differences():
    x = np.linspace(-7, 7, 1401)
    d = 1e-5
    fd = (oracle.gelu(x + d) - oracle.gelu(x - d)) / (2 * d)
    assert np.max(np.abs(fd - oracle.gelu_grad(x))) < 1e-9


def test_backward_on_hand_made_bytes():
    q = np.array([[0x38, 0xB8, 0x00]], dtype=np.uint8)  # E4M3: 1.0, -1.0, 0
    da = np.array([[1.0, 2.0, 3.0]], dtype=np.float32)
    dh = oracle.act_fp8_store_bwd(da, q, "e4m3", np.float32(2.0))  # h' = 2, -2, 0
    cdf2, pdf2 = 0.9772498680518208, 0.05399096651318806
    assert abs(dh[0, 0] - (cdf2 + 2 * pdf2)) < 1e-15
    assert abs(dh[0, 1] - 2.0 * ((1 - cdf2) - 2 * pdf2)) < 1e-15
    assert dh[0, 2] == 1.5


def test_forward_bytes_are_the_per_tensor_cast():
    g = np.random.Generator(np.random.PCG64(80))
    h = g.standard_normal((16, 40)).astype(np.float32)
    s = np.float32(448.0 / np.max(np.abs(h)))
    a, q = oracle.act_fp8_store_fwd(h, s, "e4m3")
    q2, _ = oracle.cast_transpose(h, s, "e4m3")
    assert np.array_equal(q, q2)
    assert np.array_equal(a, oracle.gelu(h.astype(np.float64)))


def test_acceptance_rule_rejects_a_planted_error():
    g = np.random.Generator(np.random.PCG64(81))
    h = g.standard_normal(1000)
    ref = oracle.gelu(h)
    assert oracle.elementwise_check(ref * (1 + 2.0 ** -10), ref)[0]
    assert not oracle.elementwise_check(ref * 1.01, ref)[0]
