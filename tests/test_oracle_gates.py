"""Pins of the oracle's raw-gate evaluation (oracle/gates.py) against what
the mathematics fixes, independent of how the oracle writes it:
- with A_log = 0 and dt_bias = 0 the decay exp(-softplus(a)) is 1 / (1 + e^a),
  the logistic function of -a (scipy's expit);
- A_log = log 2 doubles the rate, so the decay is squared;
- dt_bias only shifts the input;
- beta is the logistic function (scipy's expit), odd about 1/2;
- extreme inputs give the limits 1 and 0 with no overflow; NaN rows stay NaN.
A dropped exp on A_log, a lost dt_bias, a sign error or softplus and the
logistic swapped fails at least one of these."""
import numpy as np
import pytest
from scipy.special import expit

from oracle.gates import gates_from_raw, sigmoid, softplus


def _params(Hv, A_log=0.0, dt_bias=0.0):
    return np.stack([np.full(Hv, A_log), np.full(Hv, dt_bias)])


def test_unit_rate_decay_is_the_logistic_of_minus_a():
    a = np.linspace(-30.0, 30.0, 241).reshape(-1, 1)
    alpha, _ = gates_from_raw(a, np.zeros_like(a), _params(1))
    np.testing.assert_allclose(alpha, 1.0 / (1.0 + np.exp(a)), rtol=1e-13, atol=0)
    np.testing.assert_allclose(alpha, expit(-a), rtol=1e-13, atol=0)


def test_rate_doubling_squares_the_decay():
    a = np.random.default_rng(3).standard_normal((50, 4)) * 3
    a0, _ = gates_from_raw(a, a, _params(4, A_log=0.0, dt_bias=-1.5))
    a2, _ = gates_from_raw(a, a, _params(4, A_log=np.log(2.0), dt_bias=-1.5))
    np.testing.assert_allclose(a2, a0 ** 2, rtol=1e-13)


def test_dt_bias_shifts_the_input():
    a = np.random.default_rng(4).standard_normal((30, 3))
    gp = np.stack([np.array([0.3, 1.1, 2.0]), np.array([-4.0, -2.5, 0.7])])
    shifted, _ = gates_from_raw(a + gp[1], a, np.stack([gp[0], np.zeros(3)]))
    direct, _ = gates_from_raw(a, a, gp)
    np.testing.assert_allclose(direct, shifted, rtol=1e-14)
    # per head: head h uses column h of the parameters
    for h in range(3):
        one, _ = gates_from_raw(a[:, h:h + 1], a[:, h:h + 1], gp[:, h:h + 1])
        np.testing.assert_allclose(direct[:, h:h + 1], one, rtol=0, atol=0)


def test_beta_is_the_logistic_function():
    b = np.linspace(-40.0, 40.0, 321).reshape(-1, 1)
    _, beta = gates_from_raw(np.zeros_like(b), b, _params(1))
    np.testing.assert_allclose(beta, expit(b), rtol=1e-14, atol=0)
    np.testing.assert_allclose(beta + beta[::-1], 1.0, rtol=1e-15)
    assert beta[160, 0] == 0.5


def test_limits_and_nan_rows():
    a = np.array([[-1000.0], [1000.0], [np.nan]])
    alpha, beta = gates_from_raw(a, a, _params(1, A_log=np.log(16.0), dt_bias=-7.0))
    assert alpha[0, 0] == 1.0 and beta[0, 0] == 0.0
    assert alpha[1, 0] == 0.0 and beta[1, 0] == 1.0
    assert np.isnan(alpha[2, 0]) and np.isnan(beta[2, 0])
    assert np.isfinite(softplus(np.array([1e308, -1e308]))).all()
    s = sigmoid(np.array([-700.0]))[0]  # e^-700: no overflow or cancellation on the negative side
    assert s > 0.0 and abs(s / np.exp(-700.0) - 1.0) < 1e-12


@pytest.mark.parametrize("A_log", [0.0, 1.0, 2.7])
def test_decay_is_monotone_and_in_the_unit_interval(A_log):
    a = np.linspace(-20.0, 20.0, 401).reshape(-1, 1)
    alpha, _ = gates_from_raw(a, a, _params(1, A_log=A_log, dt_bias=-3.0))
    assert ((alpha > 0) & (alpha <= 1)).all()
    assert (np.diff(alpha[:, 0]) <= 0).all()
