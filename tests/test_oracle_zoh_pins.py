"""Pins of the exact zero-order-hold (ZOH) variant of the scan's input matrix (CPU).

The Jamba Guide's discretisation equation ("Inside the Mamba State-Space Layers: Mathematical Mechanics")
gives Bbar = (delta A)^-1 (exp(delta A) - I) delta B, with delta B as its approximation.  ZOH is exact for an
input held constant over the step, which fixes properties that neither a typo in the formula nor the Euler
form satisfies: two half steps equal one whole step, the state settles at the continuous system's steady
state -B x / A whatever delta is, and as |delta A| -> 0 the two forms agree.
"""

import numpy as np
import pytest

import oracle


def _scan(xc, delta, A_log, Bn, Cn, D, h0, zoh):
    return oracle.selective_scan(xc, delta, A_log, Bn, Cn, D, h0, zoh=zoh)


def _const_problem(seed, L, C=3, N=4, delta=0.3):
    rng = np.random.default_rng(seed)
    A_log = np.log(rng.uniform(0.5, 4.0, (C, N)))
    x = np.broadcast_to(rng.normal(0, 1, (1, 1, C)), (1, L, C)).copy()
    Bv = np.broadcast_to(rng.normal(0, 1, (1, 1, N)), (1, L, N)).copy()
    Cv = rng.normal(0, 1, (1, L, N))
    h0 = rng.normal(0, 1, (1, C, N))
    return x, np.full((1, L, C), delta), A_log, Bv, Cv, np.zeros(C), h0


def test_two_half_steps_equal_one_step():
    # constant input over the interval: ZOH is the exact flow of h' = A h + B x, so it composes
    x, d, A_log, Bv, Cv, D, h0 = _const_problem(1, 2)
    _, h_half = _scan(x, d / 2, A_log, Bv, Cv, D, h0, zoh=True)             # two steps of delta / 2
    _, h_one = _scan(x[:, :1], d[:, :1], A_log, Bv[:, :1], Cv[:, :1], D, h0, zoh=True)
    np.testing.assert_allclose(h_half, h_one, rtol=1e-13, atol=1e-14)
    # the Euler form does not compose
    _, e_half = _scan(x, d / 2, A_log, Bv, Cv, D, h0, zoh=False)
    _, e_one = _scan(x[:, :1], d[:, :1], A_log, Bv[:, :1], Cv[:, :1], D, h0, zoh=False)
    assert np.abs(e_half - e_one).max() > 1e-3


@pytest.mark.parametrize("delta", [0.05, 0.7])
def test_steady_state_is_the_continuous_one(delta):
    # with x and B held, h_t -> Bbar x / (1 - exp(delta A)) = -B x / A for ZOH, independent of delta
    x, d, A_log, Bv, Cv, D, h0 = _const_problem(2, 4000, delta=delta)
    _, h = _scan(x, d, A_log, Bv, Cv, D, h0, zoh=True)
    A = -np.exp(A_log)
    expect = -Bv[0, 0][None, None, :] * x[0, 0][None, :, None] / A[None]
    np.testing.assert_allclose(h, expect, rtol=1e-10, atol=1e-12)


def test_small_steps_agree_with_the_euler_form():
    rng = np.random.default_rng(3)
    B, L, C, N = 2, 9, 4, 4
    xc = rng.normal(0, 1, (B, L, C))
    delta = rng.uniform(1e-9, 2e-9, (B, L, C))
    A_log = np.log(rng.uniform(0.5, 8.0, (C, N)))
    Bn, Cn = rng.normal(0, 1, (B, L, N)), rng.normal(0, 1, (B, L, N))
    D = rng.normal(1, 0.2, C)
    h0 = rng.normal(0, 1, (B, C, N))
    yz, hz = _scan(xc, delta, A_log, Bn, Cn, D, h0, zoh=True)
    ye, he = _scan(xc, delta, A_log, Bn, Cn, D, h0, zoh=False)
    np.testing.assert_allclose(yz, ye, rtol=1e-8, atol=1e-14)
    np.testing.assert_allclose(hz, he, rtol=1e-8, atol=1e-14)


def test_zoh_input_term_in_closed_form():
    # one step from h0 = 0: h = (exp(delta A) - 1) / A * B * x exactly
    rng = np.random.default_rng(4)
    C, N = 3, 4
    xc = rng.normal(0, 1, (1, 1, C))
    delta = rng.uniform(0.01, 1.0, (1, 1, C))
    A_log = np.log(rng.uniform(0.5, 8.0, (C, N)))
    Bn = rng.normal(0, 1, (1, 1, N))
    _, h = _scan(xc, delta, A_log, Bn, np.zeros((1, 1, N)), np.zeros(C), None, zoh=True)
    A = -np.exp(A_log)
    expect = (np.exp(delta[0, 0][:, None] * A) - 1.0) / A * Bn[0, 0][None, :] * xc[0, 0][:, None]
    np.testing.assert_allclose(h[0], expect, rtol=1e-13, atol=1e-15)


def test_zero_A_takes_the_limit_delta_B():
    # A = 0 (A_log = -inf): (exp(delta A) - 1) / A -> delta, so ZOH and the Euler form coincide exactly and
    # the state is h0 plus the cumulative sum of delta * B * x (no decay)
    rng = np.random.default_rng(5)
    B, L, C, N = 2, 11, 3, 4
    xc = rng.normal(0, 1, (B, L, C))
    delta = rng.uniform(0.01, 0.5, (B, L, C))
    A_log = np.log(rng.uniform(0.5, 4.0, (C, N)))
    A_log[1] = -np.inf                                   # channel 1 has A = 0 in every state
    Bn, Cn = rng.normal(0, 1, (B, L, N)), rng.normal(0, 1, (B, L, N))
    D = rng.normal(1, 0.2, C)
    h0 = rng.normal(0, 1, (B, C, N))
    yz, hz = _scan(xc, delta, A_log, Bn, Cn, D, h0, zoh=True)
    ye, he = _scan(xc, delta, A_log, Bn, Cn, D, h0, zoh=False)
    assert np.isfinite(yz).all() and np.isfinite(hz).all()
    # equal up to the order of the products (dt * B) * x against (dt * x) * B
    np.testing.assert_allclose(hz[:, 1], he[:, 1], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(yz[:, :, 1], ye[:, :, 1], rtol=1e-14, atol=1e-15)
    cum = h0[:, 1][:, None] + np.cumsum((delta[:, :, 1] * xc[:, :, 1])[..., None] * Bn, axis=1)
    np.testing.assert_allclose(hz[:, 1], cum[:, -1], rtol=1e-12, atol=1e-12)
    # the other channels are the plain ZOH
    _, h_rest = _scan(xc[..., [0, 2]], delta[..., [0, 2]], A_log[[0, 2]], Bn, Cn, D[[0, 2]], h0[:, [0, 2]], zoh=True)
    np.testing.assert_array_equal(hz[:, [0, 2]], h_rest)
