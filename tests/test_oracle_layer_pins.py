"""Pins of the whole-layer oracle (CPU): properties the layer's definition fixes, each chosen so that a
plausible mistake (a dropped residual, the norm after in_proj or missing, x and z swapped, the norm weight
added instead of multiplied, out_proj scaling the residual) fails at least one of them.

The layer: out = x_res + out_proj(mixer(in_proj(rms_norm(x_res)))) with in_proj's rows ordered x | z
(the neurarch "Jamba" page's Structure table and Exported PyTorch listing; llm-architectures-explained,
"Jamba v0.1", Facts; TransformerLens Jamba architecture overview).
"""

import math

import numpy as np
import pytest

import oracle


def _problem(seed=0, B=2, L=9, C=6, N=4, R=3, K=4, Dm=5, conv_b_zero=False):
    rng = np.random.default_rng(seed)
    w = {
        "conv_w": rng.uniform(-0.5, 0.5, (C, K)),
        "conv_b": np.zeros(C) if conv_b_zero else rng.normal(0, 0.1, C),
        "x_proj_w": rng.normal(0, 1 / math.sqrt(C), (R + 2 * N, C)),
        "dt_norm_w": rng.uniform(0.5, 1.5, R),
        "b_norm_w": rng.uniform(0.5, 1.5, N),
        "c_norm_w": rng.uniform(0.5, 1.5, N),
        "dt_proj_w": rng.normal(0, 1 / math.sqrt(R), (C, R)),
        "dt_proj_b": np.log(np.expm1(rng.uniform(1e-3, 0.1, C))),
        "A_log": np.log(rng.uniform(0.5, 8.0, (C, N))),
        "D": rng.normal(1.0, 0.3, C),
    }
    lw = {
        "norm_w": rng.uniform(0.5, 1.5, Dm),
        "in_proj_w": rng.normal(0, 1 / math.sqrt(Dm), (2 * C, Dm)),
        "out_proj_w": rng.normal(0, 1 / math.sqrt(C), (Dm, C)),
    }
    x_res = rng.normal(0, 1, (B, L, Dm))
    cs = rng.normal(0, 1, (B, C, K - 1))
    h0 = rng.normal(0, 0.3, (B, C, N))
    return x_res, lw, w, cs, h0, R, N


def test_zero_norm_weight_passes_the_residual_through():
    # rms_norm(x) * 0 = 0, so x = z = 0; with no conv state and no conv bias xc = SiLU(0) = 0, B = C = 0,
    # and out = x_res + out_proj(0 * SiLU(0)) = x_res exactly, while the state decays as
    # exp(A * L * softplus(b_dt)) (the bias alone sets dt)
    x_res, lw, w, cs, h0, R, N = _problem(1, conv_b_zero=True)
    lw = dict(lw, norm_w=np.zeros_like(lw["norm_w"]))
    out, conv, h = oracle.layer_prefill(x_res, lw, w, R, N, ssm_state=h0)
    assert np.array_equal(out, x_res)
    L = x_res.shape[1]
    dt = np.log1p(np.exp(w["dt_proj_b"]))
    A = -np.exp(w["A_log"])
    np.testing.assert_allclose(h, np.exp(A[None] * L * dt[None, :, None]) * h0, rtol=1e-12, atol=0)
    assert np.array_equal(conv, np.zeros_like(conv))


def test_layer_increment_is_invariant_to_scaling_the_residual():
    # with eps = 0 the pre-norm removes any positive scale of its input, so out - x_res is unchanged when
    # x_res is scaled: fails if the norm is missing or sits after in_proj
    x_res, lw, w, cs, h0, R, N = _problem(2)
    a, _, _ = oracle.layer_prefill(x_res, lw, w, R, N, layer_eps=0.0, conv_state=cs, ssm_state=h0)
    b, _, _ = oracle.layer_prefill(3.7 * x_res, lw, w, R, N, layer_eps=0.0, conv_state=cs, ssm_state=h0)
    np.testing.assert_allclose(b - 3.7 * x_res, a - x_res, rtol=1e-11, atol=1e-12)


def test_out_proj_scales_only_the_increment():
    # doubling out_proj doubles out - x_res: the residual is added after out_proj, unscaled
    x_res, lw, w, cs, h0, R, N = _problem(3)
    a, _, _ = oracle.layer_prefill(x_res, lw, w, R, N, conv_state=cs, ssm_state=h0)
    b, _, _ = oracle.layer_prefill(x_res, dict(lw, out_proj_w=2 * lw["out_proj_w"]), w, R, N, conv_state=cs,
                                   ssm_state=h0)
    np.testing.assert_allclose(b - x_res, 2 * (a - x_res), rtol=1e-12, atol=1e-14)


def test_norm_weight_multiplies_the_normalised_input():
    # rms_norm(x) * (2 w) then in_proj equals rms_norm(x) * w then in_proj with doubled rows
    x_res, lw, w, cs, h0, R, N = _problem(4)
    a, _, _ = oracle.layer_prefill(x_res, dict(lw, norm_w=2 * lw["norm_w"]), w, R, N, conv_state=cs, ssm_state=h0)
    b, _, _ = oracle.layer_prefill(x_res, dict(lw, in_proj_w=2 * lw["in_proj_w"]), w, R, N, conv_state=cs,
                                   ssm_state=h0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_in_proj_rows_are_x_then_z():
    # the second half of in_proj feeds the gate: zeroing it makes z = 0 and SiLU(0) = 0, so out = x_res
    # exactly whatever the scan does; zeroing the first half instead leaves a non-zero increment
    x_res, lw, w, cs, h0, R, N = _problem(5)
    C = w["D"].shape[0]
    wz0 = lw["in_proj_w"].copy()
    wz0[C:] = 0.0
    out, _, _ = oracle.layer_prefill(x_res, dict(lw, in_proj_w=wz0), w, R, N, conv_state=cs, ssm_state=h0)
    assert np.array_equal(out, x_res)
    wx0 = lw["in_proj_w"].copy()
    wx0[:C] = 0.0
    out, _, _ = oracle.layer_prefill(x_res, dict(lw, in_proj_w=wx0), w, R, N, conv_state=cs, ssm_state=h0)
    assert np.abs(out - x_res).max() > 1e-3


@pytest.mark.parametrize("seed", [6, 7])
def test_layer_prefill_equals_decode_steps(seed):
    x_res, lw, w, cs, h0, R, N = _problem(seed)
    out, conv, h = oracle.layer_prefill(x_res, lw, w, R, N, conv_state=cs, ssm_state=h0)
    c, hh = cs, h0
    for t in range(x_res.shape[1]):
        o, c, hh = oracle.layer_decode_step(x_res[:, t], lw, w, R, N, c, hh)
        np.testing.assert_allclose(o, out[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hh, h, rtol=1e-12, atol=1e-14)
    # the conv state holds in_proj outputs, which the matmul of a whole sequence and of one token may round
    # differently in the last bit
    np.testing.assert_allclose(c, conv, rtol=1e-13, atol=1e-14)
