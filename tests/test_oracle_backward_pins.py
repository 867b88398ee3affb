"""Pins of the scan-backward oracle (CPU).

The backward is pinned to the forward, not to itself: every gradient must match central finite differences
of the objective  sum(dout * out) + sum(dh_final * h_L)  computed with the forward alone
(oracle.scan_forward_gated, itself checked against the mixer oracle here).  A dropped term, a wrong sign, a
missing chain factor (dA/dA_log = A, SiLU') or an off-by-one in the reverse loop fails one of them.  Two
structural pins follow: channel subsets sum to the full dB / dC, and a backward split in time at any token
(state and gradient handed across) equals the whole one.
"""

import math

import numpy as np
import pytest

import oracle


def _problem(seed, B=2, L=7, C=3, N=4):
    rng = np.random.default_rng(seed)
    return {
        "xc": rng.normal(0, 1, (B, L, C)),
        "delta": rng.uniform(0.05, 0.6, (B, L, C)),
        "A_log": np.log(rng.uniform(0.5, 3.0, (C, N))),
        "Bn": rng.normal(0, 1, (B, L, N)),
        "Cn": rng.normal(0, 1, (B, L, N)),
        "D": rng.normal(1.0, 0.3, C),
        "z": rng.normal(0, 1.5, (B, L, C)),
        "h0": rng.normal(0, 0.5, (B, C, N)),
    }, rng.normal(0, 1, (B, L, C)), rng.normal(0, 1, (B, C, N))


def _objective(p, dout, dh_final):
    out, _, hL = oracle.scan_forward_gated(p["xc"], p["delta"], p["A_log"], p["Bn"], p["Cn"], p["D"], p["z"],
                                           p["h0"])
    return float(np.sum(dout * out) + np.sum(dh_final * hL))


GRAD_OF = {"xc": "dxc", "delta": "ddelta", "A_log": "dA_log", "Bn": "dB", "Cn": "dC", "D": "dD", "z": "dz",
           "h0": "dh0"}


def test_forward_matches_the_mixer_oracle_scan():
    p, _, _ = _problem(1)
    out, y, hL = oracle.scan_forward_gated(p["xc"], p["delta"], p["A_log"], p["Bn"], p["Cn"], p["D"], p["z"],
                                           p["h0"])
    y2, h2 = oracle.selective_scan(p["xc"], p["delta"], p["A_log"], p["Bn"], p["Cn"], p["D"], p["h0"])
    np.testing.assert_allclose(y, y2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(hL, h2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out, y2 * oracle.silu(p["z"]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("name", sorted(GRAD_OF))
@pytest.mark.parametrize("seed", [2, 3])
def test_gradients_match_central_differences(name, seed):
    p, dout, dhf = _problem(seed)
    g = oracle.selective_scan_backward(p["xc"], p["delta"], p["A_log"], p["Bn"], p["Cn"], p["D"], p["z"], dout,
                                       p["h0"], dhf)
    rng = np.random.default_rng(100 + seed)
    v = rng.normal(0, 1, p[name].shape)
    eps = 1e-6
    hi = dict(p, **{name: p[name] + eps * v})
    lo = dict(p, **{name: p[name] - eps * v})
    fd = (_objective(hi, dout, dhf) - _objective(lo, dout, dhf)) / (2 * eps)
    an = float(np.sum(g[GRAD_OF[name]] * v))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)


def test_every_element_of_a_tiny_problem():
    # element-wise differences on a 1 x 3 x 2 x 2 problem: catches an error confined to one index
    p, dout, dhf = _problem(4, B=1, L=3, C=2, N=2)
    g = oracle.selective_scan_backward(p["xc"], p["delta"], p["A_log"], p["Bn"], p["Cn"], p["D"], p["z"], dout,
                                       p["h0"], dhf)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        for idx in np.ndindex(p[name].shape):
            hi = {k: v.copy() for k, v in p.items()}
            lo = {k: v.copy() for k, v in p.items()}
            hi[name][idx] += eps
            lo[name][idx] -= eps
            fd = (_objective(hi, dout, dhf) - _objective(lo, dout, dhf)) / (2 * eps)
            assert math.isclose(fd, g[gname][idx], rel_tol=1e-6, abs_tol=1e-8), (name, idx, fd, g[gname][idx])


def test_channel_subsets_sum_to_the_shared_gradients():
    p, dout, dhf = _problem(5, C=6)
    full = oracle.selective_scan_backward(p["xc"], p["delta"], p["A_log"], p["Bn"], p["Cn"], p["D"], p["z"], dout,
                                          p["h0"], dhf)
    parts = []
    for sel in (slice(0, 2), slice(2, 6)):
        parts.append(oracle.selective_scan_backward(p["xc"][..., sel], p["delta"][..., sel], p["A_log"][sel],
                                                    p["Bn"], p["Cn"], p["D"][sel], p["z"][..., sel],
                                                    dout[..., sel], p["h0"][:, sel], dhf[:, sel]))
        for k in ("dxc", "ddelta", "dz"):
            np.testing.assert_allclose(parts[-1][k], full[k][..., sel], rtol=1e-13, atol=1e-14)
    for k in ("dB", "dC"):
        np.testing.assert_allclose(parts[0][k] + parts[1][k], full[k], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("split", [1, 4, 6])
def test_backward_split_in_time_equals_whole(split):
    # the second part runs from the first part's final state; the first part receives the second part's dh0
    p, dout, dhf = _problem(6)
    full = oracle.selective_scan_backward(p["xc"], p["delta"], p["A_log"], p["Bn"], p["Cn"], p["D"], p["z"], dout,
                                          p["h0"], dhf)
    a = {k: (v[:, :split] if v.ndim == 3 and k not in ("h0",) else v) for k, v in p.items()}
    b = {k: (v[:, split:] if v.ndim == 3 and k not in ("h0",) else v) for k, v in p.items()}
    _, _, h_mid = oracle.scan_forward_gated(a["xc"], a["delta"], a["A_log"], a["Bn"], a["Cn"], a["D"], a["z"],
                                            a["h0"])
    b["h0"] = h_mid
    gb = oracle.selective_scan_backward(b["xc"], b["delta"], b["A_log"], b["Bn"], b["Cn"], b["D"], b["z"],
                                        dout[:, split:], b["h0"], dhf)
    ga = oracle.selective_scan_backward(a["xc"], a["delta"], a["A_log"], a["Bn"], a["Cn"], a["D"], a["z"],
                                        dout[:, :split], a["h0"], gb["dh0"])
    for k in ("dxc", "ddelta", "dz", "dB", "dC"):
        np.testing.assert_allclose(np.concatenate([ga[k], gb[k]], axis=1), full[k], rtol=1e-12, atol=1e-13)
    for k in ("dA_log", "dD"):
        np.testing.assert_allclose(ga[k] + gb[k], full[k], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ga["dh0"], full["dh0"], rtol=1e-12, atol=1e-13)
