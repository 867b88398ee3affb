"""GPU parity of the gated scan alone and of its backward (include/jm_scan.h) against the fp64 oracle.

The backward's gradients are sums (over tokens for dA_log and dD, over channels for dB and dC), so they are
compared relative to their largest magnitude: fp32 within 1e-4 * max(1, max |ref|), bf16 within 2e-2 of
max |ref| (the bf16 I/O tolerance of the forward).  Cases span many 32-token pieces, ragged sub-chunks and
pieces, a single short piece, no initial state, no tokens, and Jamba's widths at 1024 tokens.
"""

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import MixerConfig, make_scan_problem, to_f64
from parity_util import assert_close, log

pytestmark = pytest.mark.gpu

DEV = "cuda"
GRADS = (("dx", "dxc"), ("ddelta", "ddelta"), ("dz", "dz"), ("dA_log", "dA_log"), ("dD", "dD"), ("dh0", "dh0"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _f64(t):
    return None if t is None else to_f64(t)


def _check_backward(cfg, with_state=True, saved=False):
    import mamba_selective_scan_05_amd as jm
    p = make_scan_problem(cfg, DEV, with_state)
    B, L, C, N = cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state
    log(f"[{cfg.name}] B={B} L={L} C={C} {cfg.io_dtype} state={with_state} saved={saved}")
    states = None
    if saved:
        states = jm.scan_forward(p["x"], p["delta"], p["z"], p["bc"], p["A_log"], p["D"], p["h0"], save=True)[2]
    g = jm.scan_backward(p["x"], p["delta"], p["z"], p["bc"], p["A_log"], p["D"], p["dout"], p["h0"], p["dh_final"],
                         saved_states=states)
    torch.cuda.synchronize()
    bc = to_f64(p["bc"]).reshape(B, L, 2 * N)
    r = oracle.selective_scan_backward(to_f64(p["x"]), to_f64(p["delta"]), to_f64(p["A_log"]), bc[..., :N],
                                       bc[..., N:], to_f64(p["D"]), to_f64(p["z"]), to_f64(p["dout"]), _f64(p["h0"]),
                                       _f64(p["dh_final"]))
    scaled = cfg.io_dtype == "f32"
    for mine, ref in GRADS:
        assert_close(mine, g[mine], r[ref], cfg.io_dtype, magnitude_scaled=scaled)
    dbc = g["dbc"].reshape(B, L, 2 * N)
    assert_close("dB", dbc[..., :N], r["dB"], cfg.io_dtype, magnitude_scaled=scaled)
    assert_close("dC", dbc[..., N:], r["dC"], cfg.io_dtype, magnitude_scaled=scaled)
    return p, g


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_backward_pieces_and_ragged_tail(io):
    # 300 tokens: nine full 32-token pieces and a ragged last piece of 12 (its sub-chunks ragged too)
    cfg = MixerConfig(f"scan_bwd_{io}", batch=2, seqlen=300, d_inner=128, io_dtype=io, seed=61)
    _check_backward(cfg)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_backward_one_short_piece_without_state(io):
    cfg = MixerConfig(f"scan_bwd_short_{io}", batch=3, seqlen=37, d_inner=64, io_dtype=io, seed=62)
    _check_backward(cfg, with_state=False)


def test_scan_backward_exact_piece_multiple():
    cfg = MixerConfig("scan_bwd_256", batch=1, seqlen=256, d_inner=192, io_dtype="f32", seed=63)
    _check_backward(cfg)


def test_scan_backward_jamba_widths_1024_tokens():
    # Jamba v0.1's d_inner 8192 at a length whose full fp64 reference (every state kept) fits the host
    cfg = MixerConfig("scan_bwd_jamba_L1024", batch=1, seqlen=1024, d_inner=8192, io_dtype="bf16", seed=64)
    _check_backward(cfg)


def test_scan_backward_deterministic():
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig("scan_bwd_det", batch=2, seqlen=200, d_inner=128, io_dtype="bf16", seed=65)
    p = make_scan_problem(cfg, DEV)
    args = (p["x"], p["delta"], p["z"], p["bc"], p["A_log"], p["D"], p["dout"], p["h0"], p["dh_final"])
    g1 = jm.scan_backward(*args)
    g2 = jm.scan_backward(*args)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_scan_backward_no_tokens():
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig("scan_bwd_empty", batch=2, seqlen=0, d_inner=64, io_dtype="f32", seed=66)
    p = make_scan_problem(cfg, DEV)
    g = jm.scan_backward(p["x"], p["delta"], p["z"], p["bc"], p["A_log"], p["D"], p["dout"], p["h0"], p["dh_final"])
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], p["dh_final"])
    assert not g["dA_log"].any() and not g["dD"].any()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_forward(io):
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig(f"scan_fwd_{io}", batch=2, seqlen=700, d_inner=128, io_dtype=io, seed=67)
    p = make_scan_problem(cfg, DEV)
    N = cfg.d_state
    out, h = jm.scan_forward(p["x"], p["delta"], p["z"], p["bc"], p["A_log"], p["D"], p["h0"])
    torch.cuda.synchronize()
    bc = to_f64(p["bc"]).reshape(cfg.batch, cfg.seqlen, 2 * N)
    ro, _, rh = oracle.scan_forward_gated(to_f64(p["x"]), to_f64(p["delta"]), to_f64(p["A_log"]), bc[..., :N],
                                          bc[..., N:], to_f64(p["D"]), to_f64(p["z"]), to_f64(p["h0"]))
    assert_close("out", out, ro, io)
    assert_close("h_out", h, rh, io)


def _piece_states(p, cfg):
    """The oracle's state entering tokens 0, 32, 64, ... of every sequence: [B, ceil(L / 32), N, C]."""
    B, L, N = cfg.batch, cfg.seqlen, cfg.d_state
    bc = to_f64(p["bc"]).reshape(B, L, 2 * N)
    x, dl, z, A_log, D = (to_f64(p[k]) for k in ("x", "delta", "z", "A_log", "D"))
    h = np.zeros((B, cfg.d_inner, N)) if p["h0"] is None else to_f64(p["h0"])
    res = []
    for s0 in range(0, L, 32):
        res.append(h.transpose(0, 2, 1))
        e = min(L, s0 + 32)
        h = oracle.scan_forward_gated(x[:, s0:e], dl[:, s0:e], A_log, bc[:, s0:e, :N], bc[:, s0:e, N:], D,
                                      z[:, s0:e], h)[2]
    return np.stack(res, axis=1)


@pytest.mark.parametrize("io,L", [("f32", 700), ("bf16", 700), ("f32", 37), ("bf16", 4096)])
def test_scan_forward_train_saves_piece_states(io, L):
    # the training forward returns the plain forward's outputs bit for bit, plus the states at every 32-token
    # boundary (written by whichever forward piece holds the boundary; several forward pieces at these sizes)
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig(f"scan_fwd_train_{io}_{L}", batch=2, seqlen=L, d_inner=128, io_dtype=io, seed=68)
    p = make_scan_problem(cfg, DEV)
    log(f"[{cfg.name}] B={cfg.batch} L={L} C={cfg.d_inner} {io}")
    args = (p["x"], p["delta"], p["z"], p["bc"], p["A_log"], p["D"], p["h0"])
    out, h = jm.scan_forward(*args)
    out2, h2, saved = jm.scan_forward(*args, save=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(h, h2)
    assert saved.shape == (cfg.batch, (L + 31) // 32, cfg.d_state, cfg.d_inner)
    assert_close("saved_states", saved, _piece_states(p, cfg), io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_backward_from_saved_states(io):
    cfg = MixerConfig(f"scan_bwd_saved_{io}", batch=2, seqlen=300, d_inner=128, io_dtype=io, seed=61)
    _check_backward(cfg, saved=True)


def test_scan_backward_from_saved_states_short_and_wide():
    _check_backward(MixerConfig("scan_bwd_saved_short", batch=3, seqlen=37, d_inner=64, io_dtype="f32", seed=62),
                    with_state=False, saved=True)
    _check_backward(MixerConfig("scan_bwd_saved_jamba_L1024", batch=1, seqlen=1024, d_inner=8192,
                                io_dtype="bf16", seed=64), saved=True)
