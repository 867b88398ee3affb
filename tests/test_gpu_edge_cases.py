"""GPU parity of the method's degenerate cases, through the C ABI, against the fp64 oracle.

The oracle's CPU pins fix each case in closed form (tests/test_oracle_pins.py, tests/test_oracle_zoh_pins.py);
here the HIP path runs them over many scan pieces, in fp32 and bf16 and in both discretisations:

  - A = 0 (A_log = -inf): no decay, so the state is h0 plus the running sum of delta * B * x and every piece
    boundary carries the whole history forward (the carry composes exp(A * sum(delta)) = 1 exactly); the
    exact zero-order hold takes its limit delta * B there.  Also at the 256K workload's full size.
  - delta -> 0 (dt_proj_w = 0, dt_proj_b = -40): the state is left unchanged and out = (C . h0 + D xc) SiLU(z);
    the library's softplus gives exactly 0 below -17 (a reading of the softplus threshold), so the final
    state equals h0 bit for bit.
  - zero input (x = 0, conv bias 0, zero conv state): xc = 0 makes every projection, B and C zero, so out = 0
    exactly and the state decays as exp(A * L * softplus(dt_proj_b)) h0.

Discretisation equations and recurrence: Jamba Guide, "Inside the Mamba State-Space Layers".
"""

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import CONFIGS, MixerConfig, make_activations, make_state, make_weights, to_f64
from parity_util import assert_bitwise, assert_close, log, oracle_long_sampled, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _mixer(cfg, w, zoh):
    import mamba_selective_scan_05_amd as jm
    return jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, zoh=zoh)


def _cfg(name, io, seed):
    # 2 x 2500 tokens over 128 channels: about twenty scan pieces per sequence and a ragged last piece
    return MixerConfig(name, batch=2, seqlen=2500, d_inner=128, dt_rank=16, io_dtype=io, seed=seed)


def _run(cfg, w, a, st, zoh):
    m = _mixer(cfg, w, zoh)
    import mamba_selective_scan_05_amd as jm
    pieces = jm.workspace_layout(m.dims(cfg.batch, cfg.seqlen)).scan_chunks
    out, cs, hs = m.prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    h0 = None if st["ssm_state"] is None else to_f64(st["ssm_state"])
    ro, rc, rh = oracle.mixer_prefill(to_f64(a["x"]), to_f64(a["z"]), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                      cfg.norm_eps, None if st["conv_state"] is None else to_f64(st["conv_state"]),
                                      h0, zoh=zoh)
    return pieces, (out, cs, hs), (ro, rc, rh)


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_A_zero_carries_the_whole_history(io, zoh):
    cfg = _cfg(f"A_zero_{io}", io, 71)
    w = make_weights(cfg, DEV)
    w["A_log"] = torch.full_like(w["A_log"], float("-inf"))
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    log(f"[{cfg.name} {'zoh' if zoh else 'euler'}] A_log = -inf, B={cfg.batch} L={cfg.seqlen} C={cfg.d_inner}")
    pieces, (out, cs, hs), (ro, rc, rh) = _run(cfg, w, a, st, zoh)
    assert pieces > 8
    # the state is a random walk of size ~1 over 2500 tokens: fp32 is held to 1e-4 of the largest value
    assert_close("out", out, ro, io, magnitude_scaled=True)
    assert_close("h_final", hs, rh, io, magnitude_scaled=True)
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


def test_A_zero_long_context_256k_sampled_channels():
    # the 256K workload with A = 0: a piece's carry is the sum of every earlier piece's increment
    cfg = CONFIGS[3]
    w = make_weights(cfg, DEV)
    w["A_log"] = torch.full_like(w["A_log"], float("-inf"))
    a = make_activations(cfg, DEV)
    log(f"[{cfg.name} A_log = -inf] B={cfg.batch} L={cfg.seqlen} C={cfg.d_inner}")
    m = _mixer(cfg, w, False)
    out, cs, hs = m.prefill(a["x"], a["z"])
    torch.cuda.synchronize()
    sel = np.array([1, 513, 2222, 4096, 7001, 8190])
    sel_t = torch.as_tensor(sel, device=DEV)
    log("  oracle on sampled channels ...")
    ro, rh, rc = oracle_long_sampled(cfg, weights_f64(w), a["x"], a["z"], sel)
    assert_close("out[sampled]", out.index_select(2, sel_t), ro, "bf16")
    assert_close("h_final[sampled]", hs.index_select(1, sel_t), rh, "bf16")
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_delta_to_zero_leaves_the_state(io, zoh):
    cfg = _cfg(f"dt_zero_{io}", io, 72)
    w = make_weights(cfg, DEV)
    w["dt_proj_w"] = torch.zeros_like(w["dt_proj_w"])
    w["dt_proj_b"] = torch.full_like(w["dt_proj_b"], -40.0)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    log(f"[{cfg.name} {'zoh' if zoh else 'euler'}] dt_proj_w = 0, dt_proj_b = -40")
    pieces, (out, cs, hs), (ro, rc, rh) = _run(cfg, w, a, st, zoh)
    assert pieces > 8
    assert torch.equal(hs, st["ssm_state"]), "the state moved although delta is 0"
    assert_close("out", out, ro, io)
    assert_close("h_final", hs, rh, io)
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))
    # without a state the output is the skip term alone: D xc SiLU(z)
    out0, _, h_zero = _mixer(cfg, w, zoh).prefill(a["x"], a["z"], st["conv_state"], None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(h_zero) == 0
    xc, _ = oracle.causal_conv1d_silu(to_f64(a["x"]), to_f64(w["conv_w"]), to_f64(w["conv_b"]),
                                      to_f64(st["conv_state"]))
    assert_close("out (no state)", out0, to_f64(w["D"]) * xc * oracle.silu(to_f64(a["z"])), io)


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_zero_input_decays_the_state(io, zoh):
    cfg = _cfg(f"zero_input_{io}", io, 73)
    w = make_weights(cfg, DEV)
    w["conv_b"] = torch.zeros_like(w["conv_b"])
    a = make_activations(cfg, DEV)
    a = {"x": torch.zeros_like(a["x"]), "z": a["z"]}
    st = make_state(cfg, DEV)
    st["conv_state"] = torch.zeros_like(st["conv_state"])
    log(f"[{cfg.name} {'zoh' if zoh else 'euler'}] x = 0, conv bias 0, zero conv state")
    pieces, (out, cs, hs), (ro, rc, rh) = _run(cfg, w, a, st, zoh)
    assert pieces > 8
    assert torch.count_nonzero(out) == 0, "zero input must give an exactly zero output"
    assert torch.count_nonzero(cs) == 0
    assert_close("h_final", hs, rh, io)
    # the oracle's value is the closed form (pinned on the CPU); the GPU's against it directly as well
    dt = np.logaddexp(0.0, to_f64(w["dt_proj_b"]))
    closed = np.exp(-np.exp(to_f64(w["A_log"])) * (cfg.seqlen * dt)[:, None])[None] * to_f64(st["ssm_state"])
    assert_close("h_final vs closed form", hs, closed, io)
