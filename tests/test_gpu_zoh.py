"""GPU parity of the exact zero-order-hold variant (jm_mixer_dims.discretization = JM_DISC_ZOH): the input
matrix (exp(dt A) - 1) / A * B instead of dt * B, against the fp64 oracle with zoh=True (which evaluates
expm1 exactly).  Same tolerances as the default form.  The workloads' dt * A spans both of the kernel's
branches (the series below |dt A| = 1/16 and the direct form above); one case pushes every dt * A into the
series.
"""

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import CONFIGS, MixerConfig, make_activations, make_decode_tokens, make_layer_input, \
    make_layer_weights, make_state, make_weights, to_f64
from parity_util import assert_bitwise, assert_close, log, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _mixer(cfg, w):
    import mamba_selective_scan_05_amd as jm
    return jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, zoh=True)


def _check(cfg, w=None, channels=None, differs=True):
    w = w if w is not None else make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    log(f"[{cfg.name}] B={cfg.batch} L={cfg.seqlen} C={cfg.d_inner} {cfg.io_dtype} zoh")
    out, cs, hs = _mixer(cfg, w).prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    h0 = to_f64(st["ssm_state"])
    sel = slice(None) if channels is None else channels
    ro, rc, rh = oracle.mixer_prefill(to_f64(a["x"]), to_f64(a["z"]), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                      cfg.norm_eps, to_f64(st["conv_state"]),
                                      h0 if channels is None else h0[:, channels], channels=channels, zoh=True)
    assert_close("out", out[..., sel], ro, cfg.io_dtype)
    assert_close("h_final", hs[:, sel], rh, cfg.io_dtype)
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))
    if differs:   # at these step sizes the variant is a different computation from the default form
        import mamba_selective_scan_05_amd as jm
        e_out, _, _ = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps).prefill(
            a["x"], a["z"], st["conv_state"], st["ssm_state"])
        torch.cuda.synchronize()
        assert (e_out.float() - out.float()).abs().max() > 1e-3


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_zoh_prefill_pieces(io):
    _check(MixerConfig(f"zoh_{io}", batch=2, seqlen=700, d_inner=256, dt_rank=16, io_dtype=io, seed=71,
                       with_state=True))


def test_zoh_series_branch():
    # A ~ -2e-9: every |dt A| is far below 1/16, where exp(dt A) - 1 would cancel; the result must still match
    # (and there ZOH and dt * B agree, the limit the oracle pins)
    cfg = MixerConfig("zoh_series", batch=1, seqlen=300, d_inner=128, dt_rank=16, io_dtype="f32", seed=72,
                      with_state=True)
    w = make_weights(cfg, DEV)
    w["A_log"] = torch.full_like(w["A_log"], -20.0)
    _check(cfg, w, differs=False)


def test_zoh_jamba_prefill_4k_sampled_channels():
    cfg = CONFIGS[1].replace(name="zoh_jamba_B1_L4096", with_state=True, seed=73)
    _check(cfg, channels=np.arange(3, cfg.d_inner, 53))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_zoh_decode_steps(io):
    cfg = MixerConfig(f"zoh_decode_{io}", batch=3, seqlen=1, d_inner=128, dt_rank=16, io_dtype=io, seed=74,
                      decode_steps=5, with_state=True)
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    tok = make_decode_tokens(cfg, DEV)
    m = _mixer(cfg, w)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    outs = []
    for t in range(cfg.decode_steps):
        o, _, _ = m.decode_step(tok["x"][:, t], tok["z"][:, t], cs, hs, in_place=True)
        outs.append(o.clone())
    torch.cuda.synchronize()
    ro, rc, rh = oracle.mixer_prefill(to_f64(tok["x"]), to_f64(tok["z"]), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                      cfg.norm_eps, to_f64(st["conv_state"]), to_f64(st["ssm_state"]), zoh=True)
    assert_close("decode out", torch.stack(outs, dim=1), ro, io)
    assert_close("h_final", hs, rh, io)


def test_zoh_packed_prefill():
    import mamba_selective_scan_05_amd as jm
    lens = [150, 0, 3, 300, 60]
    cfg = MixerConfig("zoh_varlen", batch=len(lens), seqlen=1, d_inner=128, dt_rank=16, io_dtype="bf16", seed=75,
                      with_state=True)
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    T = sum(lens)
    a = make_activations(cfg.replace(batch=1, seqlen=T), DEV)
    x, z = a["x"][0].contiguous(), a["z"][0].contiguous()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    out, co, so = _mixer(cfg, w).prefill_varlen(x, z, cu, st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    ro, rc, rh = oracle.mixer_prefill_varlen(to_f64(x), to_f64(z), cu.cpu().numpy(), weights_f64(w), cfg.dt_rank,
                                             cfg.d_state, cfg.norm_eps, to_f64(st["conv_state"]),
                                             to_f64(st["ssm_state"]), zoh=True)
    assert_close("out", out, ro, "bf16")
    assert_close("ssm_state", so, rh, "bf16")


def test_zoh_layer():
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig("zoh_layer", batch=2, seqlen=200, d_inner=128, dt_rank=16, io_dtype="bf16", seed=76,
                      d_model=64, with_state=True)
    w = make_weights(cfg, DEV)
    lw = make_layer_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    xr = make_layer_input(cfg, DEV)
    layer = jm.Layer(lw, w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, 1e-6, zoh=True)
    out, cs, hs = layer.prefill(xr, st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    ro, rc, rh = oracle.layer_prefill(to_f64(xr), weights_f64(lw), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                      cfg.norm_eps, 1e-6, to_f64(st["conv_state"]), to_f64(st["ssm_state"]),
                                      zoh=True)
    assert_close("out", out, ro, "bf16")
    assert_close("h_final", hs, rh, "bf16")
