"""GPU parity at the library's size limits (through the C ABI): the longest prefill a call accepts (2^21
tokens), more tokens than a grid's y axis holds (fp32 path, checked in full), and the largest batch (65536
sequences, one decode step)."""

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import MixerConfig, make_activations, make_state, make_weights, to_f64
from parity_util import assert_bitwise, assert_close, log, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_SEQLEN = 1 << 21
MAX_BATCH = 1 << 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _mixer(cfg, w):
    import mamba_selective_scan_05_amd as jm
    return jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)


def test_fp32_prefill_beyond_65536_token_rows():
    # 70000 tokens in fp32: the vector-ALU projections index tokens past 65535; compared in full
    cfg = MixerConfig("limits_f32_L70000", batch=1, seqlen=70000, d_inner=64, dt_rank=8, io_dtype="f32", seed=81,
                      with_state=True)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    log(f"[{cfg.name}] L={cfg.seqlen} C={cfg.d_inner}")
    out, cs, hs = _mixer(cfg, w).prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    ro, rc, rh = oracle.mixer_prefill(to_f64(a["x"]), to_f64(a["z"]), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                      cfg.norm_eps, to_f64(st["conv_state"]), to_f64(st["ssm_state"]))
    assert_close("out", out, ro, "f32", magnitude_scaled=True)
    assert_close("h_final", hs, rh, "f32", magnitude_scaled=True)
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(torch.float32))


def test_longest_prefill_tail_against_oracle():
    # 2^21 tokens in one call; the last 256 tokens and the final states are checked against the oracle run
    # from the state a separate GPU call leaves after the first 2^21 - 256 tokens
    cfg = MixerConfig("limits_bf16_L2M", batch=1, seqlen=MAX_SEQLEN, d_inner=64, dt_rank=8, io_dtype="bf16",
                      seed=82, with_state=True)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    m = _mixer(cfg, w)
    log(f"[{cfg.name}] L={cfg.seqlen} C={cfg.d_inner}")
    out, cs, hs = m.prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    tail = 256
    head = cfg.seqlen - tail
    _, cp, hp = m.prefill(a["x"][:, :head], a["z"][:, :head], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ro, rc, rh = oracle.mixer_prefill(to_f64(a["x"][:, head:]), to_f64(a["z"][:, head:]), weights_f64(w),
                                      cfg.dt_rank, cfg.d_state, cfg.norm_eps, to_f64(cp), to_f64(hp))
    assert_close("out[tail]", out[:, head:], ro, "bf16")
    assert_close("h_final", hs, rh, "bf16")
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(torch.bfloat16))


def test_largest_batch_decode_step():
    cfg = MixerConfig("limits_B65536", batch=MAX_BATCH, seqlen=1, d_inner=64, dt_rank=8, io_dtype="bf16", seed=83,
                      with_state=True)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    log(f"[{cfg.name}] B={cfg.batch} C={cfg.d_inner}")
    x, z = a["x"][:, 0].contiguous(), a["z"][:, 0].contiguous()
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    out, _, _ = _mixer(cfg, w).decode_step(x, z, cs, hs, in_place=True)
    torch.cuda.synchronize()
    ro, rc, rh = oracle.mixer_decode_step(to_f64(x), to_f64(z), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                          to_f64(st["conv_state"]), to_f64(st["ssm_state"]), cfg.norm_eps)
    assert_close("out", out, ro, "bf16")
    assert_close("h", hs, rh, "bf16")
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(torch.bfloat16))
