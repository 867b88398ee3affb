"""GPU parity with a nonzero conv bias (the input recipe's conv bias is zero, so the other suites never add
one): every kernel that runs the conv, against the fp64 oracle, through the C ABI.

- the prefill's conv pass (`conv_silu_kernel`: a few hundred tokens, two sequences, with and without states);
- the one-token step (`conv_step_kernel`) over a few steps, the states carried;
- the step as one cooperative kernel (`decode_step_kernel`, bf16, d_inner a multiple of 256);
- the packed variable-length prefill (`conv_silu_varlen_kernel`).
The long-input path (the conv inside x_proj) is covered in test_gpu_parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import MixerConfig, make_activations, make_state, make_weights, to_f64
from parity_util import assert_bitwise, assert_close, log, oracle_prefill, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _weights_with_bias(cfg, seed):
    w = make_weights(cfg, DEV)
    g = torch.Generator(device="cpu").manual_seed(seed)
    w["conv_b"] = (0.5 * torch.randn(cfg.d_inner, generator=g)).to(cfg.torch_dtype).to(DEV)
    return w


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [True, False])
def test_prefill_conv_bias(io, with_state):
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig(f"bias_prefill_{io}", batch=2, seqlen=333, d_inner=256, dt_rank=32, io_dtype=io, seed=61)
    log(f"[{cfg.name}] with_state={with_state}")
    w = _weights_with_bias(cfg, 62)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV) if with_state else {"conv_state": None, "ssm_state": None}
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    out, cs, hs = m.prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    h0 = None if st["ssm_state"] is None else to_f64(st["ssm_state"])
    ro, rc, rh = oracle_prefill(cfg, weights_f64(w), a["x"], a["z"], st["conv_state"], h0)
    assert_close("out", out, ro, io)
    assert_close("h_final", hs, rh, io)
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


@pytest.mark.parametrize("single_kernel", [False, True])
def test_decode_steps_conv_bias(single_kernel):
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig("bias_decode", batch=40, seqlen=1, d_inner=512, dt_rank=64, io_dtype="bf16", seed=63,
                      with_state=True)
    log(f"[{cfg.name}] single_kernel={single_kernel}")
    w = _weights_with_bias(cfg, 64)
    st = make_state(cfg, DEV)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    w64 = weights_f64(w)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    c64, h64 = to_f64(cs), to_f64(hs)
    g = torch.Generator(device=DEV)
    g.manual_seed(65)
    for t in range(3):
        x = torch.randn((cfg.batch, cfg.d_inner), generator=g, device=DEV).to(cfg.torch_dtype)
        z = torch.randn((cfg.batch, cfg.d_inner), generator=g, device=DEV).to(cfg.torch_dtype)
        out, _, _ = m.decode_step(x, z, cs, hs, in_place=True, single_kernel=single_kernel)
        torch.cuda.synchronize()
        ro, c64, h64 = oracle.mixer_decode_step(to_f64(x), to_f64(z), w64, cfg.dt_rank, cfg.d_state, c64, h64,
                                                cfg.norm_eps)
        assert_close(f"step {t} out", out, ro, "bf16")
    assert_close("ssm_state after 3 steps", hs, h64, "bf16")
    assert_bitwise("conv_state after 3 steps", cs, torch.from_numpy(c64).to(cfg.torch_dtype))


def test_packed_prefill_conv_bias():
    import mamba_selective_scan_05_amd as jm
    lengths = [5, 300, 1, 0, 120]
    T, C, R = sum(lengths), 256, 16
    cfg = MixerConfig("bias_packed", batch=len(lengths), seqlen=T, d_inner=C, dt_rank=R, io_dtype="bf16", seed=66,
                      with_state=True)
    w = _weights_with_bias(cfg, 67)
    st = make_state(cfg, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(68)
    x = torch.randn((T, C), generator=g, device=DEV).to(cfg.torch_dtype)
    z = torch.randn((T, C), generator=g, device=DEV).to(cfg.torch_dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=DEV)
    m = jm.Mixer(w, R, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    out, cs, hs = m.prefill_varlen(x, z, cu, st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    w64 = weights_f64(w)
    t0 = 0
    for s, n in enumerate(lengths):
        if n == 0:
            assert torch.equal(cs[s], st["conv_state"][s]) and torch.equal(hs[s], st["ssm_state"][s])
            continue
        ro, rc, rh = oracle.mixer_prefill(to_f64(x[t0:t0 + n])[None], to_f64(z[t0:t0 + n])[None], w64, R,
                                          cfg.d_state, cfg.norm_eps, to_f64(st["conv_state"][s:s + 1]),
                                          to_f64(st["ssm_state"][s:s + 1]))
        assert_close(f"out of sequence {s}", out[t0:t0 + n], ro[0], "bf16")
        assert_close(f"ssm_state of sequence {s}", hs[s], rh[0], "bf16")
        assert_bitwise(f"conv_state of sequence {s}", cs[s], torch.from_numpy(rc[0]).to(cfg.torch_dtype))
        t0 += n
