"""GPU parity of the whole Mamba layer (include/jm_layer.h: pre-norm, in_proj, mixer, out_proj, residual)
against the fp64 layer oracle, through the C ABI.

Tolerances are the mixer's (parity_util) applied to the layer output and the final SSM state.  At the layer
level the conv state holds in_proj outputs, which the library rounds to the I/O type like every activation,
so it is compared with the same tolerance instead of bit for bit.  In bf16 mode the output also carries the
rounding of x_res + increment to bf16.
"""

import pytest
import torch

import oracle
from jm_inputs import LAYER_CONFIGS, MixerConfig, make_layer_input, make_layer_weights, make_state, make_weights, \
    to_f64
from parity_util import assert_close, log, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _layer(cfg, w, lw):
    import mamba_selective_scan_05_amd as jm
    return jm.Layer(lw, w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, 1e-6)


def _check_prefill(cfg, with_state=True, in_place=False):
    w = make_weights(cfg, DEV)
    lw = make_layer_weights(cfg, DEV)
    x_res = make_layer_input(cfg, DEV)
    st = make_state(cfg, DEV) if with_state else {"conv_state": None, "ssm_state": None}
    log(f"[{cfg.name}] B={cfg.batch} L={cfg.seqlen} d_model={cfg.d_model} C={cfg.d_inner} R={cfg.dt_rank} "
        f"{cfg.io_dtype} state={with_state} in_place={in_place}")
    layer = _layer(cfg, w, lw)
    x64 = to_f64(x_res)
    buf = x_res.clone() if in_place else None
    out, cs, hs = layer.prefill(buf if in_place else x_res, st["conv_state"], st["ssm_state"], out=buf)
    torch.cuda.synchronize()
    if in_place:
        assert out.data_ptr() == buf.data_ptr()
    ro, rc, rh = oracle.layer_prefill(x64, weights_f64(lw), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                      cfg.norm_eps, 1e-6,
                                      None if st["conv_state"] is None else to_f64(st["conv_state"]),
                                      None if st["ssm_state"] is None else to_f64(st["ssm_state"]))
    assert_close("out", out, ro, cfg.io_dtype)
    if cfg.io_dtype == "f32":     # the increment alone (in bf16 the output rounding dominates it)
        assert_close("increment", to_f64(out) - x64, ro - x64, cfg.io_dtype)
    assert_close("h_final", hs, rh, cfg.io_dtype)
    assert_close("conv_state", cs, rc, cfg.io_dtype)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [True, False])
def test_layer_prefill_small(io, with_state):
    # several scan pieces and x_proj tiles, a ragged tail, d_model != d_inner
    cfg = MixerConfig(f"layer_small_{io}", batch=2, seqlen=700, d_inner=256, dt_rank=16, io_dtype=io, seed=31,
                      d_model=192)
    _check_prefill(cfg, with_state)


def test_layer_prefill_in_place_residual():
    cfg = MixerConfig("layer_in_place", batch=1, seqlen=300, d_inner=128, dt_rank=16, io_dtype="bf16", seed=32,
                      d_model=256)
    _check_prefill(cfg, True, in_place=True)


def test_layer_jamba_widths_512_tokens():
    # Jamba v0.1's widths (d_model 4096, d_inner 8192, dt_rank 256) at a length the fp64 oracle finishes
    # in seconds
    cfg = LAYER_CONFIGS[0].replace(name="jamba_layer_L512", seqlen=512)
    _check_prefill(cfg, False)


def test_layer_jamba_widths_200_tokens():
    # at most 256 tokens at Jamba's widths: both projections on the weight-streaming kernel with the column
    # blocks and K splits of the benched B = 256 decode step, here with a ragged last token group
    cfg = LAYER_CONFIGS[0].replace(name="jamba_layer_L200", seqlen=200)
    _check_prefill(cfg, False)


@pytest.mark.parametrize("B,L", [(2, 100), (1, 1), (1, 256)])
def test_layer_prefill_up_to_256_tokens_in_place(B, L):
    # at most 256 tokens in bf16: both projections run on the library's weight-streaming kernel; d_inner 1024
    # against d_model 128 splits out_proj's K range (fp32 partials added by the reduce kernel, with the
    # residual read from the output buffer itself)
    cfg = MixerConfig(f"layer_skinny_B{B}_L{L}", batch=B, seqlen=L, d_inner=1024, dt_rank=64, io_dtype="bf16",
                      seed=35, d_model=128)
    _check_prefill(cfg, True, in_place=True)


def test_layer_prefill_wide_in_proj_blocks():
    # d_inner 8192 makes in_proj 16384 columns wide: the weight-streaming kernel takes 128-column blocks over
    # two K slices (partial sums added by the reduce kernel); 200 tokens leave a ragged last token group
    cfg = MixerConfig("layer_skinny_wide", batch=2, seqlen=100, d_inner=8192, dt_rank=64, io_dtype="bf16", seed=36,
                      d_model=512)
    _check_prefill(cfg, True, in_place=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_layer_decode_steps(io):
    cfg = MixerConfig(f"layer_decode_{io}", batch=3, seqlen=1, d_inner=128, dt_rank=16, io_dtype=io, seed=33,
                      d_model=64, with_state=True)
    w = make_weights(cfg, DEV)
    lw = make_layer_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    xs = make_layer_input(cfg, DEV, steps=5)
    layer = _layer(cfg, w, lw)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    c64, h64 = to_f64(st["conv_state"]), to_f64(st["ssm_state"])
    w64, lw64 = weights_f64(w), weights_f64(lw)
    for t in range(xs.shape[1]):
        x = xs[:, t].contiguous()
        out, _, _ = layer.decode_step(x, cs, hs, in_place=True)
        torch.cuda.synchronize()
        ro, c64, h64 = oracle.layer_decode_step(to_f64(x), lw64, w64, cfg.dt_rank, cfg.d_state, c64, h64,
                                                cfg.norm_eps, 1e-6)
        assert_close(f"out[{t}]", out, ro, io)
    assert_close("h_final", hs, h64, io)
    assert_close("conv_state", cs, c64, io)


def test_layer_rejects_bad_dims():
    import mamba_selective_scan_05_amd as jm
    d = jm.make_layer_dims(1, 16, 128, 16, jm.JM_BF16, 60)          # d_model not a multiple of 8
    assert jm.layer_workspace_size(d) == 0
    d = jm.make_layer_dims(1, 16, 100, 16, jm.JM_BF16, 64)          # d_inner not a multiple of 64
    assert jm.layer_workspace_size(d) == 0
    cfg = MixerConfig("layer_bad", batch=1, seqlen=16, d_inner=128, dt_rank=16, io_dtype="bf16", seed=34,
                      d_model=64)
    layer = _layer(cfg, make_weights(cfg, DEV), make_layer_weights(cfg, DEV))
    x = make_layer_input(cfg, DEV)
    d = layer.dims(1, 16)
    s = jm.call_layer(d, layer.packed, x.data_ptr(), x.data_ptr(), None, None, None, None, None, 0,
                      torch.cuda.current_stream().cuda_stream)
    assert s == jm._lib.JM_ERR_INVALID_ARG          # no state outputs
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    co = torch.empty((1, 128, 3), dtype=torch.bfloat16, device=DEV)
    ho = torch.empty((1, 128, 16), dtype=torch.float32, device=DEV)
    s = jm.call_layer(d, layer.packed, x.data_ptr(), x.data_ptr(), None, co.data_ptr(), None, ho.data_ptr(),
                      ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert s == jm._lib.JM_ERR_WORKSPACE


def test_layer_decode_unsplit_wide_blocks():
    # d_inner 16384 makes in_proj 32768 columns wide over K = d_model = 64: 256 blocks of 128 columns fill the
    # GPU without a K split, so the weight-streaming kernel writes bf16 results directly (no partial sums)
    cfg = MixerConfig("layer_skinny_unsplit", batch=3, seqlen=1, d_inner=16384, dt_rank=16, io_dtype="bf16",
                      seed=37, d_model=64, with_state=True)
    w = make_weights(cfg, DEV)
    lw = make_layer_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    xs = make_layer_input(cfg, DEV, steps=2)
    layer = _layer(cfg, w, lw)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    c64, h64 = to_f64(st["conv_state"]), to_f64(st["ssm_state"])
    w64, lw64 = weights_f64(w), weights_f64(lw)
    for t in range(xs.shape[1]):
        x = xs[:, t].contiguous()
        out, _, _ = layer.decode_step(x, cs, hs, in_place=True)
        torch.cuda.synchronize()
        ro, c64, h64 = oracle.layer_decode_step(to_f64(x), lw64, w64, cfg.dt_rank, cfg.d_state, c64, h64,
                                                cfg.norm_eps, 1e-6)
        assert_close(f"out[{t}]", out, ro, "bf16")
    assert_close("h_final", hs, h64, "bf16")
    assert_close("conv_state", cs, c64, "bf16")
