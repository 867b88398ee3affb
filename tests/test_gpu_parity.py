"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle, element by element.

Small cases span several tiles, several scan pieces and ragged tails and are compared in full; the five
workloads run at full size in the launch configuration the benchmark uses and are compared in full where
the oracle finishes in seconds (the tiny fp32 mixer, the 4K prefill) and on sampled channels otherwise
(batched prefill, 256K context, 128 decode steps).  Tolerances are in parity_util.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import CONFIGS, MixerConfig, make_activations, make_decode_tokens, make_state, make_weights, to_f64
from parity_util import (assert_bitwise, assert_close, log, oracle_long_sampled, oracle_prefill, weights_f64)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()          # loads the built library or raises


def _mixer(cfg: MixerConfig, w):
    import mamba_selective_scan_05_amd as jm
    return jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)


def _small(name, B, L, C, R, io, seed, **kw):
    return MixerConfig(name, batch=B, seqlen=L, d_inner=C, dt_rank=R, io_dtype=io, seed=seed, **kw)


def _run_and_check(cfg, with_state=True, row_stride=None, w=None, check_label="", magnitude_scaled=False):
    w = w if w is not None else make_weights(cfg, DEV)
    a = make_activations(cfg, DEV, row_stride=row_stride)
    st = make_state(cfg, DEV) if with_state else {"conv_state": None, "ssm_state": None}
    log(f"[{cfg.name}{check_label}] B={cfg.batch} L={cfg.seqlen} C={cfg.d_inner} R={cfg.dt_rank} {cfg.io_dtype}")
    m = _mixer(cfg, w)
    out, cs, hs = m.prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    w64 = weights_f64(w)
    h0 = None if st["ssm_state"] is None else to_f64(st["ssm_state"])
    ro, rc, rh = oracle_prefill(cfg, w64, a["x"], a["z"], st["conv_state"], h0)
    assert_close("out", out, ro, cfg.io_dtype, magnitude_scaled)
    assert_close("h_final", hs, rh, cfg.io_dtype, magnitude_scaled)
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))
    return m, out, cs, hs


# ----------------------------------------------------------------------------- small and ragged cases

def test_tiny_f32_workload():
    _run_and_check(CONFIGS[0], with_state=False)
    _run_and_check(CONFIGS[0].replace(with_state=True), with_state=True, check_label="+state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ragged_multi_piece(io):
    # 2 x 700 tokens over 128 channels: the scan runs in several pieces with a ragged last piece, the
    # projections over several token tiles with a ragged last tile
    cfg = _small(f"ragged_{io}", 2, 700, 128, 16, io, 11)
    _run_and_check(cfg)


def test_f32_jamba_widths_split_projections():
    # fp32 I/O at d_inner 8192, dt_rank 256: x_proj's fp32 matrix-core GEMM splits its channels over 16
    # slices (4 token tiles x 3 column tiles of 128 x 96), dt_proj's covers 4 x 64 tiles of 128 x 128 with a
    # 32-wide K loop
    import mamba_selective_scan_05_amd as jm
    cfg = _small("f32_jamba_widths", 1, 512, 8192, 256, "f32", 31)
    w = make_weights(cfg, DEV)
    assert jm.workspace_layout(_mixer(cfg, w).dims(cfg.batch, cfg.seqlen)).dbc_splits == 16
    _run_and_check(cfg, w=w)


def test_f32_many_token_tiles():
    # fp32 I/O over 2 x 4096 tokens: x_proj's fp32 GEMM runs 64 token tiles (its 96 columns one tile) over 8
    # channel slices, dt_proj's 64 x 8 tiles; the scan over several pieces per sequence
    import mamba_selective_scan_05_amd as jm
    cfg = _small("f32_many_tiles", 2, 4096, 1024, 64, "f32", 32)
    w = make_weights(cfg, DEV)
    assert jm.workspace_layout(_mixer(cfg, w).dims(cfg.batch, cfg.seqlen)).dbc_splits == 8
    _run_and_check(cfg, w=w)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_largest_dt_rank(io):
    # dt_rank 512 (the largest supported): x_proj runs as two column groups and dt_proj takes its
    # general path (the K loop over dt_rank slices)
    cfg = _small(f"rank512_{io}", 2, 300, 256, 512, io, 20)
    _run_and_check(cfg)


def test_bf16_wide_strided_views():
    # x and z as strided halves of one [B, L, 2C + 64] buffer, as an in_proj output holds them
    cfg = _small("bf16_strided", 2, 333, 512, 64, "bf16", 12)
    _run_and_check(cfg, row_stride=2 * 512 + 64)


@pytest.mark.parametrize("with_state", [True, False])
def test_bf16_wide_xproj_tiles_across_sequences(with_state):
    # enough tokens for x_proj's 288-column tiles (its three-stage LDS pipeline): sequence starts fall inside
    # 128-token tiles, a ragged last tile, strided x and z, with and without incoming states
    import mamba_selective_scan_05_amd as jm
    cfg = _small(f"wide_xproj_{'state' if with_state else 'nostate'}", 3, 2900, 256, 16, "bf16", 21)
    assert jm.workspace_layout(jm.make_dims(3, 2900, 256, 16, jm.JM_BF16)).xproj_path == 0
    _run_and_check(cfg, with_state=with_state, row_stride=528)


@pytest.mark.parametrize("R", [16, 512])
def test_bf16_tall_xproj_ragged(R):
    # 32768 tokens or more: x_proj takes 256-token tiles (eight waves, two LDS stages) and computes the conv
    # itself; 40000 tokens leave a ragged last tile of 64, dt_rank 512 makes two 288-column groups (only the
    # first writes xc)
    import mamba_selective_scan_05_amd as jm
    cfg = _small(f"tall_xproj_R{R}", 1, 40000, 256, R, "bf16", 23)
    assert jm.workspace_layout(jm.make_dims(1, 40000, 256, R, jm.JM_BF16)).xproj_path == 4
    _run_and_check(cfg)


@pytest.mark.parametrize("with_state", [True, False])
def test_bf16_conv_inside_tall_xproj_across_sequences(with_state):
    # 3 x 11000 tokens: the conv runs inside the tall x_proj.  Sequence starts fall inside 256-token tiles
    # (their first 3 tokens take the conv state as left context), x and z are strided views, the channels
    # are split over two slices, the last tile is ragged.  Against the oracle, and xc bit for bit against the
    # conv kernel on its own (the same tokens as one packed batch, whose conv runs as a separate pass).
    import mamba_selective_scan_05_amd as jm
    B, L, C = 3, 11000, 256
    cfg = _small(f"conv_in_xproj_{'state' if with_state else 'nostate'}", B, L, C, 16, "bf16", 24)
    lay = jm.workspace_layout(jm.make_dims(B, L, C, 16, jm.JM_BF16, x_row_stride=528, z_row_stride=528))
    assert lay.xproj_path == 4 and lay.dbc_splits == 2
    m, _, _, _ = _run_and_check(cfg, with_state=with_state, row_stride=528)
    xc_fused = m._ws[lay.xc:lay.xc + B * L * C * 2].view(torch.bfloat16).clone()
    a = make_activations(cfg, DEV, row_stride=528)
    st = make_state(cfg, DEV) if with_state else {"conv_state": None, "ssm_state": None}
    cu = torch.tensor([0, L, 2 * L, 3 * L], dtype=torch.int32, device=DEV)
    m.prefill_varlen(a["x"].reshape(B * L, C), a["z"].reshape(B * L, C), cu, st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    xc_sep = m._ws[:B * L * C * 2].view(torch.bfloat16)
    assert_bitwise("xc (conv inside x_proj vs the conv kernel)", xc_fused, xc_sep)


@pytest.mark.parametrize("L", [2, 4, 5])
def test_bf16_conv_inside_tall_xproj_short_sequences(L):
    # many short sequences reaching the long-input layout (at least 32768 tokens): with L = 2 every token is
    # fewer than 3 positions into its sequence (all taken from the conv kernel's rows), with 4 and 5 most are
    import mamba_selective_scan_05_amd as jm
    B = -(-32768 // L)
    cfg = _small(f"conv_in_xproj_L{L}", B, L, 64, 8, "bf16", 27)
    assert jm.workspace_layout(jm.make_dims(B, L, 64, 8, jm.JM_BF16)).xproj_path == 4
    _run_and_check(cfg)


def test_bf16_conv_inside_tall_xproj_bias():
    # the recipe's conv bias is zero: here a random one, through the conv inside x_proj (33000 tokens, two
    # sequences, a ragged last tile) against the oracle and, bit for bit, against the packed-batch path (whose
    # conv is the separate kernel); then no bias at all (a NULL pointer) equals a zero bias bit for bit
    import mamba_selective_scan_05_amd as jm
    B, L, C, R = 2, 16500, 256, 16
    cfg = _small("conv_in_xproj_bias", B, L, C, R, "bf16", 25)
    assert jm.workspace_layout(jm.make_dims(B, L, C, R, jm.JM_BF16)).xproj_path == 4
    w = make_weights(cfg, DEV)
    g = torch.Generator(device="cpu").manual_seed(26)
    w["conv_b"] = (0.5 * torch.randn(C, generator=g)).to(cfg.torch_dtype).to(DEV)
    m, out, _, _ = _run_and_check(cfg, w=w)
    lay = jm.workspace_layout(m.dims(B, L))
    xc_fused = m._ws[lay.xc:lay.xc + B * L * C * 2].view(torch.bfloat16).clone()
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    cu = torch.tensor([0, L, 2 * L], dtype=torch.int32, device=DEV)
    m.prefill_varlen(a["x"].reshape(B * L, C), a["z"].reshape(B * L, C), cu, st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    assert_bitwise("xc with a bias (conv inside x_proj vs the conv kernel)", xc_fused, m._ws[:B * L * C * 2].view(torch.bfloat16))
    w0 = dict(w)
    w0["conv_b"] = torch.zeros_like(w["conv_b"])
    wn = {k: v for k, v in w.items() if k != "conv_b"}
    outs = []
    for ww in (w0, wn):
        mm = _mixer(cfg, ww)
        o, cs, hs = mm.prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
        torch.cuda.synchronize()
        outs.append((o, cs, hs))
    for i, name in enumerate(("out", "conv_state", "ssm_state")):
        assert torch.equal(outs[0][i], outs[1][i]), f"{name}: NULL conv bias differs from a zero bias"


@pytest.mark.parametrize("B,L", [(1, 450), (2, 155)])
def test_bf16_few_token_tiles_dt_proj(B, L):
    # at most 8 64-token tiles: dt_proj takes 128-channel workgroups; at d_inner 8192 they hold two tiles
    # each (the first case) or one or two with an empty last group (the second), with a ragged last tile
    cfg = _small(f"few_tiles_B{B}_L{L}", B, L, 8192, 256, "bf16", 22)
    _run_and_check(cfg)


@pytest.mark.parametrize("L", [0, 1, 2, 3, 5, 64, 65])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_short_sequences_and_conv_state(L, io):
    cfg = _small(f"short_L{L}_{io}", 3, L, 64, 8, io, 13)
    if L == 0:
        w = make_weights(cfg, DEV)
        st = make_state(cfg, DEV)
        m = _mixer(cfg, w)
        x = torch.empty((3, 0, 64), dtype=cfg.torch_dtype, device=DEV)
        _, cs, hs = m.prefill(x, x, st["conv_state"], st["ssm_state"])
        assert_bitwise("conv_state", cs, st["conv_state"])
        assert torch.equal(hs, st["ssm_state"])
        return
    _run_and_check(cfg)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_slow_decay_carries_and_scan_term_alone(io):
    """A_log - 6 makes the state remember thousands of tokens, so every piece boundary of the scan matters,
    and D = 0 leaves the scan term alone in the output (no skip term to hide an error)."""
    cfg = _small(f"slow_decay_{io}", 2, 2500, 128, 16, io, 14)
    w = make_weights(cfg, DEV)
    w["A_log"] = (w["A_log"].float() - 6.0).to(cfg.torch_dtype)
    w["D"] = torch.zeros_like(w["D"])
    import mamba_selective_scan_05_amd as jm
    lay = jm.workspace_layout(_mixer(cfg, w).dims(cfg.batch, cfg.seqlen))
    assert lay.scan_chunks > 1
    # slow decay lets the state grow to |out| ~ 400: the fp32 bound is taken relative to that magnitude
    _run_and_check(cfg, w=w, magnitude_scaled=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_intermediates_step_by_step(io):
    import mamba_selective_scan_05_amd as jm
    cfg = _small(f"steps_{io}", 2, 300, 256, 64, io, 15)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    m = _mixer(cfg, w)
    out, _, _ = m.prefill(a["x"], a["z"])
    torch.cuda.synchronize()
    dims = m.dims(cfg.batch, cfg.seqlen)
    lay = jm.workspace_layout(dims)
    ws = m._ws
    T, C, R, W = cfg.batch * cfg.seqlen, cfg.d_inner, cfg.dt_rank, cfg.width
    dt = cfg.torch_dtype
    esz = 4 if io == "f32" else 2

    def view(off, n, dtype):
        nbytes = n * (4 if dtype == torch.float32 else 2)
        return ws[off:off + nbytes].view(dtype)

    w64 = weights_f64(w)
    _, _, _, inter = oracle.mixer_prefill(to_f64(a["x"]), to_f64(a["z"]), w64, R, cfg.d_state, cfg.norm_eps,
                                          return_intermediates=True)
    xc = view(lay.xc, T * C, dt).view(cfg.batch, cfg.seqlen, C)
    assert_close("xc", xc, inter["xc"], io)
    dbc = view(lay.dbc, lay.dbc_splits * T * W, torch.float32).view(lay.dbc_splits, cfg.batch, cfg.seqlen, W).sum(0)
    assert_close("dbc", dbc, inter["dbc"], io)
    bc = view(lay.bc, T * 32, torch.float32).view(cfg.batch, cfg.seqlen, 32)
    assert_close("Bn", bc[..., :16], inter["Bn"], io)
    assert_close("Cn", bc[..., 16:], inter["Cn"], io)
    dln = view(lay.dln, T * R, dt).view(cfg.batch, cfg.seqlen, R)
    assert_close("dln", dln, inter["dln"], io)
    delta = view(lay.delta, T * C, dt).view(cfg.batch, cfg.seqlen, C)
    assert_close("delta", delta, inter["delta"], io)
    del esz


@pytest.mark.parametrize("split", [1, 2, 300])
def test_split_prefill_matches_whole(split):
    cfg = _small("split", 2, 700, 128, 16, "bf16", 16)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    m = _mixer(cfg, w)
    x1, z1 = a["x"][:, :split].contiguous(), a["z"][:, :split].contiguous()
    x2, z2 = a["x"][:, split:].contiguous(), a["z"][:, split:].contiguous()
    o1, c1, h1 = m.prefill(x1, z1, st["conv_state"], st["ssm_state"])
    o2, c2, h2 = m.prefill(x2, z2, c1, h1)
    torch.cuda.synchronize()
    ro, rc, rh = oracle_prefill(cfg, weights_f64(w), a["x"], a["z"], st["conv_state"], to_f64(st["ssm_state"]))
    assert_close("out", torch.cat([o1, o2], dim=1), ro, "bf16")
    assert_close("h_final", h2, rh, "bf16")
    assert_bitwise("conv_state", c2, torch.from_numpy(rc).to(cfg.torch_dtype))


@pytest.mark.parametrize("L", [2, 700])
def test_states_updated_in_place(L):
    cfg = _small("inplace", 2, L, 128, 16, "bf16", 17)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    ro, rc, rh = oracle_prefill(cfg, weights_f64(w), a["x"], a["z"], st["conv_state"], to_f64(st["ssm_state"]))
    m = _mixer(cfg, w)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    out, cs2, hs2 = m.prefill(a["x"], a["z"], cs, hs, conv_state_out=cs, ssm_state_out=hs)
    torch.cuda.synchronize()
    assert cs2.data_ptr() == cs.data_ptr() and hs2.data_ptr() == hs.data_ptr()
    assert_close("out", out, ro, "bf16")
    assert_close("h_final", hs, rh, "bf16")
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_steps_small(io):
    cfg = _small(f"decode_{io}", 3, 1, 128, 16, io, 18, decode_steps=6, with_state=True)
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
    ro, rc, rh = oracle_prefill(cfg, weights_f64(w), tok["x"], tok["z"], st["conv_state"], to_f64(st["ssm_state"]))
    assert_close("decode out", torch.stack(outs, dim=1), ro, io)
    assert_close("h_final", hs, rh, io)
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


def test_deterministic_and_every_output_written():
    cfg = _small("determinism", 2, 700, 256, 64, "bf16", 19)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    m = _mixer(cfg, w)
    nan = torch.full((2, 700, 256), float("nan"), dtype=cfg.torch_dtype, device=DEV)
    o1, c1, h1 = m.prefill(a["x"], a["z"], out=nan.clone(),
                           conv_state_out=torch.full((2, 256, 3), float("nan"), dtype=cfg.torch_dtype, device=DEV),
                           ssm_state_out=torch.full((2, 256, 16), float("nan"), device=DEV))
    m._ws.fill_(0xFF)   # poison the workspace between the runs: nothing may depend on its old contents
    o2, c2, h2 = m.prefill(a["x"], a["z"])
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(h1).all() and torch.isfinite(c1.float()).all()
    assert torch.equal(o1, o2) and torch.equal(h1, h2) and torch.equal(c1, c2)


# ----------------------------------------------------------------------------- the five workloads

def test_workload_prefill_4k_full():
    cfg = CONFIGS[1]
    _run_and_check(cfg, with_state=False)


def test_workload_batched_prefill_sampled_channels():
    cfg = CONFIGS[2]
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    log(f"[{cfg.name}] B={cfg.batch} L={cfg.seqlen} C={cfg.d_inner}")
    m = _mixer(cfg, w)
    out, cs, hs = m.prefill(a["x"], a["z"])
    torch.cuda.synchronize()
    sel = np.arange(3, cfg.d_inner, 61)          # 135 channels spread over all 64-channel groups
    ro, rc, rh = oracle_prefill(cfg, weights_f64(w), a["x"], a["z"], channels=sel)
    assert_close("out[sampled]", out[..., torch.as_tensor(sel, device=DEV)], ro, "bf16")
    assert_close("h_final[sampled]", hs[:, torch.as_tensor(sel, device=DEV)], rh, "bf16")
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


def test_workload_long_context_256k_sampled_channels():
    cfg = CONFIGS[3]
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    log(f"[{cfg.name}] B={cfg.batch} L={cfg.seqlen} C={cfg.d_inner}")
    m = _mixer(cfg, w)
    out, cs, hs = m.prefill(a["x"], a["z"])
    torch.cuda.synchronize()
    sel = np.array([0, 77, 1000, 2049, 4095, 5120, 6143, 8191])
    sel_t = torch.as_tensor(sel, device=DEV)
    log("  oracle on sampled channels ...")
    ro, rh, rc = oracle_long_sampled(cfg, weights_f64(w), a["x"], a["z"], sel)
    assert_close("out[sampled]", out.index_select(2, sel_t), ro, "bf16")
    assert_close("h_final[sampled]", hs.index_select(1, sel_t), rh, "bf16")
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


def test_workload_decode_128_steps():
    cfg = CONFIGS[4]
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    tok = make_decode_tokens(cfg, DEV)
    log(f"[{cfg.name}] B={cfg.batch} steps={cfg.decode_steps} C={cfg.d_inner}")
    m = _mixer(cfg, w)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    outs = torch.empty((cfg.batch, cfg.decode_steps, cfg.d_inner), dtype=cfg.torch_dtype, device=DEV)
    for t in range(cfg.decode_steps):
        o, _, _ = m.decode_step(tok["x"][:, t], tok["z"][:, t], cs, hs, in_place=True)
        outs[:, t] = o
    # the same 128 tokens as one prefill from the same states
    po, pc, ph = m.prefill(tok["x"], tok["z"], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    sel = np.arange(5, cfg.d_inner, 67)
    sel_t = torch.as_tensor(sel, device=DEV)
    ro, rc, rh = oracle_prefill(cfg, weights_f64(w), tok["x"], tok["z"], st["conv_state"],
                                to_f64(st["ssm_state"])[:, sel], channels=sel)
    assert_close("decode out[sampled]", outs.index_select(2, sel_t), ro, "bf16")
    assert_close("decode h_final[sampled]", hs.index_select(1, sel_t), rh, "bf16")
    assert_bitwise("decode conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))
    assert_close("prefill out[sampled]", po.index_select(2, sel_t), ro, "bf16")
    # GPU decode against GPU prefill over every channel
    assert_close("decode vs prefill out", outs, po.double().cpu().numpy(), "bf16")
    assert_close("decode vs prefill h", hs, ph.double().cpu().numpy(), "bf16")
    assert_bitwise("decode vs prefill conv", cs, pc)
